"""Host logic of bench.py (no GPU): the algorithmic bytes and flops behind
the roofline figures, the comment-insensitive source hash that keys the HBM
traffic summaries, the one-GPU guard, and the host copy of the decode's split
rule (which sizes the e4m3 second-pass estimate).

The expected byte and flop counts are written out from the shapes here, not
taken from bench.py: per cached token the cache holds the latent row and the
rotary row (plus an f32 scale for an e4m3 latent), and every visible (row,
key) pair costs 2 * (576 + 512) flops (score over the 576-dim absorbed query,
output over the 512-dim latent)."""

import os
import subprocess
import sys

import numpy as np

import bench
from head_latent_attention_03_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_bytes_and_flops_b64_l4096_bf16():
    spec = inputs.workload(2)
    seqlens = np.full(64, 4096, dtype=np.int32)
    dec_b, dec_f = bench.algorithmic(spec, seqlens)["decode"]
    cache = 64 * 4096 * (512 * 2 + 64 * 2)            # bf16 latent + bf16 rotary rows
    assert cache == 301_989_888
    query = 64 * 128 * (512 + 64) * 2                 # absorbed query and rotated q_pe
    meta = 64 * 4 + 64 * (4096 // 64) * 4             # seqlens + the pages' table entries
    assert dec_b == cache + query + meta == 311_443_712
    assert dec_f == 64 * 128 * 4096 * 2 * (576 + 512) == 73_014_444_032


def test_decode_bytes_e4m3_cache():
    spec = inputs.workload(4)
    seqlens = np.full(64, 4096, dtype=np.int32)
    dec_b, dec_f = bench.algorithmic(spec, seqlens)["decode"]
    per_token = 512 + 64 * 2 + 4                      # e4m3 latent, bf16 rotary, f32 scale
    assert per_token == 644
    query = 64 * 128 * (512 + 4 + 64 * 2)             # e4m3 query + its scale, bf16 q_pe
    meta = 64 * 4 + 64 * 64 * 4
    assert dec_b == 64 * 4096 * per_token + query + meta
    assert dec_f == 64 * 128 * 4096 * 2 * (576 + 512)


def test_causal_two_query_tokens_count_visible_keys():
    spec = inputs.workload(5, batch=2, seqlen=[10, 3])
    assert spec.q_len == 2 and spec.causal
    seqlens = np.array([10, 3], dtype=np.int32)
    dec_f = bench.algorithmic(spec, seqlens)["decode"][1]
    # query j of a sequence of L tokens sees L - 2 + j + 1 keys
    visible = (9 + 10) + (2 + 3)
    assert dec_f == spec.n_heads * visible * 2 * (576 + 512)


def test_source_hash_ignores_comments_only():
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    recommented = "// f: the successor\nint f(int x) {\n\n  return x + 1;\n}\n"
    changed = "int f(int x) {\n  return x + 2;  // one more\n}\n"
    assert bench._code_lines(code) == bench._code_lines(recommented)
    assert bench._code_lines(code) != bench._code_lines(changed)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _ceil(a, b):
    return -(-a // b)


def test_split_plan_rule():
    """bench.plan_split_counts, the host copy of the decode's split rule,
    checked against properties computed here by brute force: the chunk count
    stays within the budget (G when the proportional counts fit in G, else G
    plus the units); the chunk length is the shortest that does (every shorter
    length from 1 up overflows the budget); no chunk is longer than under the
    proportional counts; every nonempty sequence gets at least one chunk and
    an empty one none."""
    rng = np.random.default_rng(5)
    for trial in range(300):
        batch = int(rng.integers(1, 90))
        rg = int(rng.integers(1, 3))
        G = int(rng.choice([8, 64, 256]))
        tiles = [int(t) for t in rng.choice([0, 1, 3, 40, 128, int(rng.integers(0, 700))],
                                            size=batch)]
        nt = sum(tiles) * rg
        if nt == 0:
            continue
        s = bench.plan_split_counts(tiles, rg, G)
        prop = [min(t, max(1, G * t // nt)) if t > 0 else 0 for t in tiles]
        budget = G if sum(prop) * rg <= G else G + batch * rg
        assert sum(s) * rg <= budget
        longest = max(_ceil(t, q) for t, q in zip(tiles, s) if q > 0)
        assert all(q == _ceil(t, longest) for t, q in zip(tiles, s))
        for c in range(1, longest):
            assert sum(_ceil(t, c) for t in tiles) * rg > budget, (trial, c)
        assert longest <= max(_ceil(t, q) for t, q in zip(tiles, prop) if q > 0)
        assert all((q > 0) == (t > 0) for t, q in zip(tiles, s))


def test_split_plan_known_cases():
    """Uniform B=64 sequences of 128 tiles on 256 CUs: 4 chunks of 32 tiles each.
    256 units whose proportional counts overflow 256 (short units next to long
    ones) get the two-wave budget of 256 + 256 chunks."""
    assert bench.plan_split_counts([128] * 64, 1, 256) == [4] * 64
    tiles = [2] * 127 + [3000]
    s = bench.plan_split_counts(tiles, 2, 256)
    nt = sum(tiles) * 2
    prop = [min(t, max(1, 256 * t // nt)) for t in tiles]
    assert sum(prop) * 2 > 256
    assert 256 < sum(s) * 2 <= 512
    assert s[:127] == [1] * 127
