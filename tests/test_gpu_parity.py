"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Reduced shapes are compared on every row; the full-size workloads are compared
on sampled rows that the oracle computes one by one.
"""

import numpy as np
import pytest
import torch

from head_latent_attention_03_amd import inputs
from gpu_helpers import check_against_oracle, run_library, sample_rows

pytestmark = pytest.mark.gpu


def _run_check(spec, rows=None, seqlens=None, **kw):
    wl = inputs.make_workload(spec, seqlens=seqlens)
    print(f"\n[case] {spec.name} batch={spec.batch} q_len={spec.q_len} seqlens="
          f"{list(wl.seqlens[:8])}{'...' if spec.batch > 8 else ''}", flush=True)
    got = run_library(wl)
    errs = check_against_oracle(wl, got, rows=rows, **kw)
    print(f"[errs] {errs}", flush=True)
    return wl, got


def test_tiny_fp32_full():
    """The tiny fp32 workload, every row, max abs error 1e-4."""
    _run_check(inputs.workload(1))


@pytest.mark.parametrize("d_c", [48, 112])
def test_tiny_fp32_other_latent_widths(d_c):
    """fp32 path at latent widths that are multiples of 16 but not of 32 or 64
    (partial slices in the combine pass), two query tokens, ragged lengths."""
    _run_check(inputs.workload(1, d_c=d_c, batch=3, q_len=2, seqlen=[256, 70, 2]))


@pytest.mark.parametrize("case", range(8))
def test_random_small_fp32_shapes(case):
    """Seeded sweep of the fp32 path over the widths it accepts (latent a
    multiple of 16 up to 128, even rotary width up to 32, d_nope and d_v up
    to 128), 1-9 heads, 1-4 sequences of 0-300 tokens, 1-4 query tokens,
    shuffled or identity block tables; max abs error 1e-4 on every row."""
    rng = np.random.default_rng(2000 + case)
    batch = int(rng.integers(1, 5))
    spec = inputs.workload(
        1, batch=batch, q_len=int(rng.integers(1, 5)), n_heads=int(rng.integers(1, 10)),
        d_c=16 * int(rng.integers(1, 9)), d_rope=2 * int(rng.integers(1, 17)),
        d_nope=int(rng.choice([8, 16, 32, 64, 128])), d_v=int(rng.choice([8, 24, 32, 100, 128])),
        seqlen=[int(x) for x in rng.integers(0, 301, size=batch)],
        identity_table=bool(case % 2))
    _run_check(spec)


@pytest.mark.parametrize("seqlens", [[1], [65, 300, 31], [64, 128, 2, 5000]])
def test_bf16_reduced_ragged(seqlens):
    """DeepSeek-V3 shapes, short and ragged lengths (tails inside a page, one token)."""
    _run_check(inputs.workload(2, batch=len(seqlens), seqlen=seqlens))


def test_bf16_more_sequences_than_a_wave():
    """70 sequences (two lengths per lane in the split plan), ragged lengths
    including an empty one, bf16 and fp8 caches."""
    lens = [int(x) for x in np.random.default_rng(70).integers(0, 160, size=70)]
    lens[5] = 0
    _run_check(inputs.workload(2, batch=70, seqlen=lens))
    _run_check(inputs.workload(4, batch=70, seqlen=lens))


SPLIT_CASES = {"130_bf16": 130, "300_e4m3": 300, "100_mtp2_one_long": 100,
               "140_q2_e4m3": 140, "270_q2_bf16": 270}


@pytest.mark.parametrize("case", list(SPLIT_CASES))
def test_split_plan_large_batches(case):
    """The split plan at the batch sizes where it changes form: 130 sequences
    (four lengths per lane), 300 (the plan walks the lengths in memory, e4m3
    cache), and 100 sequences of two query tokens (200 units) with one 6000-token
    sequence among short ones, where the proportional chunk counts pass the
    workgroup target and the chunk budget grows to workgroups + units; then the
    four-per-lane and in-memory forms again with two query tokens (two row
    groups per sequence: 140 sequences on an e4m3 cache, 270 on bf16), where a
    unit's chunk number splits into row group and chunk.  Sampled rows plus 16
    heads of each query token of one sequence."""
    rng = np.random.default_rng(SPLIT_CASES[case])
    if case == "130_bf16":
        spec = inputs.workload(2, batch=130,
                               seqlen=[int(x) for x in rng.integers(0, 400, size=130)])
    elif case == "300_e4m3":
        lens = [int(x) for x in rng.integers(0, 200, size=300)]
        lens[299] = 0
        spec = inputs.workload(4, batch=300, seqlen=lens)
    elif case == "140_q2_e4m3":
        lens = [int(x) for x in rng.integers(0, 300, size=140)]
        lens[3], lens[37] = 1, 2000
        spec = inputs.workload(4, batch=140, q_len=2, seqlen=lens)
    elif case == "270_q2_bf16":
        lens = [int(x) for x in rng.integers(0, 150, size=270)]
        lens[0], lens[37] = 0, 1500
        spec = inputs.workload(5, batch=270, seqlen=lens, init="fan_in")
    else:
        lens = [int(x) for x in rng.integers(1, 100, size=100)]
        lens[37] = 6000
        spec = inputs.workload(5, batch=100, seqlen=lens, init="fan_in")
    wl = inputs.make_workload(spec)
    rows = sample_rows(wl, 40, seed=5)
    if spec.q_len == 2:
        heads = np.arange(0, spec.n_heads, spec.n_heads // 16)
        long_rows = np.stack([np.full(32, 37), np.repeat([0, 1], 16), np.tile(heads, 2)], axis=1)
        rows = np.concatenate([rows, long_rows])
        rows = rows[np.lexsort((rows[:, 2], rows[:, 1], rows[:, 0]))]
    _run_check(spec, rows=rows)


@pytest.mark.parametrize("n_heads,q_len,seqlens", [(16, 1, [5, 300, 64]),
                                                   (200, 3, [3, 300, 1000]),
                                                   (128, 8, [8, 97])])
def test_bf16_other_head_counts_and_query_lengths(n_heads, q_len, seqlens):
    """Head counts that leave a partial 128-row group (16 heads: one group with
    16 valid rows; 200 heads x 3 query tokens: 600 rows in 5 groups, the last
    with 88) and the longest supported query run (8 tokens), causal, with a
    sequence exactly as long as its query run (its first query sees one key)."""
    _run_check(inputs.workload(2, batch=len(seqlens), n_heads=n_heads, q_len=q_len,
                               seqlen=seqlens))


def test_fp8_cache_other_head_count():
    """e4m3 cache with 40 heads and 4 query tokens (160 rows: a full group and a
    partial one), causal."""
    _run_check(inputs.workload(4, batch=3, n_heads=40, q_len=4, seqlen=[4, 129, 700]))


@pytest.mark.parametrize("case", range(12))
def test_random_small_shapes(case):
    """Seeded sweep of small shapes through the whole path, every row against
    the oracle: bf16 or e4m3 cache, 1-6 sequences of 0-700 tokens (empty ones
    and ones shorter than their query run included), 1-4 query tokens
    (causal), 8-136 heads."""
    rng = np.random.default_rng(1000 + case)
    cfg = 2 if case % 2 == 0 else 4
    batch = int(rng.integers(1, 7))
    q_len = int(rng.integers(1, 5))
    n_heads = int(rng.choice([8, 16, 40, 64, 128, 136]))
    lens = [int(x) for x in rng.integers(0, 701, size=batch)]
    if case % 3 == 0:
        lens[0] = int(rng.integers(0, q_len + 1))
    _run_check(inputs.workload(cfg, batch=batch, q_len=q_len, n_heads=n_heads, seqlen=lens))


def test_bf16_reduced_sharp_softmax():
    """Same shapes with N(0,1)/sqrt(dim) inputs: scores spread out, the softmax is peaked."""
    _run_check(inputs.workload(2, batch=3, seqlen=[700, 4096, 33], init="fan_in"))


@pytest.mark.parametrize("seqlens", [[2, 3, 64, 129, 500], [1, 65]])
def test_mtp_two_query_tokens_causal(seqlens):
    """Two query tokens per sequence with the causal rule between them."""
    _run_check(inputs.workload(5, batch=len(seqlens), seqlen=seqlens, init="fan_in"))


def test_long_context_reduced():
    """Long sequences split over many chunks (merged by the combine pass)."""
    _run_check(inputs.workload(3, batch=2, seqlen=[20000, 9000]))


@pytest.mark.parametrize("seqlens", [[1], [65, 300, 31], [64, 128, 2, 5000]])
def test_fp8_cache_reduced_ragged(seqlens):
    """e4m3 latent with per-token scales, short and ragged lengths, 6e-2 against the
    dequantised cache."""
    _run_check(inputs.workload(4, batch=len(seqlens), seqlen=seqlens))


def test_fp8_cache_peaked_softmax():
    """e4m3 latent with N(0,1)/sqrt(dim) inputs: peaked rows whose maximum grows
    from tile to tile, against the exact oracle at the fp8 tolerance (6e-2)."""
    _run_check(inputs.workload(4, batch=3, seqlen=[700, 4096, 33], init="fan_in"))


def _sharp_fp8(scale):
    return inputs.workload(4, batch=3, seqlen=[700, 4096, 33], init="fan_in",
                           softmax_scale=scale)


@pytest.mark.xfail(strict=True, raises=AssertionError,
                   reason="known accuracy limit of the e4m3-cache path: with a softmax scale "
                          "of 2 or more on N(0,1)/sqrt(dim) inputs, the per-row e4m3 rounding "
                          "of the absorbed query (3 mantissa bits) moves the scores past the "
                          "6e-2 fp8 tolerance of the exact oracle (log-sum-exp 0.11 off at "
                          "scale 2, outputs ~23% off at scale 8)")
@pytest.mark.parametrize("softmax_scale", [2.0, 8.0])
def test_fp8_cache_sharp_softmax_query_rounding_limit(softmax_scale):
    """Against the exact oracle at 6e-2: expected to fail (strict), so a change in
    the fp8 path's accuracy shows up here."""
    _run_check(_sharp_fp8(softmax_scale))


@pytest.mark.parametrize("softmax_scale", [2.0, 8.0])
def test_fp8_cache_sharp_softmax_kernel_only(softmax_scale):
    """The kernel's own error at sharp softmaxes, separated from the query rounding
    by the kernel model of tests/kernel_models.py (the oracle's absorbed form fed
    the same per-row e4m3 query).  A kernel-only check, not a parity test; the
    exact-oracle error is printed."""
    from gpu_helpers import check_e4m3_kernel_model, relative_errors
    wl = inputs.make_workload(_sharp_fp8(softmax_scale))
    got = run_library(wl)
    print(f"\n[exact-oracle error, reported] {relative_errors(wl, got)}", flush=True)
    print(f"[kernel-only errs] {check_e4m3_kernel_model(wl, got)}", flush=True)


def test_fp8_cache_two_query_tokens():
    """e4m3 latent, two causal query tokens per sequence."""
    _run_check(inputs.workload(4, batch=4, q_len=2, seqlen=[2, 65, 300, 1000], init="fan_in"))


def test_full_size_fp8_sampled():
    """The B=64, L=4096 e4m3-cache workload at full size, sampled rows."""
    spec = inputs.workload(4)
    wl = inputs.make_workload(spec)
    got = run_library(wl)
    check_against_oracle(wl, got, rows=sample_rows(wl, 12, seed=4))
    assert np.all(np.isfinite(got["out"])) and np.all(np.isfinite(got["out_latent"]))


def test_full_size_b64_l4096_sampled():
    """The B=64, L=4096 bf16 workload at full size, sampled rows."""
    spec = inputs.workload(2)
    wl = inputs.make_workload(spec)
    got = run_library(wl)
    check_against_oracle(wl, got, rows=sample_rows(wl, 12, seed=1))
    assert np.all(np.isfinite(got["out"])) and np.all(np.isfinite(got["out_latent"]))


def test_full_size_mtp_sampled():
    spec = inputs.workload(5)
    wl = inputs.make_workload(spec)
    got = run_library(wl)
    check_against_oracle(wl, got, rows=sample_rows(wl, 12, seed=2))
    assert np.all(np.isfinite(got["out"]))


def test_full_size_long_context_sampled():
    spec = inputs.workload(3)
    wl = inputs.make_workload(spec)
    got = run_library(wl)
    check_against_oracle(wl, got, rows=sample_rows(wl, 6, seed=3))
    assert np.all(np.isfinite(got["out"]))
