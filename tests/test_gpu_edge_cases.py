"""GPU parity on edge cases of the plan and of the e4m3 cache, and the
MLA_VALIDATE device check of the decode's preconditions."""

import numpy as np
import pytest
import torch

from head_latent_attention_03_amd import _binding as B
from head_latent_attention_03_amd import inputs
from head_latent_attention_03_amd.runner import DeviceBatch
from gpu_helpers import check_against_oracle, run_library, to_f64

pytestmark = pytest.mark.gpu


def _announce(name, wl):
    print(f"\n[case] {name} batch={wl.spec.batch} q_len={wl.spec.q_len} "
          f"lens={list(wl.seqlens[:8])}", flush=True)


@pytest.mark.parametrize("cfg", [2, 4])
def test_general_plan_with_two_row_groups(cfg):
    """70 sequences (past one lane per sequence: the plan's general path) with two
    query tokens x 128 heads (256 rows: two row groups per sequence, so units with
    rg = 1), short ragged lengths including empty sequences and ones shorter than
    the query run; every row, bf16 and e4m3 caches."""
    rng = np.random.default_rng(71)
    lens = [int(x) for x in rng.integers(0, 200, size=70)]
    lens[3], lens[40], lens[69] = 0, 1, 2
    wl = inputs.make_workload(inputs.workload(cfg, batch=70, q_len=2, seqlen=lens))
    _announce("two-row-groups", wl)
    got = run_library(wl)
    print(f"[errs] {check_against_oracle(wl, got)}", flush=True)


@pytest.mark.parametrize("cfg,q_len", [(2, 1), (2, 2), (4, 1)])
def test_long_chunks_every_row(cfg, q_len):
    """64 sequences of 1000-2100 tokens with 8 heads (one row group each, so the
    plan gives every unit 4 chunks of ~8-16 tiles): the loop's steady state runs
    for many tiles, including chunks that end in a partial tile and the causal
    tail of two query tokens; every row, bf16 and e4m3 caches."""
    rng = np.random.default_rng(64 + q_len)
    lens = [int(x) for x in rng.integers(1000, 2100, size=64)]
    lens[0], lens[1] = 2048, 1024
    wl = inputs.make_workload(inputs.workload(cfg, batch=64, q_len=q_len, n_heads=8,
                                              seqlen=lens, init="fan_in"))
    _announce("long-chunks", wl)
    got = run_library(wl)
    print(f"[errs] {check_against_oracle(wl, got, rows=_rows_bhj(wl.spec, range(64)))}",
          flush=True)


def test_fp8_all_zero_latent_rows():
    """e4m3 cache where a quarter of the tokens (and the first of each sequence, which
    sets the chunk's reference) are all-zero latent rows carrying scale 1, as the
    cache append writes them (a zero scale is outside the call's preconditions):
    they add nothing to the output but still take their share of the softmax, so
    dropping them from the sum would scale the output by ~4/3.  Every row."""
    wl = inputs.make_workload(inputs.workload(4, batch=3, seqlen=[100, 700, 33]))
    rng = np.random.default_rng(9)
    for b, L in enumerate(wl.seqlens):
        picks = list(rng.choice(int(L), size=max(1, int(L) // 4), replace=False)) + [0]
        for t in picks:
            p, s = wl.block_table[b, t // 64], t % 64
            wl.kv_latent[p, s] = 0
            wl.kv_scale[p, s] = 1.0
    _announce("fp8-all-zero-rows", wl)
    got = run_library(wl)
    print(f"[errs] {check_against_oracle(wl, got)}", flush=True)


def test_fp8_long_chunk_with_odd_first_tile():
    """e4m3 cache, 16 sequences of 8384 tokens (262 tiles of 32) with 8 query tokens
    x 128 heads: 128 units on 256 compute units give 2 chunks per unit, the second
    starting at tile 131 (odd) and 4192 tokens long, so the token-scale prefetch
    runs past the 64-page window it starts from.  Unused slots' scales hold 1e30,
    which would swamp the chunk's largest scale if any were read.  Every row of
    the first and the last sequence."""
    wl = inputs.make_workload(inputs.workload(4, batch=16, q_len=8, seqlen=8384))
    n_used = (8384 + 63) // 64
    used = set(int(x) for b in range(16) for x in wl.block_table[b, :n_used])
    spare = [p for p in range(wl.num_pages) if p not in used and p != wl.poison_page]
    # physical page 0 becomes unused (a lookup that falls back to 0 reads a poisoned
    # scale): its contents move to a spare page, and the table follows
    if 0 in used:
        q = spare.pop(0)
        for arr in (wl.kv_latent, wl.kv_scale, wl.kv_rope):
            arr[q] = arr[0]
        wl.block_table[wl.block_table == 0] = q
        used.discard(0)
    for p in range(wl.num_pages):
        if p not in used:
            wl.kv_scale[p] = np.float32(1e30)
    _announce("fp8-long-odd-chunk", wl)
    got = run_library(wl)
    for b in (0, 15):
        rows = np.array([[b, j, h] for h in range(128) for j in range(8)])
        print(f"[errs b={b}] {check_against_oracle(wl, got, rows=rows)}", flush=True)


def _rows_bhj(spec, seqs):
    """Every (j, h) row of the given sequences, (b, h, j) order (one expansion per head)."""
    return np.array([[b, j, h] for b in seqs for h in range(spec.n_heads)
                     for j in range(spec.q_len)])


@pytest.mark.parametrize("cfg", [2, 4])
def test_full_size_every_row(cfg):
    """The B=64, L=4096 workload at full size (bf16 and e4m3 caches), every one of
    its 8192 rows against the oracle."""
    spec = inputs.workload(cfg)
    wl = inputs.make_workload(spec)
    _announce(spec.name, wl)
    got = run_library(wl)
    errs = check_against_oracle(wl, got, rows=_rows_bhj(spec, range(spec.batch)))
    print(f"[errs] {errs}", flush=True)


@pytest.mark.parametrize("cfg", [3, 5])
def test_full_size_longest_sequence_every_row(cfg):
    """The long-context (B=16, 16k-64k) and two-token MTP (B=128) workloads at full
    size: every row of the longest sequence (the one split over the most chunks)
    and of the shortest, against the oracle."""
    spec = inputs.workload(cfg)
    wl = inputs.make_workload(spec)
    _announce(spec.name, wl)
    got = run_library(wl)
    seqs = [int(np.argmax(wl.seqlens)), int(np.argmin(wl.seqlens))]
    print(f"[seqs] {seqs} lens {[int(wl.seqlens[s]) for s in seqs]}", flush=True)
    errs = check_against_oracle(wl, got, rows=_rows_bhj(spec, seqs))
    print(f"[errs] {errs}", flush=True)
    assert np.all(np.isfinite(got["out"]))


def _decode_latent(db, kv_latent=None, kv_rope=None, block_table=None):
    db.decode(kv_latent=kv_latent, kv_rope=kv_rope, block_table=block_table)
    db.combine(with_uv=False)
    torch.cuda.synchronize()
    return to_f64(db.out_latent)


def test_validation_mode(monkeypatch):
    """MLA_VALIDATE=1: a decode over good tables gives the same bits as without the
    check; a used table entry outside [0, num_pages) or a length past max_seqlen is
    rejected with MLA_ERR_BAD_SHAPE and no decode runs.  (The broken entries still
    point inside the allocated buffers, so nothing could be read out of bounds.)"""
    wl = inputs.make_workload(inputs.workload(2, batch=2, seqlen=[100, 200]))
    db = DeviceBatch.from_workload(wl, "cuda:0")
    db.absorb()
    ref = _decode_latent(db)
    monkeypatch.setenv("MLA_VALIDATE", "1")
    assert np.array_equal(_decode_latent(db), ref)
    # the pool seen by the library is one page short; a used page names that page
    P = db.kv_latent.shape[0]
    lat_v, rope_v = db.kv_latent[:P - 1], db.kv_rope[:P - 1]
    bt = db.block_table.clone()
    bt[1, 2] = P - 1
    with pytest.raises(B.MlaError) as e:
        db.decode(kv_latent=lat_v, kv_rope=rope_v, block_table=bt)
    assert e.value.code == 2
    # a length past max_seqlen (still inside the table row: 4 pages of 64)
    sl = db.seqlens.clone()
    db.seqlens[0] = 201
    with pytest.raises(B.MlaError) as e:
        db.decode()
    assert e.value.code == 2
    db.seqlens.copy_(sl)
    monkeypatch.delenv("MLA_VALIDATE")
    assert np.array_equal(_decode_latent(db), ref)
