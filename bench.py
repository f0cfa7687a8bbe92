"""Benchmark of the MLA paged-decode hot path on one MI355X.

A step is one pass of the whole path over one synthetic decode batch:
mla_absorb_q (q~ = W_UK^T q^C, RoPE of q^R) -> mla_decode_paged (split-KV
attention over the paged latent cache) -> mla_combine (split merge and
o = W_UV o~).  Inputs are resident in HBM before timing starts.  The cache is
replicated so consecutive steps read different copies and the 256 MB
Infinity Cache cannot serve one step's cache from the previous step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

Prints one JSON line (rank 0).  `value` is the step's algorithmic HBM bytes
per second; the line also carries TFLOP/s, query tokens per second, the
roofline of the dominant kernel (mla_decode_paged, timed with HIP events on
its stream) and the CPU oracle timed on a bounded sample of the same workload.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode latent-KV HBM GB/s + MFMA TFLOP/s vs roofline, B=64 L=4096"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
MALL_BYTES = 256 * 2 ** 20


def _elt(dt):
    return {"f32": 4, "bf16": 2, "e4m3": 1}[dt]


def algorithmic(spec, seqlens):
    """Algorithmic bytes and flops of each call of one step (no overheads)."""
    B, S, H = spec.batch, spec.q_len, spec.n_heads
    a = _elt(spec.act_dtype)
    lat = _elt(spec.latent_dtype)
    rows = B * S * H
    tokens = int(np.sum(seqlens.astype(np.int64)))
    per_tok = lat * spec.d_c + a * spec.d_rope + (4 if spec.latent_dtype == "e4m3" else 0)
    # keys visible to each query row
    L = seqlens.astype(np.int64)
    vis = 0
    for j in range(S):
        vis += int(np.sum(np.maximum(L - S + j + 1, 0) if spec.causal else L))
    q_lat_bytes = rows * (lat * spec.d_c + (4 if spec.latent_dtype == "e4m3" else 0))
    q_pe_bytes = rows * a * spec.d_rope
    absorb_b = rows * a * (spec.d_nope + spec.d_rope) + H * spec.d_nope * spec.d_c * a \
        + q_lat_bytes + q_pe_bytes
    absorb_f = 2 * rows * spec.d_nope * spec.d_c
    decode_b = tokens * per_tok + q_lat_bytes + q_pe_bytes + seqlens.size * 4 \
        + int(sum(math.ceil(x / spec.page_size) for x in seqlens)) * 4
    decode_f = 2 * H * vis * (spec.d_c + spec.d_rope) + 2 * H * vis * spec.d_c
    combine_b = H * spec.d_v * spec.d_c * a + rows * a * spec.d_v + rows * 4
    combine_f = 2 * rows * spec.d_c * spec.d_v
    return {"absorb": (absorb_b, absorb_f), "decode": (decode_b, decode_f),
            "combine": (combine_b, combine_f), "tokens": tokens, "rows": rows}


def cpu_baseline(wl, budget_s):
    """The oracle, as it stands, on a bounded sample of rows of the same workload."""
    import oracle
    from threadpoolctl import threadpool_info
    spec = wl.spec
    inp = oracle.inputs_from_workload(wl)
    rng = np.random.default_rng(7)
    done, t_used, rows_done = 0, 0.0, 0
    # rows of one (b, h) share the expansion of K and V, as in the oracle's own loop
    order = rng.permutation(spec.batch * spec.n_heads)
    t0 = time.perf_counter()
    for idx in order:
        b, h = divmod(int(idx), spec.n_heads)
        rows = np.array([[b, j, h] for j in range(spec.q_len)])
        oracle.mla_decode_expanded(inp, rows=rows)
        rows_done += len(rows)
        done += 1
        t_used = time.perf_counter() - t0
        if t_used >= budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    frac = rows_done / (spec.batch * spec.q_len * spec.n_heads)
    return t_used, frac, rows_done, threads


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has "
              "no multi-GPU path.  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from head_latent_attention_03_amd import inputs
    from head_latent_attention_03_amd.runner import DeviceBatch

    torch.cuda.set_device(0)
    spec = inputs.workload(args.config)
    wl = inputs.make_workload(spec)
    db = DeviceBatch.from_workload(wl, "cuda:0")
    cache_bytes = db.kv_latent.numel() * db.kv_latent.element_size() \
        + db.kv_rope.numel() * db.kv_rope.element_size() \
        + (db.kv_scale.numel() * 4 if db.kv_scale is not None else 0)
    n_rep = max(2, math.ceil(2 * MALL_BYTES / cache_bytes))
    reps = [(db.kv_latent, db.kv_scale, db.kv_rope)]
    for _ in range(n_rep - 1):
        reps.append((db.kv_latent.clone(), None if db.kv_scale is None else db.kv_scale.clone(),
                     db.kv_rope.clone()))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    def step(i, timed):
        lat, sc, rope = reps[i % n_rep]
        db.absorb()
        if timed:
            ev[i][0].record(stream)
        db.decode(kv_latent=lat, kv_scale=sc, kv_rope=rope)
        if timed:
            ev[i][1].record(stream)
        db.combine(with_uv=True)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    dec_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))

    alg = algorithmic(spec, wl.seqlens)
    step_bytes = sum(v[0] for k, v in alg.items() if k in ("absorb", "decode", "combine"))
    step_flops = sum(v[1] for k, v in alg.items() if k in ("absorb", "decode", "combine"))
    dec_b, dec_f = alg["decode"]
    kind = "f32" if spec.act_dtype == "f32" else ("fp8" if spec.latent_dtype == "e4m3" else "bf16")
    ridge = MFMA_PEAK_TFLOPS[kind] * 1e12 / (HBM_PEAK_GBS * 1e9)
    bound = "hbm" if dec_f / dec_b < ridge else "mfma"
    if bound == "hbm":
        achieved, peak, unit = dec_b / (dec_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = dec_f / (dec_ms * 1e-3) / 1e12, MFMA_PEAK_TFLOPS[kind], "TFLOP/s"

    out = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if kind == "bf16" else ("bf16+e4m3-cache" if kind == "fp8" else "f32"),
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.batch, "q_len": spec.q_len,
                   "seq_len": int(wl.max_seqlen) if len(set(wl.seqlens.tolist())) == 1 else "varied",
                   "tokens_in_cache": alg["tokens"], "heads": spec.n_heads,
                   "d_latent": spec.d_c, "d_rope": spec.d_rope, "page_size": spec.page_size,
                   "cache_replicas": n_rep},
        "tflops": round(step_flops / (ms_step * 1e-3) / 1e12, 2),
        "tokens_per_s": round(spec.batch * spec.q_len / (ms_step * 1e-3), 1),
        "step_bytes": int(step_bytes),
        "step_flops": int(step_flops),
        "roofline": {
            "kernel": "mla_decode_paged",
            "bound": bound,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": None,
            "launch_ms": round(dec_ms, 5),
            "algorithmic_bytes": int(dec_b),
            "algorithmic_flops": int(dec_f),
            "achieved_gbs": round(dec_b / (dec_ms * 1e-3) / 1e9, 2),
            "achieved_tflops": round(dec_f / (dec_ms * 1e-3) / 1e12, 2),
        },
    }
    if args.cpu_budget > 0:
        t_cpu, frac, rows_done, threads = cpu_baseline(wl, args.cpu_budget)
        full_s = t_cpu / frac
        out["cpu_baseline"] = {
            "value": round(step_bytes / full_s / 1e9, 6),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"{rows_done} of {spec.batch * spec.q_len * spec.n_heads} (b, j, h) rows "
                      f"of the same workload in {t_cpu:.1f} s, scaled to the whole step",
            "seconds_per_step": round(full_s, 2),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
