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
import csv
import glob
import hashlib
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
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "head_latent_attention_03_amd", "csrc")
# sources that define the decode kernel; the traffic summary is valid only for them
DECODE_SOURCES = {"bf16": ("decode_bf16.hip", "mla_common.hpp", "mla_internal.hpp"),
                  "f32": ("decode_f32.hip", "mla_common.hpp", "mla_internal.hpp"),
                  "fp8": ("decode_fp8.hip", "mla_common.hpp", "mla_internal.hpp")}
DECODE_KERNEL_NAME = {"bf16": "decode_bf16_kernel", "f32": "decode_f32_kernel",
                      "fp8": "decode_fp8_kernel"}


def _code_lines(text):
    """The source without // comments, trailing blanks and blank lines (a
    comment edit does not change the kernel; the sources hold no block
    comments and no // inside a string)."""
    out = []
    for line in text.splitlines():
        i = line.find("//")
        if i >= 0:
            line = line[:i]
        line = line.rstrip()
        if line:
            out.append(line)
    return "\n".join(out)


def source_hash(kind):
    """Hash of the code (comments stripped) of the sources a decode kernel is
    built from."""
    h = hashlib.sha256()
    for f in DECODE_SOURCES[kind]:
        with open(os.path.join(CSRC, f)) as fh:
            h.update(_code_lines(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_file(kind, workload):
    return os.path.join(PROFILES, f"{DECODE_KERNEL_NAME[kind]}_{workload}_hbm_traffic.txt")


def read_traffic(kind, workload):
    """HBM bytes per decode launch from the committed counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    path = traffic_file(kind, workload)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_hash(kind):
        return None
    return int(vals["hbm_bytes_per_launch"])


def _pmc_rows(path, counter):
    rows = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            rows.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), 0.0)
            rows[(r["Kernel_Name"], r["Dispatch_Id"])] += float(r["Counter_Value"])
    return rows


def summarize_pmc(fetch_dir, write_dir, kind, workload, copy_mib, commands):
    """Write the traffic summary from a FETCH_SIZE run and a WRITE_SIZE run.

    Both counters are KiB per dispatch.  Each is scaled by what it reads for
    the plain device copy of copy_mib MiB in the same run (reads copy_mib MiB,
    writes copy_mib MiB), so that the summary is in bytes of the copy's own
    ruler."""
    def load(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit(f"no counter_collection.csv under {d}")
        return _pmc_rows(f[0], counter)
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = load(d, counter)
        dec = {int(i): v for (k, i), v in rows.items() if DECODE_KERNEL_NAME[kind] in k}
        # the calibration copy is the last device copy before the first decode
        # (earlier copies are the cache replicas)
        cpy = {int(i): v for (k, i), v in rows.items()
               if "copyBuffer" in k and dec and int(i) < min(dec)}
        if not dec or not cpy:
            raise SystemExit(f"{counter}: decode or copy dispatches missing in {d}")
        cpy_kib = cpy[max(cpy)]
        dec = list(dec.values())
        factor = copy_mib * 1024.0 / cpy_kib
        out[counter] = (float(np.mean(dec)), cpy_kib, factor)
    fetch_b = out["FETCH_SIZE"][0] * out["FETCH_SIZE"][2] * 1024
    write_b = out["WRITE_SIZE"][0] * out["WRITE_SIZE"][2] * 1024
    path = traffic_file(kind, workload)
    with open(path, "w") as fh:
        fh.write(f"# HBM traffic of {DECODE_KERNEL_NAME[kind]} on workload {workload}\n")
        fh.write("# from two rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE), KiB per dispatch,\n")
        fh.write(f"# each scaled by the same counter on a plain {copy_mib} MiB device copy in the run\n")
        for c in commands:
            fh.write(f"# command: {c}\n")
        for counter, (dec, cpy, factor) in out.items():
            fh.write(f"{counter.lower()}_decode_kib_avg: {dec:.1f}\n")
            fh.write(f"{counter.lower()}_copy_kib: {cpy:.1f}\n")
            fh.write(f"{counter.lower()}_scale: {factor:.4f}\n")
        fh.write(f"hbm_read_bytes_per_launch: {int(fetch_b)}\n")
        fh.write(f"hbm_write_bytes_per_launch: {int(write_b)}\n")
        fh.write(f"hbm_bytes_per_launch: {int(fetch_b + write_b)}\n")
        fh.write(f"source_sha256_16: {source_hash(kind)}\n")
    print(open(path).read())


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
    # append: read the new tokens' latent and rotary rows and the gain, write
    # their cache rows (latent, rotary, e4m3 scale)
    append_b = B * S * (a * (spec.d_c + spec.d_rope) + per_tok) + a * spec.d_c \
        + seqlens.size * 4 + B * S * 4
    return {"append": append_b, "absorb": (absorb_b, absorb_f), "decode": (decode_b, decode_f),
            "combine": (combine_b, combine_f), "tokens": tokens, "rows": rows}


def append_time(spec, db, stream, steps):
    """Average duration (us, HIP events) of mla_append_kv writing one new token
    per query position of every sequence (the tokens at the end of the cache)."""
    import torch
    from head_latent_attention_03_amd import _binding as B
    S, dev = spec.q_len, db.kv_latent.device
    act = db.dims.act_torch
    g = torch.Generator(device="cpu").manual_seed(31)
    kv_c = torch.randn((spec.batch, S, spec.d_c), generator=g).to(act).to(dev)
    k_r = torch.randn((spec.batch, S, spec.d_rope), generator=g).to(act).to(dev)
    w = (1 + 0.1 * torch.randn((spec.d_c,), generator=g)).to(act).to(dev)
    call = lambda: B.mla_append_kv(db.dims, kv_c, k_r, w, 1e-6, db.seqlens, db.block_table,
                                   db.kv_latent, db.kv_scale, db.kv_rope, stream=stream)
    for _ in range(5):
        call()
    n = max(10, min(steps, 100))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3


def e4m3_cache_decode(cfg, launches):
    """The decode alone over an e4m3 latent cache of the same B=64, L=4096 shape:
    average launch duration (HIP events on the launch stream) and its roofline
    figures.  The cache is replicated past the last-level cache, as in the main
    loop, so every launch reads HBM."""
    import torch
    from head_latent_attention_03_amd import inputs
    from head_latent_attention_03_amd.runner import DeviceBatch
    spec = inputs.workload(cfg)
    wl = inputs.make_workload(spec)
    db = DeviceBatch.from_workload(wl, "cuda:0")
    cache_bytes = db.kv_latent.numel() * db.kv_latent.element_size() \
        + db.kv_rope.numel() * db.kv_rope.element_size() + db.kv_scale.numel() * 4
    n_rep = max(2, math.ceil(2 * MALL_BYTES / cache_bytes))
    reps = [(db.kv_latent, db.kv_scale, db.kv_rope)]
    for _ in range(n_rep - 1):
        reps.append((db.kv_latent.clone(), db.kv_scale.clone(), db.kv_rope.clone()))
    stream = torch.cuda.current_stream()
    db.absorb()
    for i in range(10):
        lat, sc, rope = reps[i % n_rep]
        db.decode(kv_latent=lat, kv_scale=sc, kv_rope=rope)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(launches)]
    for i, (a, b) in enumerate(ev):
        lat, sc, rope = reps[i % n_rep]
        a.record(stream)
        db.decode(kv_latent=lat, kv_scale=sc, kv_rope=rope)
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    dec_b, dec_f = algorithmic(spec, wl.seqlens)["decode"]
    gbs = dec_b / (ms * 1e-3) / 1e9
    tfs = dec_f / (ms * 1e-3) / 1e12
    traffic = read_traffic("fp8", spec.name)
    del reps, db
    torch.cuda.empty_cache()
    return {
        "kernel": "mla_decode_paged", "workload": spec.name, "bound": "hbm",
        "launch_ms": round(ms, 5), "timed_launches": launches, "cache_replicas": n_rep,
        "algorithmic_bytes": int(dec_b), "algorithmic_flops": int(dec_f),
        "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(gbs / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "achieved_tflops": round(tfs, 2), "mfma_peak_tflops": MFMA_PEAK_TFLOPS["fp8"],
        "mfma_frac": round(tfs / MFMA_PEAK_TFLOPS["fp8"], 4),
    }


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
    ap.add_argument("--event-every", type=int, default=8,
                    help="bracket the decode launch of every N-th timed step with HIP events")
    ap.add_argument("--e4m3-launches", type=int, default=40,
                    help="time this many decode launches over an e4m3 cache of the same "
                         "shape after the main loop (0: skip)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0: skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size first (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the decode traffic summary from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--pmc-command", action="append", default=[],
                    help="command lines of the counter runs, recorded in the summary")
    args = ap.parse_args()
    if args.summarize_pmc:
        from head_latent_attention_03_amd import inputs
        spec = inputs.workload(args.config)
        kind = "f32" if spec.act_dtype == "f32" else ("fp8" if spec.latent_dtype == "e4m3" else "bf16")
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], kind, spec.name,
                      args.copy_calibration_mib, args.pmc_command)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); there is "
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

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * 2 ** 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_(0, 255)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()
    # the decode launches of every event_every-th timed step are bracketed by
    # HIP events (a timing event is not free: bracketing every launch adds
    # several microseconds per step to the whole-step time)
    ev_steps = [i for i in range(args.steps) if i % args.event_every == args.event_every - 1]
    if not ev_steps:
        ev_steps = [args.steps - 1]
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for i in ev_steps}

    def step(i, timed):
        lat, sc, rope = reps[i % n_rep]
        db.absorb()
        if timed and i in ev:
            ev[i][0].record(stream)
        db.decode(kv_latent=lat, kv_scale=sc, kv_rope=rope)
        if timed and i in ev:
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
    dec_ms = float(np.mean([a.elapsed_time(b) for a, b in ev.values()]))

    # the cache append of the step's new tokens (the step before decode, timed
    # on its own after the main loop: it is not part of the metric's step)
    app_us = append_time(spec, db, stream, args.steps)

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

    traffic = read_traffic(kind, spec.name)
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
            "traffic": traffic,
            "traffic_over_algorithmic": None if traffic is None else round(traffic / dec_b, 4),
            "launch_ms": round(dec_ms, 5),
            "timed_launches": len(ev),
            "algorithmic_bytes": int(dec_b),
            "algorithmic_flops": int(dec_f),
            "achieved_gbs": round(dec_b / (dec_ms * 1e-3) / 1e9, 2),
            "achieved_tflops": round(dec_f / (dec_ms * 1e-3) / 1e12, 2),
        },
    }
    app_b = alg["append"]
    out["append"] = {
        "kernel": "mla_append_kv", "us": round(app_us, 3), "tokens": spec.batch * spec.q_len,
        "algorithmic_bytes": int(app_b),
        "achieved_gbs": round(app_b / (app_us * 1e-6) / 1e9, 2),
        "note": "one wave per new token; at this size the launch latency is the bound, "
                "not HBM (the bytes would take well under 1 us at 8 TB/s)",
    }
    if args.e4m3_launches > 0 and args.config == 2:
        out["e4m3_cache"] = e4m3_cache_decode(4, args.e4m3_launches)
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
