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
N_CU = 256                # compute units of the MI355X
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
        if f:
            return _pmc_rows(f[0], counter)
        dbs = glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True)
        if not dbs:
            raise SystemExit(f"no counter_collection.csv or rocprofv3 database under {d}")
        import sqlite3
        rows = {}
        con = sqlite3.connect(dbs[0])
        for name, disp, val in con.execute(
                "select kernel_name, dispatch_id, value from counters_collection "
                "where counter_name = ?", (counter,)):
            rows[(name, str(disp))] = rows.get((name, str(disp)), 0.0) + float(val)
        con.close()
        return rows
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


def summarize_trace(db_glob, out_name, title, commands, window=None, bench_log=None):
    """Write a kernel-duration summary (profiles/<out_name>) from a rocprofv3
    --kernel-trace run: calls, mean, median, min and max per kernel.
    `window` = (kernel name substring, first, end): also the statistics of that
    kernel's calls first .. end - 1 in start order (e.g. the launches a bench
    object timed).  `bench_log`: the bench output of the same run, whose
    roofline timing is copied next to them."""
    import sqlite3
    paths = sorted(glob.glob(db_glob, recursive=True))
    if not paths:
        raise SystemExit(f"no rocprofv3 database matches {db_glob}")
    durs = {}
    ordered = []
    for path in paths:
        con = sqlite3.connect(path)
        for name, start, end in con.execute("select name, start, end from kernels"):
            durs.setdefault(name, []).append((end - start) / 1e3)
            ordered.append((start, name, (end - start) / 1e3))
        con.close()
    ordered.sort()
    out = os.path.join(PROFILES, out_name)
    total = sum(sum(v) for v in durs.values())
    with open(out, "w") as fh:
        fh.write(f"# kernel durations (us): {title}\n")
        for c in commands:
            fh.write(f"# command: {c}\n")
        fh.write(f"{'kernel':72s} {'calls':>5s} {'mean':>8s} {'median':>8s} {'min':>8s} "
                 f"{'max':>8s} {'share':>6s}\n")
        for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
            v = np.asarray(v)
            short = name.replace("mla::(anonymous namespace)::", "")
            fh.write(f"{short[:72]:72s} {len(v):5d} {v.mean():8.2f} {np.median(v):8.2f} "
                     f"{v.min():8.2f} {v.max():8.2f} {100 * v.sum() / total:5.1f}%\n")
        if window is not None:
            sub, first, end = window[0], int(window[1]), int(window[2])
            calls = [d for _, name, d in ordered if sub in name]
            # (negative indices count from the end; END 0 is the end)
            sel = calls[first:(end if end != 0 else None)]
            v = np.asarray(sel)
            if v.size == 0:
                raise SystemExit(f"no calls {first}..{end - 1} of a kernel matching {sub}")
            lo = first if first >= 0 else len(calls) + first
            fh.write(f"# calls {lo} .. {lo + v.size - 1} of the kernel matching '{sub}' "
                     f"(in start order, of {len(calls)}):\n")
            fh.write(f"{'  window':72s} {v.size:5d} {v.mean():8.2f} {np.median(v):8.2f} "
                     f"{v.min():8.2f} {v.max():8.2f}\n")
        if bench_log is not None:
            line = [ln for ln in open(bench_log).read().splitlines() if ln.startswith("{")][-1]
            roof = json.loads(line)["roofline"]
            fh.write(f"# the bench line of the same run: roofline launch_ms {roof['launch_ms']} "
                     f"(median {roof['launch_ms_median']}, p10 {roof['launch_ms_p10']}, "
                     f"p90 {roof['launch_ms_p90']}), frac {roof['frac']}\n")
    print(open(out).read())


def summarize_counters(db_glob, out_name, title, commands):
    """Write per-kernel averages of every counter in rocprofv3 --pmc databases
    (profiles/<out_name>), with the derived MFMA rate and busy fractions when
    the MFMA counters are present.  The MOPS counters count 512-flop units and
    GRBM_GUI_ACTIVE is summed over the 8 XCDs."""
    import sqlite3
    paths = sorted(glob.glob(db_glob, recursive=True))
    if not paths:
        raise SystemExit(f"no rocprofv3 database matches {db_glob}")
    per = {}
    for path in paths:
        con = sqlite3.connect(path)
        for name, disp, cname, val in con.execute(
                "select kernel_name, dispatch_id, counter_name, value from counters_collection"):
            d = per.setdefault(name, {}).setdefault(cname, {})
            d[disp] = d.get(disp, 0.0) + float(val)
        con.close()
    out = os.path.join(PROFILES, out_name)
    with open(out, "w") as fh:
        fh.write(f"# per-dispatch counter averages: {title}\n")
        for c in commands:
            fh.write(f"# command: {c}\n")
        fh.write("# derived: mfma_flops = (MOPS_BF16 + MOPS_F8 + MOPS_F6F4) * 512; "
                 "kernel_cycles = GRBM_GUI_ACTIVE / 8;\n"
                 "#          mfma_busy = VALU_MFMA_BUSY_CYCLES / (4 SIMDs x 256 CUs x kernel_cycles);  "
                 "lds_conflict = LDS_BANK_CONFLICT / LDS_IDX_ACTIVE\n")
        for name, cs in sorted(per.items()):
            short = name.replace("mla::(anonymous namespace)::", "")
            if "mla::" not in name:
                continue
            avg = {c: float(np.mean(list(v.values()))) for c, v in cs.items()}
            n = max(len(v) for v in cs.values())
            fh.write(f"\n{short}  ({n} dispatches)\n")
            for c in sorted(avg):
                fh.write(f"  {c:36s} {avg[c]:16.1f}\n")
            mops = sum(avg.get(f"SQ_INSTS_VALU_MFMA_MOPS_{t}", 0.0) for t in ("BF16", "F8", "F6F4"))
            if mops:
                fh.write(f"  {'mfma_flops':36s} {mops * 512:16.4g}\n")
            if "GRBM_GUI_ACTIVE" in avg:
                fh.write(f"  {'kernel_cycles':36s} {avg['GRBM_GUI_ACTIVE'] / 8:16.1f}\n")
            if avg.get("GRBM_GUI_ACTIVE") and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                # (the busy count is summed over the SIMDs, 4 per CU)
                simd_cycles = 4 * N_CU * avg["GRBM_GUI_ACTIVE"] / 8
                fh.write(f"  {'mfma_busy':36s} "
                         f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:16.4f}\n")
            if avg.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in avg:
                fh.write(f"  {'lds_conflict':36s} "
                         f"{avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_LDS_IDX_ACTIVE']:16.4f}\n")
    print(open(out).read())


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
    n = max(10, min(steps, 100))
    return float(np.mean(time_launches(lambda i: call(), n, warm=5))) * 1e3


def kind_of(spec):
    if spec.act_dtype == "f32":
        return "f32"
    return "fp8" if spec.latent_dtype == "e4m3" else "bf16"


def replicate_cache(db, read_bytes=None):
    """Copies of the cache so that consecutive launches read different copies and
    together exceed twice the 256 MB last-level cache (`read_bytes`: the bytes
    one launch reads, when it reads less than the whole cache)."""
    cache_bytes = db.kv_latent.numel() * db.kv_latent.element_size() \
        + db.kv_rope.numel() * db.kv_rope.element_size() \
        + (db.kv_scale.numel() * 4 if db.kv_scale is not None else 0)
    n_rep = max(2, math.ceil(2 * MALL_BYTES / (read_bytes or cache_bytes)))
    reps = [(db.kv_latent, db.kv_scale, db.kv_rope)]
    for _ in range(n_rep - 1):
        reps.append((db.kv_latent.clone(), None if db.kv_scale is None else db.kv_scale.clone(),
                     db.kv_rope.clone()))
    return reps


def calibration_copy(mib):
    """One plain device copy of `mib` MiB (the ruler of the HBM traffic counters)."""
    import torch
    n = mib * 2 ** 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_(0, 255)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


TIME_BATCH = 10   # launches between two timing events


def progress(msg):
    """A line on stderr as each part of the run ends (the JSON result alone goes
    to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# The GPU's clock comes up only after about half a second of continuous work
# (measured: B=64 L=4096 bf16 decode at 113.7 us per launch after 2 s idle,
# 77.7 us after 0.5 s of back-to-back decodes, 78.1 us after 3.5 s), so every
# timed loop first runs its work untimed for at least this long.
CLOCK_WARM_S = 0.5


_untimed = {"last": 0}   # untimed launches before the last time_launches batch


def warm_clock(call, seconds=CLOCK_WARM_S):
    """Run `call(i)` back to back, untimed, for at least `seconds` of wall time
    (synchronising every few calls); returns the number of calls."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(8):
            call(n)
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def time_launches(call, launches, warm=30, batch=TIME_BATCH):
    """Per-launch durations (ms) of back-to-back calls of `call(i)` (the i-th
    launch).  HIP events on the launch stream bracket each batch of `batch`
    consecutive launches, with no event between the launches inside a batch:
    a timing event between every two launches adds 4-7 us to each (measured:
    80.0 us per B=64 L=4096 bf16 decode back to back, 84-85 us with an event
    pair around each).  The batches follow one another without a host
    synchronisation, after at least `warm` launches and CLOCK_WARM_S seconds
    of untimed launches that bring the clock up.  Returns one mean per batch,
    ceil(launches / batch) batches."""
    import torch
    stream = torch.cuda.current_stream()
    _untimed["last"] = warm_clock(call) + warm
    for i in range(warm):
        call(i)
    nb = max(1, -(-launches // batch))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    ev[0].record(stream)
    k = 0
    for b in range(nb):
        for _ in range(batch):
            call(k)
            k += 1
        ev[b + 1].record(stream)
    torch.cuda.synchronize()
    return np.array([ev[b].elapsed_time(ev[b + 1]) / batch for b in range(nb)])


def time_decode(db, reps, launches, **view):
    """time_launches of the decode, rotating over the cache replicas (`view`:
    block_table, seqlens, max_seqlen of an eviction view)."""
    def call(i):
        lat, sc, rope = reps[i % len(reps)]
        db.decode(kv_latent=lat, kv_scale=sc, kv_rope=rope, **view)
    return time_launches(call, launches)


def decode_roofline(spec, seqlens, ms, traffic):
    """The roofline object of one decode launch shape from its durations (ms)."""
    kind = kind_of(spec)
    dec_b, dec_f = algorithmic(spec, seqlens)["decode"]
    ridge = MFMA_PEAK_TFLOPS[kind] * 1e12 / (HBM_PEAK_GBS * 1e9)
    bound = "hbm" if dec_f / dec_b < ridge else "mfma"
    mean = float(np.mean(ms))
    gbs = dec_b / (mean * 1e-3) / 1e9
    tfs = dec_f / (mean * 1e-3) / 1e12
    if bound == "hbm":
        achieved, peak, unit = gbs, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = tfs, MFMA_PEAK_TFLOPS[kind], "TFLOP/s"
    return {
        "kernel": "mla_decode_paged", "workload": spec.name, "bound": bound,
        "achieved": round(achieved, 2), "peak": peak, "unit": unit,
        "frac": round(achieved / peak, 4),
        "traffic": traffic,
        "traffic_over_algorithmic": None if traffic is None else round(traffic / dec_b, 4),
        "launch_ms": round(mean, 5),
        "launch_ms_median": round(float(np.median(ms)), 5),
        "launch_ms_p10": round(float(np.percentile(ms, 10)), 5),
        "launch_ms_p90": round(float(np.percentile(ms, 90)), 5),
        "timed_launches": int(len(ms)) * TIME_BATCH,
        "untimed_launches": _untimed["last"],
        "timing": f"HIP events around each batch of {TIME_BATCH} back-to-back launches; "
                  "launch_ms is the mean, median/p10/p90 are over the batch means",
        "algorithmic_bytes": int(dec_b), "algorithmic_flops": int(dec_f),
        "achieved_gbs": round(gbs, 2), "achieved_tflops": round(tfs, 2),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "mfma_frac": round(tfs / MFMA_PEAK_TFLOPS[kind], 4),
    }


def decode_object(cfg, launches, copy_mib=0):
    """The decode alone on workload `cfg`: `launches` timed launches (HIP events,
    cache replicated past the last-level cache) and their roofline figures."""
    import torch
    from head_latent_attention_03_amd import inputs
    from head_latent_attention_03_amd.runner import DeviceBatch
    spec = inputs.workload(cfg)
    wl = inputs.make_workload(spec)
    db = DeviceBatch.from_workload(wl, "cuda:0")
    reps = replicate_cache(db)
    if copy_mib > 0:
        calibration_copy(copy_mib)
    db.absorb()
    ms = time_decode(db, reps, launches)
    out = decode_roofline(spec, wl.seqlens, ms, read_traffic(kind_of(spec), spec.name))
    out["cache_replicas"] = len(reps)
    out["tokens_in_cache"] = int(wl.tokens)
    out["batch"], out["q_len"] = spec.batch, spec.q_len
    del reps, db
    torch.cuda.empty_cache()
    return out


def streaming_object(launches, sink_pages=1, window_pages=64):
    """Decode over the StreamingLLM-style eviction view of the long-context
    workload (B=16, L uniform in 16K..64K): 1 sink page and a recent window of
    at least 64 pages (4096 tokens) kept per sequence.  Times the view kernel
    and the decode over the kept pages; the roofline is over the kept tokens'
    bytes (cache replicated until the kept pages exceed twice the last-level
    cache)."""
    import torch
    from head_latent_attention_03_amd import inputs
    from head_latent_attention_03_amd.runner import DeviceBatch
    spec = inputs.workload(3)
    wl = inputs.make_workload(spec)
    db = DeviceBatch.from_workload(wl, "cuda:0")
    db.absorb()
    sl, bt, ms_view = db.streaming_view(sink_pages, window_pages)
    torch.cuda.synchronize()
    kept = sl.cpu().numpy()
    per_tok = spec.d_c * 2 + spec.d_rope * 2
    reps = replicate_cache(db, read_bytes=int(kept.sum()) * per_tok)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        db.streaming_view(sink_pages, window_pages)
    e1.record()
    torch.cuda.synchronize()
    view_us = e0.elapsed_time(e1) / 20 * 1e3
    ms = time_decode(db, reps, launches, block_table=bt, seqlens=sl, max_seqlen=ms_view)
    out = decode_roofline(spec, kept, ms, None)
    out["workload"] = spec.name + "-streaming-sink1-win64"
    out["tokens_kept"] = int(kept.sum())
    out["tokens_in_cache"] = int(wl.tokens)
    out["view_kernel_us"] = round(view_us, 2)
    out["cache_replicas"] = len(reps)
    out["batch"], out["q_len"] = spec.batch, spec.q_len
    del reps, db
    torch.cuda.empty_cache()
    return out


def plan_split_counts(tiles, row_groups, G):
    """Chunks per sequence of the decode's split plan (the same rule as the
    kernels'): proportional counts p = min(t, max(1, floor(G t / NT))) set a
    chunk budget, B = G when they total at most G and G + U (U units) when
    not; the chunk length is the shortest C with sum ceil(t / C) <= B, and a
    sequence of t tiles gets ceil(t / C) chunks."""
    nt = sum(tiles) * row_groups
    if nt == 0:
        return [0] * len(tiles)
    p = [min(t, max(1, G * t // nt)) if t > 0 else 0 for t in tiles]
    budget = G if sum(p) * row_groups <= G else G + len(tiles) * row_groups
    count = lambda c: sum(-(-t // c) for t in tiles) * row_groups
    lo, hi = -(-nt // budget), max(-(-t // q) for t, q in zip(tiles, p) if q > 0)
    while lo < hi:
        mid = (lo + hi) // 2
        lo, hi = (lo, mid) if count(mid) <= budget else (mid + 1, hi)
    return [-(-t // hi) for t in tiles]


def second_pass_share(wl, cus, limit=108.75):
    """Share of the e4m3 decode's workgroups that must run their chunk twice on
    workload `wl`, from the exact scores (fp32 numpy on the stored values; the
    kernel's e4m3 query moves them slightly): the plan cuts each sequence into
    chunks of 32-token tiles (plan_split_counts for G compute units).  The
    kernel works on v_t = s_t +
    log2(token scale) (log2 units); a row's reference is its largest v in the
    chunk's first tile, and the chunk is redone when any later v of any of its
    rows passes that reference by more than `limit`: 100 for the largest
    block exponent the kernel keeps plus the 8.75 by which a tile's largest
    probability sits above 2^exponent."""
    spec = wl.spec
    scale = spec.scale() * math.log2(math.e)
    dec = lambda a, dt: (a.astype(np.uint32) << 16).view(np.float32) if dt == "bf16" else a
    e4m3 = np.array([(-1.0 if c & 0x80 else 1.0) * ((c & 7) * 2.0 ** -9 if (c >> 3) & 15 == 0
                     else (1 + (c & 7) / 8) * 2.0 ** (((c >> 3) & 15) - 7)) for c in range(256)],
                    dtype=np.float32)
    w_uk = dec(wl.w_uk, "bf16")
    rows_groups = (spec.q_len * spec.n_heads + 127) // 128
    tiles = [(int(L) + 31) // 32 for L in wl.seqlens]
    splits = plan_split_counts(tiles, rows_groups, cus)
    redo = chunks = 0
    for b, L in enumerate(wl.seqlens):
        L = int(L)
        if L == 0:
            continue
        pages = wl.block_table[b, :(L + 63) // 64]
        lat = e4m3[wl.kv_latent[pages].reshape(-1, spec.d_c)[:L]] \
            * wl.kv_scale[pages].reshape(-1)[:L, None]
        kr = dec(wl.kv_rope[pages].reshape(-1, spec.d_rope)[:L], "bf16")
        qn = dec(wl.q_nope[b], "bf16").reshape(-1, spec.d_nope)        # [q_len H, d_nope]
        qr = dec(wl.q_rope[b], "bf16").reshape(-1, spec.d_rope)
        pos = L - spec.q_len + np.repeat(np.arange(spec.q_len), spec.n_heads)
        theta = 10000.0 ** (-2.0 * np.arange(spec.d_rope // 2) / spec.d_rope)
        ang = pos[:, None] * theta[None, :]
        qpe = np.empty_like(qr)
        qpe[:, 0::2] = qr[:, 0::2] * np.cos(ang) - qr[:, 1::2] * np.sin(ang)
        qpe[:, 1::2] = qr[:, 0::2] * np.sin(ang) + qr[:, 1::2] * np.cos(ang)
        heads = np.tile(np.arange(spec.n_heads), spec.q_len)
        qlat = np.einsum("rn,rnc->rc", qn, w_uk[heads])
        sc = (qlat @ lat.T + qpe @ kr.T) * scale                      # [rows, L]
        sc = sc + np.log2(wl.kv_scale[pages].reshape(-1)[:L])[None, :]
        lim = pos + 1
        sc[np.arange(L)[None, :] >= lim[:, None]] = -np.inf
        n_t = tiles[b]
        s_u = splits[b]
        for c in range(s_u):
            k0, k1 = c * n_t // s_u, (c + 1) * n_t // s_u
            first = sc[:, k0 * 32:min((k0 + 1) * 32, L)].max(axis=1)
            later = sc[:, (k0 + 1) * 32:min(k1 * 32, L)]
            jump = later.shape[1] > 0 and bool(np.any(later.max(axis=1) > first + limit))
            chunks += rows_groups
            redo += rows_groups if jump else 0
    return redo / max(chunks, 1)


def fp8_second_pass_object(launches, cus):
    """The e4m3 decode on the B=64 L=4096 e4m3 workload as drawn, with peaked
    attention (N(0,1)/sqrt(dim) inputs, softmax scale 2) and with scores spread
    over hundreds of log2 units (softmax scale 64, far past any trained
    model's): launch times and the share of workgroups whose chunk must be run
    twice."""
    import torch
    from head_latent_attention_03_amd import inputs
    from head_latent_attention_03_amd.runner import DeviceBatch
    out = {}
    for name, over in (("as_drawn", {}), ("peaked", dict(init="fan_in", softmax_scale=2.0)),
                       ("extreme", dict(init="fan_in", softmax_scale=64.0))):
        spec = inputs.workload(4, **over)
        wl = inputs.make_workload(spec)
        share = second_pass_share(wl, cus)
        db = DeviceBatch.from_workload(wl, "cuda:0")
        reps = replicate_cache(db)
        db.absorb()
        ms = time_decode(db, reps, launches)
        out[name] = {"launch_ms": round(float(np.mean(ms)), 5),
                     "launch_ms_median": round(float(np.median(ms)), 5),
                     "second_pass_share_estimate": round(share, 4)}
        del reps, db
        torch.cuda.empty_cache()
    out["note"] = ("share: workgroups whose chunk has a score (plus log2 of its token scale) "
                   "more than 108.75 log2 units past its first tile's row maximum, from the "
                   "exact scores")
    return out


def prefill_flops(spec, seqlens):
    """Algorithmic flops of the non-absorbed path: the expansion (2 d_c (d_nope + d_v)
    per cached token and head) and the causal attention (2 (d_nope + d_R + d_v) per
    visible key, query row and head)."""
    L = seqlens.astype(np.int64)
    H, S = spec.n_heads, spec.q_len
    expand = 2 * int(L.sum()) * spec.d_c * (spec.d_nope + spec.d_v) * H
    vis = sum(int(np.sum(np.clip(L - S + j + 1, 0, None))) for j in range(S))
    attend = 2 * vis * H * (spec.d_nope + spec.d_rope + spec.d_v)
    absorbed = 2 * vis * H * (2 * spec.d_c + spec.d_rope)
    return expand, attend, absorbed


def prefill_object(launches):
    """mla_prefill_paged (expand K^C and V per head, then causal attention) on a
    chunked-prefill batch: launch durations (HIP events) and the MFMA roofline."""
    import torch
    from head_latent_attention_03_amd import inputs
    from head_latent_attention_03_amd import _binding as B
    from head_latent_attention_03_amd.runner import dims_of, _to_device
    spec = inputs.prefill_workload()
    wl = inputs.make_workload(spec)
    dev = torch.device("cuda:0")
    dims = dims_of(spec)
    t = {k: _to_device(getattr(wl, k), dt, dev) for k, dt in
         (("q_nope", "bf16"), ("q_rope", "bf16"), ("kv_latent", "bf16"), ("kv_rope", "bf16"),
          ("w_uk", "bf16"), ("w_uv", "bf16"), ("block_table", "i32"), ("seqlens", "i32"))}
    ws = torch.empty(B.mla_prefill_workspace_size(dims, spec.batch, wl.max_seqlen),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((spec.batch, spec.q_len, spec.n_heads, spec.d_v), dtype=torch.bfloat16,
                      device=dev)
    call = lambda: B.mla_prefill_paged(dims, t["q_nope"], t["q_rope"], t["kv_latent"],
                                       t["kv_rope"], t["block_table"], t["seqlens"],
                                       wl.max_seqlen, t["w_uk"], t["w_uv"], ws, out)
    ms = time_launches(lambda i: call(), launches, warm=3, batch=1)
    expand, attend, absorbed = prefill_flops(spec, wl.seqlens)
    mean = float(np.mean(ms))
    tfs = (expand + attend) / (mean * 1e-3) / 1e12
    del t, ws, out
    torch.cuda.empty_cache()
    return {
        "kernel": "mla_prefill_paged (expand_kv_kernel + attn_kernel)",
        "workload": spec.name, "batch": spec.batch, "q_len": spec.q_len,
        "tokens_in_cache": int(wl.tokens), "bound": "mfma",
        "achieved": round(tfs, 2), "peak": MFMA_PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
        "frac": round(tfs / MFMA_PEAK_TFLOPS["bf16"], 4),
        "launch_ms": round(mean, 5), "launch_ms_median": round(float(np.median(ms)), 5),
        "launch_ms_p10": round(float(np.percentile(ms, 10)), 5),
        "launch_ms_p90": round(float(np.percentile(ms, 90)), 5), "timed_launches": launches,
        "algorithmic_flops": int(expand + attend), "expand_flops": int(expand),
        "attend_flops": int(attend), "absorbed_form_flops": int(absorbed),
        "query_tokens_per_s": round(spec.batch * spec.q_len / (mean * 1e-3), 1),
    }


def projection_object(launches, tokens=4096, d_model=7168, d_cq=1536, d_c=512, d_r=64):
    """mla_gemm_bf16 as the latent down-projection of a prefill chunk: [c^Q | c^KV |
    k^R] = [W^DQ; W^DKV; W^KR] h for `tokens` hidden states (bf16, fp32 accumulate),
    timed with HIP events, against the bf16 MFMA roofline.  The widths stand in for a
    DeepSeek-V3-sized layer (the pages give the attention shape, not d_model or d_cq)."""
    import torch
    from head_latent_attention_03_amd import _binding as B
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(1007)
    n = d_cq + d_c + d_r
    h = (torch.randn((tokens, d_model), generator=g) * 0.02).to(torch.bfloat16).to(dev)
    w = (torch.randn((n, d_model), generator=g) / d_model ** 0.5).to(torch.bfloat16).to(dev)
    out = torch.empty((tokens, n), dtype=torch.bfloat16, device=dev)
    ms = time_launches(lambda i: B.mla_gemm_bf16(h, w, out), launches, warm=5, batch=5)
    flops = 2 * tokens * n * d_model
    mean = float(np.mean(ms))
    tfs = flops / (mean * 1e-3) / 1e12
    del h, w, out
    torch.cuda.empty_cache()
    return {
        "kernel": "mla_gemm_bf16 (gemm_nt_wide_kernel, 256 x 160 tiles)",
        "workload": f"latent-down-projection-t{tokens}-dmodel{d_model}-n{n}",
        "bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_PEAK_TFLOPS["bf16"],
        "unit": "TFLOP/s", "frac": round(tfs / MFMA_PEAK_TFLOPS["bf16"], 4),
        "launch_ms": round(mean, 5), "launch_ms_median": round(float(np.median(ms)), 5),
        "timed_launches": launches, "algorithmic_flops": int(flops),
        "algorithmic_bytes": int(2 * (tokens * d_model + n * d_model + tokens * n)),
    }


def cpu_info():
    """CPU model name and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


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


EXTRA_WORKLOADS = {"e4m3_cache": 4, "long_context": 3, "mtp2": 5, "prefill": "prefill",
                   "projection": "projection", "e4m3_second_pass": "second_pass",
                   "streaming_eviction": "streaming"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--decode-launches", type=int, default=100,
                    help="decode launches timed one by one for each roofline object")
    ap.add_argument("--extra", default="e4m3_cache,long_context,mtp2,prefill,projection,"
                                       "e4m3_second_pass,streaming_eviction",
                    help="comma-separated decode-only objects for the other workloads "
                         f"({', '.join(EXTRA_WORKLOADS)}; empty: none)")
    ap.add_argument("--decode-only", type=int, default=0, metavar="N",
                    help="time only the decode of workload N (for profiling runs) and exit")
    ap.add_argument("--object", choices=["prefill", "projection", "e4m3_second_pass",
                                         "streaming_eviction"],
                    help="time only this extra object (for profiling runs) and exit")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0: skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size before the first decode "
                         "(counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the decode traffic summary from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--pmc-command", action="append", default=[],
                    help="command lines of the counter runs, recorded in the summary")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("DB_GLOB", "OUT_NAME", "TITLE"),
                    help="write profiles/OUT_NAME from rocprofv3 --kernel-trace databases "
                         "(the --pmc-command lines are recorded) and exit")
    ap.add_argument("--trace-window", nargs=3, metavar=("KERNEL", "FIRST", "END"),
                    help="with --summarize-trace: also the statistics of calls FIRST .. END-1 "
                         "of the kernel whose name contains KERNEL")
    ap.add_argument("--bench-log", help="with --summarize-trace: the bench output of the same "
                                        "run, whose roofline timing is recorded")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("DB_GLOB", "OUT_NAME", "TITLE"),
                    help="write profiles/OUT_NAME with per-kernel averages of the counters "
                         "in rocprofv3 --pmc databases and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.pmc_command)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.pmc_command, args.trace_window, args.bench_log)
        return
    if args.summarize_pmc:
        from head_latent_attention_03_amd import inputs
        spec = inputs.workload(args.decode_only or args.config)
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], kind_of(spec), spec.name,
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
    if args.object:
        if args.object == "prefill":
            obj = prefill_object(max(5, args.decode_launches // 5))
        elif args.object == "projection":
            obj = projection_object(max(10, args.decode_launches // 2))
        elif args.object == "streaming_eviction":
            obj = streaming_object(args.decode_launches)
        else:
            obj = fp8_second_pass_object(max(10, args.decode_launches // 2),
                                         torch.cuda.get_device_properties(0).multi_processor_count)
        print(json.dumps(obj), flush=True)
        return
    if args.decode_only:
        obj = decode_object(args.decode_only, args.decode_launches, args.copy_calibration_mib)
        print(json.dumps(obj), flush=True)
        return

    spec = inputs.workload(args.config)
    wl = inputs.make_workload(spec)
    db = DeviceBatch.from_workload(wl, "cuda:0")
    reps = replicate_cache(db)
    n_rep = len(reps)
    torch.cuda.synchronize()
    if args.copy_calibration_mib > 0:
        calibration_copy(args.copy_calibration_mib)

    def step(i):
        lat, sc, rope = reps[i % n_rep]
        db.absorb()
        db.decode(kv_latent=lat, kv_scale=sc, kv_rope=rope)
        db.combine(with_uv=True)

    # the clock's own warm-up, then the W counted warm-up steps (all untimed)
    warm_steps = warm_clock(step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    progress(f"{args.steps} steps: {ms_step * 1e3:.1f} us per step")

    # the dominant kernel, timed launch by launch in its own loop (HIP events on
    # the launch stream; the events are kept out of the step loop above, whose
    # time they would add to)
    dec_ms = time_decode(db, reps, max(20, args.decode_launches))
    roof = decode_roofline(spec, wl.seqlens, dec_ms, read_traffic(kind_of(spec), spec.name))
    progress(f"decode roofline: {roof['launch_ms'] * 1e3:.1f} us per launch")

    # the cache append of the step's new tokens (the step before decode, timed
    # on its own: it is not part of the metric's step)
    app_us = append_time(spec, db, torch.cuda.current_stream(), args.steps)

    alg = algorithmic(spec, wl.seqlens)
    step_bytes = sum(v[0] for k, v in alg.items() if k in ("absorb", "decode", "combine"))
    step_flops = sum(v[1] for k, v in alg.items() if k in ("absorb", "decode", "combine"))
    kind = kind_of(spec)
    out = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_warmup": {"seconds": CLOCK_WARM_S, "steps": warm_steps,
                         "note": "untimed steps run before the W warm-up steps, until the GPU "
                                 "clock has had half a second of continuous work"},
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
        "roofline": roof,
    }
    app_b = alg["append"]
    out["append"] = {
        "kernel": "mla_append_kv", "us": round(app_us, 3), "tokens": spec.batch * spec.q_len,
        "algorithmic_bytes": int(app_b),
        "achieved_gbs": round(app_b / (app_us * 1e-6) / 1e9, 2),
        "note": "one wave per new token; at this size the launch latency is the bound, "
                "not HBM (the bytes would take well under 1 us at 8 TB/s)",
    }
    del reps, db
    torch.cuda.empty_cache()
    if args.config == 2:
        for name in [x for x in args.extra.split(",") if x]:
            if EXTRA_WORKLOADS[name] == "prefill":
                out[name] = prefill_object(max(5, args.decode_launches // 5))
            elif EXTRA_WORKLOADS[name] == "projection":
                out[name] = projection_object(max(10, args.decode_launches // 2))
            elif EXTRA_WORKLOADS[name] == "streaming":
                out[name] = streaming_object(args.decode_launches)
            elif EXTRA_WORKLOADS[name] == "second_pass":
                out[name] = fp8_second_pass_object(max(10, args.decode_launches // 2),
                                                   torch.cuda.get_device_properties(0).multi_processor_count)
            else:
                out[name] = decode_object(EXTRA_WORKLOADS[name], args.decode_launches)
            progress(f"object {name} done")
    if args.cpu_budget > 0:
        progress(f"cpu baseline: about {args.cpu_budget:.0f} s of the oracle")
        t_cpu, frac, rows_done, threads = cpu_baseline(wl, args.cpu_budget)
        full_s = t_cpu / frac
        model, cores = cpu_info()
        out["cpu_baseline"] = {
            "value": round(step_bytes / full_s / 1e9, 6),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"{rows_done} of {spec.batch * spec.q_len * spec.n_heads} (b, j, h) rows "
                      f"of the same workload in {t_cpu:.1f} s, scaled to the whole step",
            "seconds_per_step": round(full_s, 2),
            "cpu_model": model,
            "cores_available": cores,
            "threads_note": "cores = the BLAS threads the fp64 oracle ran on",
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
