"""Build the gfx950 MLA decode library (libmla_decode.so) in-tree with hipcc.

    python -m head_latent_attention_03_amd.build      (or build() from Python)

Every source under csrc/ is compiled for gfx950 only, in parallel, and linked
into head_latent_attention_03_amd/libmla_decode.so.  Objects go to _build/.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla_decode.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 VALU ops stay disabled (the compiler would otherwise form
    # v_pk_{add,mul,fma}_f32 from ordinary float code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# per-source extra flags: the bf16 and e4m3 decodes select the VGPR form for
# the MFMAs the compiler emits (the score accumulators are read by VALU code),
# while their output accumulators are pinned to the accumulation registers by
# hand
EXTRA_FLAGS = {
    "decode_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "decode_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    out = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith(".hip") or name.endswith(".cpp"):
            out.append(os.path.join(CSRC, name))
    return out


def _compile(hipcc, src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = EXTRA_FLAGS.get(os.path.basename(src), [])
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc, "-x", "hip", *cmd[1:]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)
    return obj


def build(verbose=False, jobs=None):
    """Compile every source and link the shared library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {LIB} failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
