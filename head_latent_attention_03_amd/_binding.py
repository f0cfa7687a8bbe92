"""Thin ctypes binding of libmla_decode.so (include/mla_decode.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their device pointers and the current HIP stream are passed
to the C entry points of the same names.  Every computation runs in the HIP
kernels.  PyTorch is used only for device memory and streams.
"""

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG, "libmla_decode.so")

MLA_F32, MLA_BF16, MLA_FP8_E4M3 = 0, 1, 2
_DT = {"f32": MLA_F32, "bf16": MLA_BF16, "e4m3": MLA_FP8_E4M3}
_TORCH_DT = {MLA_F32: torch.float32, MLA_BF16: torch.bfloat16, MLA_FP8_E4M3: torch.float8_e4m3fn}

STATUS = {
    0: "MLA_OK", 1: "MLA_ERR_NULL_POINTER", 2: "MLA_ERR_BAD_SHAPE", 3: "MLA_ERR_BAD_DTYPE",
    4: "MLA_ERR_MISALIGNED", 5: "MLA_ERR_WORKSPACE_TOO_SMALL", 6: "MLA_ERR_UNSUPPORTED",
    7: "MLA_ERR_HIP", 8: "MLA_ERR_SCRATCH_TOO_SMALL",
}


class MlaError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed: {msg}")
        self.code = code


class _Dims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("d_nope", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("latent_dtype", ctypes.c_int32)]


@dataclass(frozen=True)
class MlaDims:
    """Problem dimensions (mirrors mla_dims_t)."""
    n_heads: int
    d_latent: int
    d_rope: int
    d_nope: int
    d_v: int
    page_size: int
    softmax_scale: float
    rope_base: float
    act_dtype: str = "bf16"      # 'f32' or 'bf16'
    latent_dtype: str = "bf16"   # 'f32', 'bf16' or 'e4m3'

    def c(self):
        return _Dims(self.n_heads, self.d_latent, self.d_rope, self.d_nope, self.d_v,
                     self.page_size, self.softmax_scale, self.rope_base,
                     _DT[self.act_dtype], _DT[self.latent_dtype])

    @property
    def act_torch(self):
        return _TORCH_DT[_DT[self.act_dtype]]

    @property
    def latent_torch(self):
        return _TORCH_DT[_DT[self.latent_dtype]]


_lib = None
_P = ctypes.c_void_p


def load_library(path=LIBRARY_PATH):
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first with "
                           "`python -m head_latent_attention_03_amd.build`")
    lib = ctypes.CDLL(path)
    i32, f32p, i32p = ctypes.c_int32, ctypes.POINTER(ctypes.c_float), _P
    dp = ctypes.POINTER(_Dims)
    lib.mla_absorb_q.argtypes = [dp, i32, i32, _P, _P, i32p, _P, _P, _P, _P, _P]
    lib.mla_absorb_q.restype = ctypes.c_int
    lib.mla_decode_workspace_size.argtypes = [dp, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_decode_workspace_size.restype = ctypes.c_int
    lib.mla_decode_paged.argtypes = [dp, i32, i32, i32, _P, _P, _P, _P, _P, _P, i32, _P, i32,
                                     _P, i32, _P, ctypes.c_size_t, _P]
    lib.mla_decode_paged.restype = ctypes.c_int
    lib.mla_combine.argtypes = [dp, i32, i32, _P, ctypes.c_size_t, _P, i32, _P, _P, _P, _P]
    lib.mla_combine.restype = ctypes.c_int
    lib.mla_append_kv.argtypes = [dp, i32, i32, _P, _P, _P, ctypes.c_float, i32p, i32p, i32,
                                  _P, _P, _P, i32, _P]
    lib.mla_append_kv.restype = ctypes.c_int
    lib.mla_streaming_view.argtypes = [dp, i32, i32p, i32p, i32, i32, i32, i32p, i32p, i32, _P]
    lib.mla_streaming_view.restype = ctypes.c_int
    lib.mla_validate_paged_host.argtypes = [dp, i32, i32, _P, i32, _P, i32,
                                            ctypes.POINTER(ctypes.c_int32)]
    lib.mla_validate_paged_host.restype = ctypes.c_int
    lib.mla_decode_noalloc.argtypes = [dp, i32, i32, i32, _P, _P, _P, _P, _P, _P, i32, _P, i32,
                                       _P, i32, _P, _P, _P, _P]
    lib.mla_decode_noalloc.restype = ctypes.c_int
    lib.mla_prefill_workspace_size.argtypes = [dp, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_prefill_workspace_size.restype = ctypes.c_int
    lib.mla_prefill_paged.argtypes = [dp, i32, i32, _P, _P, _P, _P, i32, _P, i32, _P, i32, _P,
                                      _P, _P, ctypes.c_size_t, _P, _P, _P]
    lib.mla_prefill_paged.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.mla_gemm_bf16.argtypes = [i32, i32, i32, i32, _P, i64, i64, _P, i64, i64, _P, i32, i64,
                                  i64, _P]
    lib.mla_gemm_bf16.restype = ctypes.c_int
    lib.mla_absorb_weights_workspace_size.argtypes = [dp, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_absorb_weights_workspace_size.restype = ctypes.c_int
    lib.mla_absorb_query_weights.argtypes = [dp, i32, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.mla_absorb_query_weights.restype = ctypes.c_int
    lib.mla_absorb_output_weights.argtypes = [dp, i32, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.mla_absorb_output_weights.restype = ctypes.c_int
    lib.mla_query_from_latent.argtypes = [dp, i32, i32, i32, _P, _P, _P, _P, _P, _P, _P]
    lib.mla_query_from_latent.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def mla_status_string(code):
    return load_library().mla_status_string(int(code)).decode()


def _check(fn, code):
    if code != 0:
        raise MlaError(fn, code, mla_status_string(code))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _expect(name, t, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def mla_absorb_q(dims, q_nope, q_rope, seqlens, w_uk, q_latent, q_latent_scale, q_pe,
                 stream=None):
    """q~ = W_UK[h]^T q^C and q_pe = RoPE(q^R); see mla_absorb_q in mla_decode.h."""
    B, S, H = q_nope.shape[0], q_nope.shape[1], dims.n_heads
    dev = q_nope.device
    act = dims.act_torch
    _expect("q_nope", q_nope, (B, S, H, dims.d_nope), act, dev)
    _expect("q_rope", q_rope, (B, S, H, dims.d_rope), act, dev)
    _expect("seqlens", seqlens, (B,), torch.int32, dev)
    _expect("w_uk", w_uk, (H, dims.d_nope, dims.d_latent), act, dev)
    lat_dt = torch.float8_e4m3fn if dims.latent_dtype == "e4m3" else act
    _expect("q_latent", q_latent, (B, S, H, dims.d_latent), lat_dt, dev)
    if dims.latent_dtype == "e4m3":
        _expect("q_latent_scale", q_latent_scale, (B, S, H), torch.float32, dev)
    _expect("q_pe", q_pe, (B, S, H, dims.d_rope), act, dev)
    d = dims.c()
    lib = load_library()
    _check("mla_absorb_q", lib.mla_absorb_q(
        ctypes.byref(d), B, S, _ptr(q_nope), _ptr(q_rope), _ptr(seqlens), _ptr(w_uk),
        _ptr(q_latent), _ptr(q_latent_scale), _ptr(q_pe), _stream(stream)))


def mla_validate_paged_host(dims, num_pages, block_table, seqlens, max_seqlen):
    """Host check of the decode's block-table and length preconditions on numpy
    int32 arrays; returns (status code, number of failing sequences)."""
    import numpy as np
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    if bt.ndim != 2 or sl.shape != (bt.shape[0],):
        raise ValueError("block_table must be [batch, max_pages] and seqlens [batch]")
    d = dims.c()
    bad = ctypes.c_int32(-1)
    code = load_library().mla_validate_paged_host(
        ctypes.byref(d), bt.shape[0], int(num_pages), bt.ctypes.data_as(_P), bt.shape[1],
        sl.ctypes.data_as(_P), int(max_seqlen), ctypes.byref(bad))
    return int(code), int(bad.value)


def mla_decode_workspace_size(dims, batch, q_len, max_seqlen):
    d = dims.c()
    n = ctypes.c_size_t(0)
    _check("mla_decode_workspace_size", load_library().mla_decode_workspace_size(
        ctypes.byref(d), int(batch), int(q_len), int(max_seqlen), ctypes.byref(n)))
    return int(n.value)


def mla_decode_paged(dims, q_latent, q_latent_scale, q_pe, kv_latent, kv_scale, kv_rope,
                     block_table, seqlens, max_seqlen, workspace, causal=True, stream=None):
    """Split-KV attention over the paged latent cache; see mla_decode_paged in mla_decode.h."""
    B, S, H = q_latent.shape[0], q_latent.shape[1], dims.n_heads
    dev = q_latent.device
    act = dims.act_torch
    P = kv_latent.shape[0]
    lat_dt = torch.float8_e4m3fn if dims.latent_dtype == "e4m3" else act
    _expect("q_latent", q_latent, (B, S, H, dims.d_latent), lat_dt, dev)
    if dims.latent_dtype == "e4m3":
        _expect("q_latent_scale", q_latent_scale, (B, S, H), torch.float32, dev)
        _expect("kv_scale", kv_scale, (P, dims.page_size), torch.float32, dev)
    _expect("q_pe", q_pe, (B, S, H, dims.d_rope), act, dev)
    _expect("kv_latent", kv_latent, (P, dims.page_size, dims.d_latent), dims.latent_torch, dev)
    _expect("kv_rope", kv_rope, (P, dims.page_size, dims.d_rope), act, dev)
    _expect("block_table", block_table, (B, block_table.shape[1]), torch.int32, dev)
    _expect("seqlens", seqlens, (B,), torch.int32, dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same device")
    d = dims.c()
    _check("mla_decode_paged", load_library().mla_decode_paged(
        ctypes.byref(d), B, S, int(bool(causal)), _ptr(q_latent), _ptr(q_latent_scale),
        _ptr(q_pe), _ptr(kv_latent), _ptr(kv_scale), _ptr(kv_rope), P, _ptr(block_table),
        block_table.shape[1], _ptr(seqlens), int(max_seqlen), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_combine(dims, workspace, seqlens, max_seqlen, w_uv, out, lse=None, q_len=1,
                stream=None):
    """Merge the splits, then out = W_UV[h] o~ (or o~ when w_uv is None); see mla_combine."""
    B, H = seqlens.shape[0], dims.n_heads
    dev = seqlens.device
    act = dims.act_torch
    _expect("seqlens", seqlens, (B,), torch.int32, dev)
    if w_uv is not None:
        _expect("w_uv", w_uv, (H, dims.d_v, dims.d_latent), act, dev)
        _expect("out", out, (B, q_len, H, dims.d_v), act, dev)
    else:
        _expect("out", out, (B, q_len, H, dims.d_latent), act, dev)
    if lse is not None:
        _expect("lse", lse, (B, q_len, H), torch.float32, dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same device")
    d = dims.c()
    _check("mla_combine", load_library().mla_combine(
        ctypes.byref(d), B, int(q_len), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(seqlens), int(max_seqlen),
        _ptr(w_uv), _ptr(out), _ptr(lse), _stream(stream)))


def mla_append_kv(dims, kv_c, k_rope, norm_weight, norm_eps, seqlens, block_table, kv_latent,
                  kv_scale, kv_rope, stream=None):
    """Write the step's new tokens (RMSNorm'd latent, rotated k^R) into the paged cache;
    see mla_append_kv in mla_decode.h."""
    B, S = kv_c.shape[0], kv_c.shape[1]
    dev = kv_c.device
    act = dims.act_torch
    P = kv_latent.shape[0]
    _expect("kv_c", kv_c, (B, S, dims.d_latent), act, dev)
    _expect("k_rope", k_rope, (B, S, dims.d_rope), act, dev)
    _expect("norm_weight", norm_weight, (dims.d_latent,), act, dev)
    _expect("seqlens", seqlens, (B,), torch.int32, dev)
    _expect("block_table", block_table, (B, block_table.shape[1]), torch.int32, dev)
    _expect("kv_latent", kv_latent, (P, dims.page_size, dims.d_latent), dims.latent_torch, dev)
    if dims.latent_dtype == "e4m3":
        _expect("kv_scale", kv_scale, (P, dims.page_size), torch.float32, dev)
    _expect("kv_rope", kv_rope, (P, dims.page_size, dims.d_rope), act, dev)
    d = dims.c()
    _check("mla_append_kv", load_library().mla_append_kv(
        ctypes.byref(d), B, S, _ptr(kv_c), _ptr(k_rope), _ptr(norm_weight), float(norm_eps),
        _ptr(seqlens), _ptr(block_table), block_table.shape[1], _ptr(kv_latent),
        _ptr(kv_scale), _ptr(kv_rope), P, _stream(stream)))


def mla_streaming_view(dims, seqlens, block_table, sink_pages, window_pages, out_seqlens,
                       out_block_table, stream=None):
    """The eviction view (kept sink pages and recent window) of a paged cache as new
    lengths and a new block table; see mla_streaming_view in mla_decode.h."""
    B = seqlens.shape[0]
    dev = seqlens.device
    _expect("seqlens", seqlens, (B,), torch.int32, dev)
    _expect("block_table", block_table, (B, block_table.shape[1]), torch.int32, dev)
    _expect("out_seqlens", out_seqlens, (B,), torch.int32, dev)
    _expect("out_block_table", out_block_table, (B, out_block_table.shape[1]), torch.int32, dev)
    d = dims.c()
    _check("mla_streaming_view", load_library().mla_streaming_view(
        ctypes.byref(d), B, _ptr(seqlens), _ptr(block_table), block_table.shape[1],
        int(sink_pages), int(window_pages), _ptr(out_seqlens), _ptr(out_block_table),
        out_block_table.shape[1], _stream(stream)))


def mla_decode_noalloc(dims, q_latent, q_latent_scale, q_pe, kv_latent, kv_scale, kv_rope,
                       block_table, seqlens, max_seqlen, w_uv, out, lse=None, causal=True,
                       stream=None):
    """Decode and merge with the library's static scratch (no workspace); see
    mla_decode_noalloc in mla_decode.h."""
    B, S, H = q_latent.shape[0], q_latent.shape[1], dims.n_heads
    dev = q_latent.device
    act = dims.act_torch
    P = kv_latent.shape[0]
    lat_dt = torch.float8_e4m3fn if dims.latent_dtype == "e4m3" else act
    _expect("q_latent", q_latent, (B, S, H, dims.d_latent), lat_dt, dev)
    if dims.latent_dtype == "e4m3":
        _expect("q_latent_scale", q_latent_scale, (B, S, H), torch.float32, dev)
        _expect("kv_scale", kv_scale, (P, dims.page_size), torch.float32, dev)
    _expect("q_pe", q_pe, (B, S, H, dims.d_rope), act, dev)
    _expect("kv_latent", kv_latent, (P, dims.page_size, dims.d_latent), dims.latent_torch, dev)
    _expect("kv_rope", kv_rope, (P, dims.page_size, dims.d_rope), act, dev)
    _expect("block_table", block_table, (B, block_table.shape[1]), torch.int32, dev)
    _expect("seqlens", seqlens, (B,), torch.int32, dev)
    if w_uv is not None:
        _expect("w_uv", w_uv, (H, dims.d_v, dims.d_latent), act, dev)
        _expect("out", out, (B, S, H, dims.d_v), act, dev)
    else:
        _expect("out", out, (B, S, H, dims.d_latent), act, dev)
    if lse is not None:
        _expect("lse", lse, (B, S, H), torch.float32, dev)
    d = dims.c()
    _check("mla_decode_noalloc", load_library().mla_decode_noalloc(
        ctypes.byref(d), B, S, int(bool(causal)), _ptr(q_latent), _ptr(q_latent_scale),
        _ptr(q_pe), _ptr(kv_latent), _ptr(kv_scale), _ptr(kv_rope), P, _ptr(block_table),
        block_table.shape[1], _ptr(seqlens), int(max_seqlen), _ptr(w_uv), _ptr(out), _ptr(lse),
        _stream(stream)))


def mla_prefill_workspace_size(dims, batch, max_seqlen):
    d = dims.c()
    n = ctypes.c_size_t(0)
    _check("mla_prefill_workspace_size", load_library().mla_prefill_workspace_size(
        ctypes.byref(d), int(batch), int(max_seqlen), ctypes.byref(n)))
    return int(n.value)


def mla_prefill_paged(dims, q_nope, q_rope, kv_latent, kv_rope, block_table, seqlens,
                      max_seqlen, w_uk, w_uv, workspace, out, lse=None, stream=None):
    """Non-absorbed causal attention of q_len query tokens per sequence; see
    mla_prefill_paged in mla_decode.h."""
    B, S, H = q_nope.shape[0], q_nope.shape[1], dims.n_heads
    dev = q_nope.device
    act = dims.act_torch
    P = kv_latent.shape[0]
    _expect("q_nope", q_nope, (B, S, H, dims.d_nope), act, dev)
    _expect("q_rope", q_rope, (B, S, H, dims.d_rope), act, dev)
    _expect("kv_latent", kv_latent, (P, dims.page_size, dims.d_latent), dims.latent_torch, dev)
    _expect("kv_rope", kv_rope, (P, dims.page_size, dims.d_rope), act, dev)
    _expect("block_table", block_table, (B, block_table.shape[1]), torch.int32, dev)
    _expect("seqlens", seqlens, (B,), torch.int32, dev)
    _expect("w_uk", w_uk, (H, dims.d_nope, dims.d_latent), act, dev)
    _expect("w_uv", w_uv, (H, dims.d_v, dims.d_latent), act, dev)
    _expect("out", out, (B, S, H, dims.d_v), act, dev)
    if lse is not None:
        _expect("lse", lse, (B, S, H), torch.float32, dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same device")
    d = dims.c()
    _check("mla_prefill_paged", load_library().mla_prefill_paged(
        ctypes.byref(d), B, S, _ptr(q_nope), _ptr(q_rope), _ptr(kv_latent), _ptr(kv_rope), P,
        _ptr(block_table), block_table.shape[1], _ptr(seqlens), int(max_seqlen), _ptr(w_uk),
        _ptr(w_uv), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
        _ptr(lse), _stream(stream)))


def mla_gemm_bf16(a, b, c, stream=None):
    """c[i] = a[i] @ b[i]^T for 2-D or 3-D (batched) bf16 tensors (a [.., m, k],
    b [.., n, k], c [.., m, n] bf16 or f32; a 2-D operand is shared by every
    batch entry); see mla_gemm_bf16 in mla_decode.h."""
    batch = max(t.shape[0] if t.dim() == 3 else 1 for t in (a, b, c))
    def geo(t):
        if t.stride(-1) != 1:
            raise ValueError("the last dimension must be contiguous")
        if t.dim() == 3:
            return t.shape[-2], t.shape[-1], t.stride(-2), t.stride(0)
        return t.shape[0], t.shape[1], t.stride(0), 0
    m, k, lda, sa = geo(a)
    n, kb, ldb, sb = geo(b)
    mc, nc, ldc, sc = geo(c)
    if kb != k or mc != m or nc != n:
        raise ValueError(f"shapes do not chain: a {tuple(a.shape)}, b {tuple(b.shape)}, c {tuple(c.shape)}")
    if a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise ValueError("a and b must be bfloat16")
    cd = {torch.bfloat16: MLA_BF16, torch.float32: MLA_F32}.get(c.dtype)
    if cd is None:
        raise ValueError("c must be bfloat16 or float32")
    _check("mla_gemm_bf16", load_library().mla_gemm_bf16(
        batch, m, n, k, _ptr(a), lda, sa, _ptr(b), ldb, sb, _ptr(c), cd, ldc, sc,
        _stream(stream)))


def mla_absorb_weights_workspace_size(dims, d_cq):
    d = dims.c()
    n = ctypes.c_size_t(0)
    _check("mla_absorb_weights_workspace_size", load_library().mla_absorb_weights_workspace_size(
        ctypes.byref(d), int(d_cq), ctypes.byref(n)))
    return int(n.value)


def mla_absorb_query_weights(dims, w_uq, w_uk, w_q_absorbed, workspace, stream=None):
    H, dn, dq = w_uq.shape
    dev = w_uq.device
    _expect("w_uq", w_uq, (dims.n_heads, dims.d_nope, dq), torch.bfloat16, dev)
    _expect("w_uk", w_uk, (dims.n_heads, dims.d_nope, dims.d_latent), torch.bfloat16, dev)
    _expect("w_q_absorbed", w_q_absorbed, (dims.n_heads, dims.d_latent, dq), torch.bfloat16, dev)
    d = dims.c()
    _check("mla_absorb_query_weights", load_library().mla_absorb_query_weights(
        ctypes.byref(d), int(dq), _ptr(w_uq), _ptr(w_uk), _ptr(w_q_absorbed), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_absorb_output_weights(dims, w_o, w_uv, w_o_absorbed, workspace, stream=None):
    dm = w_o.shape[0]
    dev = w_o.device
    _expect("w_o", w_o, (dm, dims.n_heads * dims.d_v), torch.bfloat16, dev)
    _expect("w_uv", w_uv, (dims.n_heads, dims.d_v, dims.d_latent), torch.bfloat16, dev)
    _expect("w_o_absorbed", w_o_absorbed, (dm, dims.n_heads * dims.d_latent), torch.bfloat16, dev)
    d = dims.c()
    _check("mla_absorb_output_weights", load_library().mla_absorb_output_weights(
        ctypes.byref(d), int(dm), _ptr(w_o), _ptr(w_uv), _ptr(w_o_absorbed), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_query_from_latent(dims, c_q, w_q_absorbed, w_qr, seqlens, q_latent, q_pe, stream=None):
    B, S, dq = c_q.shape
    H = dims.n_heads
    dev = c_q.device
    _expect("c_q", c_q, (B, S, dq), torch.bfloat16, dev)
    _expect("w_q_absorbed", w_q_absorbed, (H, dims.d_latent, dq), torch.bfloat16, dev)
    _expect("w_qr", w_qr, (H * dims.d_rope, dq), torch.bfloat16, dev)
    _expect("seqlens", seqlens, (B,), torch.int32, dev)
    _expect("q_latent", q_latent, (B, S, H, dims.d_latent), torch.bfloat16, dev)
    _expect("q_pe", q_pe, (B, S, H, dims.d_rope), torch.bfloat16, dev)
    d = dims.c()
    _check("mla_query_from_latent", load_library().mla_query_from_latent(
        ctypes.byref(d), B, S, int(dq), _ptr(c_q), _ptr(w_q_absorbed), _ptr(w_qr), _ptr(seqlens),
        _ptr(q_latent), _ptr(q_pe), _stream(stream)))
