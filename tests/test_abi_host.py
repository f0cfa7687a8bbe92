"""The C-ABI library on the host, with no GPU: it loads, it exports every
function include/*.h declares, and its argument checks answer before anything
touches the device (each call here returns from those checks)."""

import ctypes
import glob
import os
import re

import pytest

from head_latent_attention_03_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        names |= set(re.findall(r"^(?:mla_status_t|const char\s*\*)\s*(mla_\w+)\s*\(", text, re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    assert os.path.exists(B.LIBRARY_PATH), (
        f"{B.LIBRARY_PATH} is missing: build it with `python -m head_latent_attention_03_amd.build`")
    return B.load_library()


def test_every_declared_function_is_exported(lib):
    names = _declared()
    assert {"mla_absorb_q", "mla_decode_paged", "mla_combine", "mla_decode_workspace_size",
            "mla_status_string", "mla_append_kv"} <= set(names)
    raw = ctypes.CDLL(B.LIBRARY_PATH)
    missing = [n for n in names if not hasattr(raw, n)]
    assert not missing, missing


def test_status_strings(lib):
    for code, name in enumerate(["MLA_OK", "MLA_ERR_NULL_POINTER", "MLA_ERR_BAD_SHAPE",
                                 "MLA_ERR_BAD_DTYPE", "MLA_ERR_MISALIGNED",
                                 "MLA_ERR_WORKSPACE_TOO_SMALL", "MLA_ERR_UNSUPPORTED",
                                 "MLA_ERR_HIP"]):
        assert B.mla_status_string(code).startswith(name)
    assert B.mla_status_string(99) == "MLA_ERR_UNKNOWN"


def _dims(**kw):
    d = dict(n_heads=128, d_latent=512, d_rope=64, d_nope=128, d_v=128, page_size=64,
             softmax_scale=192 ** -0.5, rope_base=10000.0, act_dtype="bf16", latent_dtype="bf16")
    d.update(kw)
    return B.MlaDims(**d).c()


P = ctypes.c_void_p
NULL = None
A16 = P(0x10000)   # an aligned, never dereferenced address
A8 = P(0x10008)    # misaligned


def test_dims_checks(lib):
    nb = ctypes.c_size_t(0)
    ws = lambda d, b=4, s=1, L=100: lib.mla_decode_workspace_size(
        ctypes.byref(d) if d is not None else None, b, s, L, ctypes.byref(nb))
    assert ws(None) == 1                                          # NULL dims
    assert ws(_dims(n_heads=0)) == 2                              # bad shape
    assert ws(_dims(d_rope=63)) == 2                              # odd rotary width
    assert ws(_dims(softmax_scale=0.0)) == 2
    assert ws(_dims(act_dtype="e4m3")) == 3                       # fp8 activations
    assert ws(_dims(act_dtype="f32", latent_dtype="bf16")) == 3   # mixed f32 / bf16
    assert ws(_dims(d_latent=256)) == 6                           # shape not built
    assert ws(_dims(page_size=32)) == 6
    assert ws(_dims(act_dtype="f32", latent_dtype="f32", d_latent=64, d_rope=16, d_nope=32,
                    d_v=32), s=9) == 2                            # q_len > 8
    assert ws(_dims(), b=-1) == 2
    assert ws(_dims(), L=-1) == 2
    assert lib.mla_decode_workspace_size(ctypes.byref(_dims()), 4, 1, 100, None) == 1


def test_append_argument_checks(lib):
    d = _dims()
    call = lambda **kw: lib.mla_append_kv(
        ctypes.byref(kw.get("dims", d)), kw.get("batch", 2), kw.get("q_len", 1),
        kw.get("kv_c", A16), kw.get("k_rope", A16), kw.get("w", A16), kw.get("eps", 1e-6),
        kw.get("seqlens", A16), kw.get("table", A16), kw.get("max_pages", 4),
        kw.get("lat", A16), kw.get("scale", NULL), kw.get("rope", A16),
        kw.get("pages", 10), NULL)
    assert call(kv_c=NULL) == 1
    assert call(rope=NULL) == 1
    assert call(scale=A16) == 3                                   # scale with a bf16 latent
    assert call(dims=_dims(latent_dtype="e4m3")) == 1             # e4m3 needs the scales
    assert call(eps=0.0) == 2
    assert call(pages=0) == 2
    assert call(q_len=0) == 2
    assert call(kv_c=A8) == 4
    assert call(table=A8) == 4
    assert call(batch=0) == 0                                     # a no-op, nothing launched


def test_decode_and_combine_argument_checks(lib):
    d = _dims()
    dec = lambda **kw: lib.mla_decode_paged(
        ctypes.byref(d), 2, 1, 1, kw.get("q", A16), NULL, A16, A16, NULL, A16, 10, A16,
        kw.get("max_pages", 4), A16, kw.get("max_seqlen", 100), kw.get("ws", A16), 1 << 20, NULL)
    assert dec(q=NULL) == 1
    assert dec(ws=NULL) == 1
    assert dec(max_pages=1) == 2                                  # 1 page cannot hold 100 tokens
    assert dec(q=A8) == 4
    comb = lambda **kw: lib.mla_combine(ctypes.byref(d), 2, 1, kw.get("ws", A16), 1 << 20, A16,
                                        100, NULL, kw.get("out", A16), kw.get("lse", NULL), NULL)
    assert comb(ws=NULL) == 1
    assert comb(out=NULL) == 1
    assert comb(lse=A8) == 4
    absq = lambda **kw: lib.mla_absorb_q(ctypes.byref(d), 2, 1, kw.get("qn", A16), A16, A16, A16,
                                         A16, kw.get("qs", NULL), A16, NULL)
    assert absq(qn=NULL) == 1
    assert absq(qs=A16) == 3                                      # scale with a bf16 latent
    assert absq(qn=A8) == 4


def test_validate_paged_host_finds_each_broken_precondition(lib):
    """mla_validate_paged_host (the check MLA_VALIDATE=1 runs on the device before
    a decode): each sequence below breaks one precondition, or none; table entries
    past a sequence's used pages are never read and may hold anything."""
    import numpy as np
    d = B.MlaDims(n_heads=128, d_latent=512, d_rope=64, d_nope=128, d_v=128, page_size=64,
                  softmax_scale=192 ** -0.5, rope_base=10000.0)
    num_pages, max_pages, max_seqlen = 10, 4, 256
    good_t = np.array([[3, 1, -7, 99], [0, 9, 2, 5], [4, -1, -1, -1]], dtype=np.int32)
    good_l = np.array([65, 256, 0], dtype=np.int32)       # pages used: 2, 4, 0
    assert B.mla_validate_paged_host(d, num_pages, good_t, good_l, max_seqlen) == (0, 0)
    cases = [
        ([[3, 10, 0, 0]], [65]),       # a used page past the pool
        ([[3, -1, 0, 0]], [100]),      # a negative used page
        ([[3, 1, 0, 0]], [257]),       # longer than max_seqlen
        ([[3, 1, 0, 0]], [-1]),        # a negative length
    ]
    for t, l in cases:
        code, bad = B.mla_validate_paged_host(d, num_pages, np.array(t, np.int32),
                                              np.array(l, np.int32), max_seqlen)
        assert (code, bad) == (2, 1), (t, l, code, bad)
    # several at once: the count is the number of failing sequences
    t = np.array([[0, 0, 0, 0], [11, 0, 0, 0], [0, 0, 0, 12]], dtype=np.int32)
    code, bad = B.mla_validate_paged_host(d, num_pages, t, np.array([256, 1, 193], np.int32),
                                          max_seqlen)
    assert (code, bad) == (2, 2)
    # a table too narrow for max_seqlen is an argument error
    code, _ = B.mla_validate_paged_host(d, num_pages, good_t[:, :3], good_l, max_seqlen)
    assert code == 2



def test_prefill_argument_checks(lib):
    """mla_prefill_paged answers from the host checks (bf16 only; q_len up to 65536;
    table wide enough for max_seqlen; workspace size) before any device call."""
    d = _dims()
    nb = ctypes.c_size_t(0)
    assert lib.mla_prefill_workspace_size(ctypes.byref(d), 2, 100, ctypes.byref(nb)) == 0
    # K^C and V rows, padded to whole pages: 2 x B x H x 128 x 128 x 2 bytes
    assert nb.value == 2 * 2 * 128 * 128 * 128 * 2
    assert lib.mla_prefill_workspace_size(ctypes.byref(_dims(latent_dtype="e4m3")), 2, 100,
                                          ctypes.byref(nb)) == 6
    call = lambda **kw: lib.mla_prefill_paged(
        ctypes.byref(kw.get("dims", d)), 2, kw.get("q_len", 100), kw.get("qn", A16), A16, A16,
        A16, 10, A16, kw.get("max_pages", 4), A16, kw.get("max_seqlen", 100), A16, A16,
        kw.get("ws", A16), kw.get("ws_bytes", 1 << 30), kw.get("out", A16), NULL, NULL)
    assert call(qn=NULL) == 1
    assert call(out=NULL) == 1
    assert call(ws=NULL) == 1
    assert call(q_len=0) == 2 and call(q_len=65537) == 2
    assert call(max_pages=1) == 2
    assert call(qn=A8) == 4
    assert call(ws_bytes=1024) == 5
    assert call(dims=_dims(act_dtype="f32", latent_dtype="f32", d_latent=64, d_rope=16,
                           d_nope=32, d_v=32)) == 6


def test_gemm_and_weight_absorption_argument_checks(lib):
    g = lambda **kw: lib.mla_gemm_bf16(
        kw.get("batch", 1), kw.get("m", 16), kw.get("n", 16), kw.get("k", 64), kw.get("a", A16),
        kw.get("lda", 64), 0, A16, kw.get("ldb", 64), 0, kw.get("c", A16), kw.get("cd", 1),
        kw.get("ldc", 16), 0, NULL)
    assert g(k=12) == 2                                            # k not a multiple of 8
    assert g(lda=32) == 2                                          # lda < k
    assert g(ldc=8) == 2                                           # ldc < n
    assert g(cd=2) == 3                                            # fp8 output
    assert g(a=NULL) == 1
    assert g(a=A8) == 4
    assert g(m=0) == 0 and g(batch=0) == 0                         # empty: nothing launched
    assert g(batch=70000) == 2
    d = _dims()
    nb = ctypes.c_size_t(0)
    assert lib.mla_absorb_weights_workspace_size(ctypes.byref(d), 1536, ctypes.byref(nb)) == 0
    assert nb.value >= 128 * 128 * (512 + 1536) * 2
    assert lib.mla_absorb_weights_workspace_size(ctypes.byref(d), 100, ctypes.byref(nb)) == 2
    aq = lambda **kw: lib.mla_absorb_query_weights(
        ctypes.byref(d), 1536, kw.get("uq", A16), A16, A16, kw.get("ws", A16),
        kw.get("ws_bytes", 1 << 30), NULL)
    assert aq(uq=NULL) == 1
    assert aq(ws_bytes=16) == 5
    ao = lambda **kw: lib.mla_absorb_output_weights(
        ctypes.byref(d), kw.get("dm", 1024), A16, A16, A16, A16, kw.get("ws_bytes", 1 << 30), NULL)
    assert ao(dm=0) == 2
    assert ao(ws_bytes=16) == 5
    qf = lambda **kw: lib.mla_query_from_latent(
        ctypes.byref(kw.get("dims", d)), 2, kw.get("q_len", 1), 1536, A16, A16, A16, A16,
        kw.get("ql", A16), A16, NULL)
    assert qf(ql=NULL) == 1
    assert qf(q_len=9) == 2
    assert qf(dims=_dims(latent_dtype="e4m3")) == 6


def test_streaming_view_argument_checks(lib):
    """mla_streaming_view answers bad counts and null pointers from the host (no device
    call): sink_pages >= 0, window_pages >= 1, max_pages_out >= sink + window + 1."""
    d = _dims()
    call = lambda **kw: lib.mla_streaming_view(
        ctypes.byref(d), kw.get("batch", 2), kw.get("sl", A16), A16, kw.get("max_pages", 8),
        kw.get("sink", 1), kw.get("window", 4), kw.get("osl", A16), kw.get("obt", A16),
        kw.get("cols", 6), NULL)
    assert call(sl=NULL) == 1 and call(osl=NULL) == 1 and call(obt=NULL) == 1
    assert call(sink=-1) == 2 and call(window=0) == 2
    assert call(cols=5) == 2 and call(max_pages=0) == 2 and call(batch=-1) == 2
    assert call(batch=0) == 0
