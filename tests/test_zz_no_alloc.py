"""The allocation-free entry point mla_decode_noalloc against the workspace entry
points (mla_decode_paged + mla_combine) on the same inputs: the same kernels on the
same plan, so the outputs must agree bit for bit.  Two calls in a row, the second
on a smaller batch, so the second reads a scratch the first has filled."""

import ctypes

import numpy as np
import pytest
import torch

from head_latent_attention_03_amd import _binding as B
from head_latent_attention_03_amd import inputs
from head_latent_attention_03_amd.runner import DeviceBatch

pytestmark = pytest.mark.gpu


def _both(wl, with_uv):
    db = DeviceBatch.from_workload(wl, "cuda:0")
    db.absorb()
    db.decode()
    db.combine(with_uv=with_uv)
    ref_out = (db.out if with_uv else db.out_latent).clone()
    ref_lse = db.lse.clone()
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    B.mla_decode_noalloc(db.dims, db.q_latent, db.q_latent_scale, db.q_pe, db.kv_latent,
                         db.kv_scale, db.kv_rope, db.block_table, db.seqlens, db.max_seqlen,
                         db.w_uv if with_uv else None, out, lse, causal=db.causal)
    torch.cuda.synchronize()
    return ref_out, ref_lse, out, lse


@pytest.mark.parametrize("cfg", [2, 4])
@pytest.mark.parametrize("with_uv", [True, False])
def test_noalloc_matches_workspace_path_twice(cfg, with_uv):
    big = inputs.make_workload(inputs.workload(cfg, batch=9, q_len=2,
                                               seqlen=[3000, 70, 1, 0, 640, 2048, 129, 5, 900]))
    small = inputs.make_workload(inputs.workload(cfg, batch=3, q_len=1, seqlen=[300, 64, 2]))
    for name, wl in (("big", big), ("small", small)):
        print(f"\\n[case] cfg={cfg} uv={with_uv} {name} lens={list(wl.seqlens)}", flush=True)
        ref_out, ref_lse, out, lse = _both(wl, with_uv)
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                           ref_out.view(torch.int16) if out.dtype == torch.bfloat16 else ref_out)
        assert torch.equal(lse, ref_lse)


def test_noalloc_rejects_a_shape_past_its_scratch():
    """A launch shape whose partials exceed the static scratch is refused on the
    host (nothing is enqueued; the pointers are never dereferenced)."""
    lib = B.load_library()
    d = B.MlaDims(n_heads=128, d_latent=512, d_rope=64, d_nope=128, d_v=128, page_size=64,
                  softmax_scale=192 ** -0.5, rope_base=10000.0).c()
    A = ctypes.c_void_p(0x10000)
    code = lib.mla_decode_noalloc(ctypes.byref(d), 4096, 8, 1, A, None, A, A, None, A, 10, A, 1,
                                  A, 64, None, A, None, None)
    assert code == 8, B.mla_status_string(code)
