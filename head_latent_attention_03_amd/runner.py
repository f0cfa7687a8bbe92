"""Device-side buffers for one decode batch, and the three-call decode step.

Uploads a generated workload (storage-form numpy arrays) into torch device
tensors of the library's dtypes, allocates outputs and the workspace once, and
runs mla_absorb_q -> mla_decode_paged -> mla_combine on the current stream.
"""

from dataclasses import dataclass

import numpy as np
import torch

from . import _binding as B


def _to_device(arr, dtype, device):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    elif dtype == "e4m3":
        t = torch.from_numpy(np.ascontiguousarray(arr)).view(torch.float8_e4m3fn)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    elif dtype == "i32":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32))
    else:
        raise ValueError(dtype)
    return t.to(device)


def dims_of(spec):
    return B.MlaDims(n_heads=spec.n_heads, d_latent=spec.d_c, d_rope=spec.d_rope,
                     d_nope=spec.d_nope, d_v=spec.d_v, page_size=spec.page_size,
                     softmax_scale=spec.scale(), rope_base=spec.rope_base,
                     act_dtype=spec.act_dtype, latent_dtype=spec.latent_dtype)


@dataclass
class DeviceBatch:
    dims: B.MlaDims
    batch: int
    q_len: int
    causal: bool
    max_seqlen: int
    q_nope: torch.Tensor
    q_rope: torch.Tensor
    w_uk: torch.Tensor
    w_uv: torch.Tensor
    kv_latent: torch.Tensor
    kv_scale: object
    kv_rope: torch.Tensor
    block_table: torch.Tensor
    seqlens: torch.Tensor
    q_latent: torch.Tensor
    q_latent_scale: object
    q_pe: torch.Tensor
    workspace: torch.Tensor
    out: torch.Tensor
    out_latent: torch.Tensor
    lse: torch.Tensor

    @classmethod
    def from_workload(cls, wl, device="cuda:0"):
        s = wl.spec
        dims = dims_of(s)
        dev = torch.device(device)
        Bn, S, H = s.batch, s.q_len, s.n_heads
        act = dims.act_torch
        fp8 = s.latent_dtype == "e4m3"
        q_lat_dt = torch.float8_e4m3fn if fp8 else act
        ws_bytes = B.mla_decode_workspace_size(dims, Bn, S, wl.max_seqlen)
        return cls(
            dims=dims, batch=Bn, q_len=S, causal=s.causal, max_seqlen=wl.max_seqlen,
            q_nope=_to_device(wl.q_nope, s.act_dtype, dev),
            q_rope=_to_device(wl.q_rope, s.act_dtype, dev),
            w_uk=_to_device(wl.w_uk, s.act_dtype, dev),
            w_uv=_to_device(wl.w_uv, s.act_dtype, dev),
            kv_latent=_to_device(wl.kv_latent, s.latent_dtype, dev),
            kv_scale=_to_device(wl.kv_scale, "f32", dev) if fp8 else None,
            kv_rope=_to_device(wl.kv_rope, s.act_dtype, dev),
            block_table=_to_device(wl.block_table, "i32", dev),
            seqlens=_to_device(wl.seqlens, "i32", dev),
            q_latent=torch.empty((Bn, S, H, s.d_c), dtype=q_lat_dt, device=dev),
            q_latent_scale=torch.empty((Bn, S, H), dtype=torch.float32, device=dev) if fp8 else None,
            q_pe=torch.empty((Bn, S, H, s.d_rope), dtype=act, device=dev),
            workspace=torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev),
            out=torch.empty((Bn, S, H, s.d_v), dtype=act, device=dev),
            out_latent=torch.empty((Bn, S, H, s.d_c), dtype=act, device=dev),
            lse=torch.empty((Bn, S, H), dtype=torch.float32, device=dev),
        )

    # -- the three calls -------------------------------------------------------
    def absorb(self, stream=None):
        B.mla_absorb_q(self.dims, self.q_nope, self.q_rope, self.seqlens, self.w_uk,
                       self.q_latent, self.q_latent_scale, self.q_pe, stream=stream)

    def decode(self, kv_latent=None, kv_scale=None, kv_rope=None, block_table=None,
               stream=None, seqlens=None, max_seqlen=None):
        B.mla_decode_paged(self.dims, self.q_latent, self.q_latent_scale, self.q_pe,
                           self.kv_latent if kv_latent is None else kv_latent,
                           self.kv_scale if kv_scale is None else kv_scale,
                           self.kv_rope if kv_rope is None else kv_rope,
                           self.block_table if block_table is None else block_table,
                           self.seqlens if seqlens is None else seqlens,
                           self.max_seqlen if max_seqlen is None else max_seqlen,
                           self.workspace, causal=self.causal, stream=stream)

    def combine(self, with_uv=True, stream=None, seqlens=None, max_seqlen=None):
        sl = self.seqlens if seqlens is None else seqlens
        ms = self.max_seqlen if max_seqlen is None else max_seqlen
        if with_uv:
            B.mla_combine(self.dims, self.workspace, sl, ms, self.w_uv,
                          self.out, self.lse, q_len=self.q_len, stream=stream)
        else:
            B.mla_combine(self.dims, self.workspace, sl, ms, None,
                          self.out_latent, self.lse, q_len=self.q_len, stream=stream)

    def streaming_view(self, sink_pages, window_pages, stream=None):
        """The eviction view of this batch's cache (mla_streaming_view): returns
        (seqlens, block_table, max_seqlen) to pass to decode() and combine(); the
        absorb keeps the true lengths."""
        cols = sink_pages + window_pages + 1
        sl = torch.empty_like(self.seqlens)
        bt = torch.empty((self.batch, cols), dtype=torch.int32, device=self.seqlens.device)
        B.mla_streaming_view(self.dims, self.seqlens, self.block_table, sink_pages, window_pages,
                             sl, bt, stream=stream)
        return sl, bt, min(self.max_seqlen, cols * self.dims.page_size)

    def step(self, with_uv=True, stream=None):
        """One decode step: absorb, paged split-KV attention, combine."""
        self.absorb(stream)
        self.decode(stream=stream)
        self.combine(with_uv=with_uv, stream=stream)


def prefill_step(wl, device="cuda:0", stream=None):
    """Upload a workload and run mla_prefill_paged on it (the non-absorbed form):
    returns (out [B, q_len, H, d_v], lse [B, q_len, H]) on the device."""
    s = wl.spec
    dims = dims_of(s)
    dev = torch.device(device)
    Bn, S, H = s.batch, s.q_len, s.n_heads
    act = dims.act_torch
    t = dict(
        q_nope=_to_device(wl.q_nope, s.act_dtype, dev),
        q_rope=_to_device(wl.q_rope, s.act_dtype, dev),
        kv_latent=_to_device(wl.kv_latent, s.latent_dtype, dev),
        kv_rope=_to_device(wl.kv_rope, s.act_dtype, dev),
        block_table=_to_device(wl.block_table, "i32", dev),
        seqlens=_to_device(wl.seqlens, "i32", dev),
        w_uk=_to_device(wl.w_uk, s.act_dtype, dev),
        w_uv=_to_device(wl.w_uv, s.act_dtype, dev),
    )
    ws = torch.empty(max(B.mla_prefill_workspace_size(dims, Bn, wl.max_seqlen), 16),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((Bn, S, H, s.d_v), dtype=act, device=dev)
    lse = torch.empty((Bn, S, H), dtype=torch.float32, device=dev)
    B.mla_prefill_paged(dims, t["q_nope"], t["q_rope"], t["kv_latent"], t["kv_rope"],
                        t["block_table"], t["seqlens"], wl.max_seqlen, t["w_uk"], t["w_uv"], ws,
                        out, lse, stream=stream)
    return out, lse
