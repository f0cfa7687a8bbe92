"""GPU parity of the dense products around the attention (mla_gemm_bf16, the
weight-level absorptions, mla_query_from_latent) against oracle/projections.py,
and a whole decode layer through absorbed weights against the oracle's
unabsorbed chain."""

import numpy as np
import pytest
import torch

import oracle
from head_latent_attention_03_amd import _binding as B
from head_latent_attention_03_amd import inputs
from head_latent_attention_03_amd.runner import DeviceBatch, dims_of
from gpu_helpers import to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bf16(rng, shape, scale=1.0):
    """A seeded bf16 device tensor and its exact fp64 host values."""
    t = (torch.from_numpy(rng.standard_normal(shape).astype(np.float32)) * scale).to(torch.bfloat16)
    return t.to(DEV), t.double().numpy()


def _rel(got, ref):
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


@pytest.mark.parametrize("m,n,k,batch", [(1, 1, 8, 1), (77, 130, 200, 1), (256, 384, 512, 3),
                                         (300, 129, 1032, 2), (1300, 2112, 1032, 2),
                                         (1030, 2000, 520, 3)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_gemm_matches_oracle(m, n, k, batch, out):
    """Ragged sizes (m, n past a 128 tile, k past a 64 chunk), batched operands with
    the first one shared by every batch entry; bf16 and f32 outputs.  The last two
    shapes (at least 512 rows and 128 tiles of 256 x 160) take the wide-tile kernel,
    with m past a 256 tile and n past a 160 tile."""
    rng = np.random.default_rng(m * 7 + n + k)
    a, a64 = _bf16(rng, (m, k), 1 / np.sqrt(k))
    b, b64 = _bf16(rng, (batch, n, k))
    c = torch.empty((batch, m, n), dtype=torch.float32 if out == "f32" else torch.bfloat16,
                    device=DEV)
    B.mla_gemm_bf16(a, b, c)
    torch.cuda.synchronize()
    got = to_f64(c)
    for i in range(batch):
        ref = oracle.down_project(a64, b64[i])
        r = _rel(got[i], ref)
        assert r <= (1e-5 if out == "f32" else 2e-2), (i, r)


def test_gemm_at_the_down_projection_shape():
    """The 4096-token x 7168 -> 2112 latent down-projection that the projection
    bench times (wide-tile kernel), every output against the fp64 product."""
    rng = np.random.default_rng(4096)
    a, a64 = _bf16(rng, (4096, 7168), 0.02)
    b, b64 = _bf16(rng, (1, 2112, 7168), 1 / np.sqrt(7168))
    c = torch.empty((1, 4096, 2112), dtype=torch.bfloat16, device=DEV)
    B.mla_gemm_bf16(a, b, c)
    torch.cuda.synchronize()
    r = _rel(to_f64(c)[0], oracle.down_project(a64, b64[0]))
    assert r <= 2e-2, r


def _dims(H, **kw):
    return dims_of(inputs.workload(2, n_heads=H, **kw))


def test_absorbed_weights_match_oracle():
    """W~ = W_UK^T W_UQ and W~O = W_O W_UV at the DeepSeek-V3 head shape (128 heads,
    128-dim content and value heads, 512-dim latent), d_cq = 1536, d_model = 1024."""
    rng = np.random.default_rng(5)
    dims = _dims(128)
    H, dn, dc, dv, dq, dm = 128, 128, 512, 128, 1536, 1024
    w_uq, w_uq64 = _bf16(rng, (H, dn, dq), 1 / np.sqrt(dq))
    w_uk, w_uk64 = _bf16(rng, (H, dn, dc), 1 / np.sqrt(dc))
    w_uv, w_uv64 = _bf16(rng, (H, dv, dc), 1 / np.sqrt(dc))
    w_o, w_o64 = _bf16(rng, (dm, H * dv), 1 / np.sqrt(H * dv))
    ws = torch.empty(B.mla_absorb_weights_workspace_size(dims, dq), dtype=torch.uint8, device=DEV)
    wq = torch.empty((H, dc, dq), dtype=torch.bfloat16, device=DEV)
    wo = torch.empty((dm, H * dc), dtype=torch.bfloat16, device=DEV)
    B.mla_absorb_query_weights(dims, w_uq, w_uk, wq, ws)
    B.mla_absorb_output_weights(dims, w_o, w_uv, wo, ws)
    torch.cuda.synchronize()
    r1 = _rel(to_f64(wq), oracle.absorb_query_weights(w_uq64, w_uk64))
    r2 = _rel(to_f64(wo), oracle.absorb_output_weights(w_o64, w_uv64))
    print(f"\n[errs] query weights {r1:.3e} output weights {r2:.3e}", flush=True)
    assert r1 <= 2e-2 and r2 <= 2e-2


def _model(rng, H, dm, dq, dc=512, dr=64, dn=128, dv=128):
    w = {}
    w["w_dq"] = _bf16(rng, (dq, dm), 1 / np.sqrt(dm))
    w["w_dkv"] = _bf16(rng, (dc, dm), 1 / np.sqrt(dm))
    w["w_kr"] = _bf16(rng, (dr, dm), 1 / np.sqrt(dm))
    w["w_uq"] = _bf16(rng, (H, dn, dq), 1 / np.sqrt(dq))
    w["w_qr"] = _bf16(rng, (H * dr, dq), 1 / np.sqrt(dq))
    w["w_uk"] = _bf16(rng, (H, dn, dc), 1 / np.sqrt(dc))
    w["w_uv"] = _bf16(rng, (H, dv, dc), 1 / np.sqrt(dc))
    w["w_o"] = _bf16(rng, (dm, H * dv), 1 / np.sqrt(H * dv))
    g = (torch.from_numpy(rng.standard_normal(dc).astype(np.float32)) * 0.1 + 1.0).to(torch.bfloat16)
    w["gain"] = (g.to(DEV), g.double().numpy())
    return w


def test_query_from_latent_matches_oracle():
    """q~ = (W_UK^T W_UQ) c^Q and q_pe = RoPE(W_QR c^Q) at positions L - q_len + j."""
    rng = np.random.default_rng(6)
    H, dq, dm = 128, 1536, 512
    dims = _dims(H)
    w = _model(rng, H, dm, dq)
    Bn, S = 5, 2
    c_q, c_q64 = _bf16(rng, (Bn, S, dq))
    seqlens = torch.tensor([2, 70, 300, 4096, 65535], dtype=torch.int32, device=DEV)
    ws = torch.empty(B.mla_absorb_weights_workspace_size(dims, dq), dtype=torch.uint8, device=DEV)
    wq = torch.empty((H, 512, dq), dtype=torch.bfloat16, device=DEV)
    B.mla_absorb_query_weights(dims, w["w_uq"][0], w["w_uk"][0], wq, ws)
    q_lat = torch.empty((Bn, S, H, 512), dtype=torch.bfloat16, device=DEV)
    q_pe = torch.empty((Bn, S, H, 64), dtype=torch.bfloat16, device=DEV)
    B.mla_query_from_latent(dims, c_q, wq, w["w_qr"][0], seqlens, q_lat, q_pe)
    torch.cuda.synchronize()
    cq = c_q64.reshape(Bn * S, dq)
    q_nope, q_rope = oracle.up_project_query(cq, w["w_uq"][1],
                                             w["w_qr"][1].reshape(H, 64, dq))
    ref_lat = np.einsum("hnc,thn->thc", w["w_uk"][1], q_nope)
    pos = (seqlens.cpu().numpy()[:, None] - S + np.arange(S)[None, :]).reshape(-1)
    ref_pe = oracle.apply_rope(q_rope, pos[:, None], 10000.0)
    r1 = _rel(to_f64(q_lat).reshape(Bn * S, H, 512), ref_lat)
    r2 = _rel(to_f64(q_pe).reshape(Bn * S, H, 64), ref_pe)
    print(f"\n[errs] q_latent {r1:.3e} q_pe {r2:.3e}", flush=True)
    assert r1 <= 2e-2 and r2 <= 2e-2


def test_decode_layer_through_absorbed_weights():
    """Hidden states of the step's new tokens -> c^Q, c^KV, k^R (GEMMs) -> cache append
    (RMSNorm, RoPE) -> query from the absorbed query weights -> paged decode -> merge to
    the latent outputs -> layer output through the absorbed W^O.  Against the oracle's
    unabsorbed chain: the same projections, q^C = W_UQ c^Q, expanded attention
    (K^C = W_UK c, V = W_UV c), y = W_O [o_1; ...; o_H]."""
    rng = np.random.default_rng(7)
    H, dq, dm, S = 16, 384, 1024, 2
    seqlens = [100, 300, 2]
    spec = inputs.workload(2, batch=3, q_len=S, n_heads=H, seqlen=seqlens, init="fan_in")
    wl = inputs.make_workload(spec)
    dims = dims_of(spec)
    w = _model(rng, H, dm, dq)
    h, h64 = _bf16(rng, (3, S, dm))
    # device chain
    db = DeviceBatch.from_workload(wl, DEV)
    T = 3 * S
    hf = h.reshape(T, dm)
    c_q = torch.empty((T, dq), dtype=torch.bfloat16, device=DEV)
    kv_c = torch.empty((T, 512), dtype=torch.bfloat16, device=DEV)
    k_r = torch.empty((T, 64), dtype=torch.bfloat16, device=DEV)
    B.mla_gemm_bf16(hf, w["w_dq"][0], c_q)
    B.mla_gemm_bf16(hf, w["w_dkv"][0], kv_c)
    B.mla_gemm_bf16(hf, w["w_kr"][0], k_r)
    B.mla_append_kv(dims, kv_c.view(3, S, 512), k_r.view(3, S, 64), w["gain"][0], 1e-6,
                    db.seqlens, db.block_table, db.kv_latent, None, db.kv_rope)
    ws = torch.empty(B.mla_absorb_weights_workspace_size(dims, dq), dtype=torch.uint8, device=DEV)
    wq = torch.empty((H, 512, dq), dtype=torch.bfloat16, device=DEV)
    wo = torch.empty((dm, H * 512), dtype=torch.bfloat16, device=DEV)
    B.mla_absorb_query_weights(dims, w["w_uq"][0], w["w_uk"][0], wq, ws)
    B.mla_absorb_output_weights(dims, w["w_o"][0], w["w_uv"][0], wo, ws)
    B.mla_query_from_latent(dims, c_q.view(3, S, dq), wq, w["w_qr"][0], db.seqlens, db.q_latent,
                            db.q_pe)
    db.decode()
    db.combine(with_uv=False)
    y = torch.empty((T, dm), dtype=torch.float32, device=DEV)
    B.mla_gemm_bf16(db.out_latent.reshape(T, H * 512), wo, y)
    torch.cuda.synchronize()
    # oracle chain (fp64, unabsorbed)
    hh = h64.reshape(T, dm)
    cq = oracle.down_project(hh, w["w_dq"][1])
    ckv = oracle.down_project(hh, w["w_dkv"][1]).reshape(3, S, 512)
    kr = oracle.down_project(hh, w["w_kr"][1]).reshape(3, S, 64)
    ap = oracle.append_kv(ckv, kr, w["gain"][1], wl.seqlens, S, wl.block_table, 64, 10000.0)
    inp = oracle.inputs_from_workload(wl)
    for b in range(3):
        for j in range(S):
            if ap["pos"][b, j] >= 0:
                inp["kv_latent"][ap["page"][b, j], ap["slot"][b, j]] = ap["y"][b, j]
                inp["kv_rope"][ap["page"][b, j], ap["slot"][b, j]] = ap["kr"][b, j]
    q_nope, q_rope = oracle.up_project_query(cq, w["w_uq"][1], w["w_qr"][1].reshape(H, 64, dq))
    inp["q_nope"] = q_nope.reshape(3, S, H, 128)
    inp["q_rope"] = q_rope.reshape(3, S, H, 64)
    inp["w_uk"], inp["w_uv"] = w["w_uk"][1], w["w_uv"][1]
    ref = oracle.mla_decode_expanded(inp)
    y_ref = oracle.output_project(ref.out.reshape(T, H * 128), w["w_o"][1])
    r = _rel(to_f64(y), y_ref)
    print(f"\n[errs] layer output {r:.3e}", flush=True)
    assert r <= 2e-2
