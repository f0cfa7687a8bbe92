"""Seeded synthetic inputs for MLA paged decode.

This module only draws random numbers and lays them out in the storage formats
the library reads; it holds none of the attention arithmetic.  Both the GPU
tests/benchmark and the CPU oracle consume exactly the arrays built here.

Storage forms (numpy):
  'f32'  -> float32 values
  'bf16' -> uint16 bit patterns (float32 draws rounded to bf16 by torch's cast)
  'e4m3' -> uint8 OCP e4m3 bit patterns (torch's float8_e4m3fn cast) plus a
            float32 per-token scale

Cache layout (the paged latent cache):
  kv_latent [num_pages, page_size, d_c]   latent c^KV, latent dtype
  kv_scale  [num_pages, page_size]        float32, e4m3 latent only
  kv_rope   [num_pages, page_size, d_R]   decoupled rotary key k^R, activation
                                          dtype, stored already rotated
  block_table [batch, max_pages] int32    logical page -> physical page
  seqlens [batch] int32                   tokens in cache, new tokens included

Poison: pages no sequence uses, table entries past a sequence's last page
(which point at a poison page) and the slots past the last token of each
sequence all hold NaN, so a stray read shows up as NaN in the output.

The five named workloads (``workload(n)``) follow the DeepSeek-V3/V2 attention
shape: 128 heads, 512-dim latent, 64-dim rotary key, 128-dim content query and
value; seeds are 1000 + n.  Every draw happens in a fixed order:
seqlens, block table, latent, (scales), rotary key, q^C, q^R, W_UK, W_UV.
"""

from dataclasses import dataclass, field, replace
import math

import numpy as np
import torch

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)
E4M3_MAX = 448.0


@dataclass
class Spec:
    """Shape, dtype and distribution of one synthetic decode batch."""
    name: str
    batch: int
    q_len: int
    n_heads: int
    d_c: int
    d_rope: int
    d_nope: int
    d_v: int
    page_size: int = 64
    act_dtype: str = "bf16"          # 'f32' or 'bf16'
    latent_dtype: str = "bf16"       # 'f32', 'bf16' or 'e4m3'
    seqlen: object = 4096            # int, ('uniform', lo, hi), ('lognormal_mean', mean, sigma, lo, hi) or a list
    causal: bool = True
    rope_base: float = 10000.0
    softmax_scale: float = None      # default 1/sqrt(d_nope + d_rope)
    init: str = "std"                # 'std': N(0,1)*std ; 'fan_in': N(0,1)/sqrt(dim)
    std: float = 0.02
    latent_std: float = None         # e4m3 latent: N(0,1) clipped at +-448 by default
    identity_table: bool = False
    spare_frac: float = 0.05
    seed: int = 0

    def scale(self):
        if self.softmax_scale is not None:
            return float(self.softmax_scale)
        return 1.0 / math.sqrt(self.d_nope + self.d_rope)


def workload(n, **overrides):
    """The five named workloads; keyword overrides make reduced variants."""
    if n == 1:
        s = Spec("tiny-fp32", batch=1, q_len=1, n_heads=4, d_c=64, d_rope=16,
                 d_nope=32, d_v=32, act_dtype="f32", latent_dtype="f32",
                 seqlen=256, init="fan_in", identity_table=True)
    elif n == 2:
        s = Spec("dsv3-bf16-b64-l4096", batch=64, q_len=1, n_heads=128, d_c=512,
                 d_rope=64, d_nope=128, d_v=128, seqlen=4096)
    elif n == 3:
        s = Spec("dsv3-bf16-long-b16", batch=16, q_len=1, n_heads=128, d_c=512,
                 d_rope=64, d_nope=128, d_v=128, seqlen=("uniform", 16384, 65536))
    elif n == 4:
        s = Spec("dsv3-fp8cache-b64-l4096", batch=64, q_len=1, n_heads=128,
                 d_c=512, d_rope=64, d_nope=128, d_v=128, seqlen=4096,
                 latent_dtype="e4m3", latent_std=1.0)
    elif n == 5:
        s = Spec("dsv3-bf16-mtp2-b128", batch=128, q_len=2, n_heads=128, d_c=512,
                 d_rope=64, d_nope=128, d_v=128,
                 seqlen=("lognormal_mean", 2048.0, 1.0, 2, 32768))
    else:
        raise ValueError(f"no workload {n}")
    s = replace(s, seed=1000 + n)
    return replace(s, **overrides) if overrides else s


def prefill_workload(**overrides):
    """A chunked-prefill batch for the non-absorbed path: 4 sequences of 4096 cached
    tokens whose last 1024 are the chunk being attended (DeepSeek-V3 shapes, bf16,
    N(0,1)*0.02 as the B=64 decode workload); seed 1006."""
    s = Spec("dsv3-bf16-prefill-b4-q1024-l4096", batch=4, q_len=1024, n_heads=128, d_c=512,
             d_rope=64, d_nope=128, d_v=128, seqlen=4096, seed=1006)
    return replace(s, **overrides) if overrides else s


def _f32_to_bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f32_to_e4m3_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _store(x, dtype):
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return _f32_to_bf16_bits(x)
    raise ValueError(dtype)


def _nan_of(dtype):
    return {"f32": np.float32(np.nan), "bf16": BF16_NAN, "e4m3": E4M3_NAN}[dtype]


def draw_seqlens(spec, rng):
    sl = spec.seqlen
    if isinstance(sl, (int, np.integer)):
        return np.full(spec.batch, int(sl), dtype=np.int32)
    if isinstance(sl, (list, tuple, np.ndarray)) and not isinstance(sl[0], str):
        out = np.asarray(sl, dtype=np.int32)
        assert out.shape == (spec.batch,)
        return out
    kind = sl[0]
    if kind == "uniform":                       # integers, both ends inclusive
        return rng.integers(sl[1], sl[2] + 1, size=spec.batch).astype(np.int32)
    if kind == "lognormal_mean":                # arithmetic mean of the lengths = sl[1]
        mean, sigma, lo, hi = sl[1], sl[2], sl[3], sl[4]
        mu = math.log(mean) - 0.5 * sigma * sigma
        x = rng.lognormal(mu, sigma, size=spec.batch)
        return np.clip(np.rint(x), lo, hi).astype(np.int32)
    raise ValueError(f"seqlen spec {sl!r}")


def _normal(rng, shape, spec, fan_in):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if spec.init == "fan_in":
        x *= np.float32(1.0 / math.sqrt(fan_in))
    else:
        x *= np.float32(spec.std)
    return x


@dataclass
class Workload:
    spec: Spec
    seqlens: np.ndarray
    block_table: np.ndarray
    num_pages: int
    poison_page: int
    kv_latent: np.ndarray
    kv_scale: object
    kv_rope: np.ndarray
    q_nope: np.ndarray
    q_rope: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    extra: dict = field(default_factory=dict)

    @property
    def max_seqlen(self):
        return int(self.seqlens.max()) if len(self.seqlens) else 0

    @property
    def tokens(self):
        return int(self.seqlens.astype(np.int64).sum())


def make_workload(spec, seqlens=None):
    """Draw one workload.  ``seqlens`` overrides the spec's length rule."""
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    sl = draw_seqlens(spec, rng) if seqlens is None else np.asarray(seqlens, np.int32)
    page = spec.page_size
    n_pages_seq = (sl.astype(np.int64) + page - 1) // page
    needed = int(n_pages_seq.sum())
    spares = max(1, int(math.ceil(spec.spare_frac * needed)))
    num_pages = needed + spares
    max_pages = max(1, int(n_pages_seq.max()) if len(sl) else 1)

    if spec.identity_table:
        perm = np.arange(num_pages)
    else:
        perm = rng.permutation(num_pages)
    used, spare = perm[:needed], perm[needed:]
    poison = int(spare[0])
    table = np.full((spec.batch, max_pages), poison, dtype=np.int32)
    off = 0
    for b in range(spec.batch):
        k = int(n_pages_seq[b])
        table[b, :k] = used[off:off + k]
        off += k

    # latent c^KV, drawn page by page over the whole pool
    lat_shape = (num_pages, page, spec.d_c)
    kv_scale = None
    if spec.latent_dtype == "e4m3":
        std = 1.0 if spec.latent_std is None else spec.latent_std
        lat = np.empty(lat_shape, dtype=np.uint8)
        kv_scale = np.empty((num_pages, page), dtype=np.float32)
        chunk = 256
        for p0 in range(0, num_pages, chunk):
            x = rng.standard_normal(size=(min(chunk, num_pages - p0), page, spec.d_c),
                                    dtype=np.float32) * np.float32(std)
            x = np.clip(x, -E4M3_MAX, E4M3_MAX)
            amax = np.max(np.abs(x), axis=-1)
            s = np.maximum(amax / np.float32(E4M3_MAX), np.float32(1e-12)).astype(np.float32)
            lat[p0:p0 + len(x)] = _f32_to_e4m3_bits(x / s[..., None])
            kv_scale[p0:p0 + len(x)] = s
    else:
        lat = np.empty(lat_shape, dtype=np.float32 if spec.latent_dtype == "f32" else np.uint16)
        chunk = 256
        for p0 in range(0, num_pages, chunk):
            x = _normal(rng, (min(chunk, num_pages - p0), page, spec.d_c), spec, spec.d_c)
            lat[p0:p0 + len(x)] = _store(x, spec.latent_dtype)
    kv_rope = _store(_normal(rng, (num_pages, page, spec.d_rope), spec, spec.d_rope),
                     spec.act_dtype)

    # poison: spare pages and the tail slots of each sequence's last page
    lat[spare] = _nan_of(spec.latent_dtype)
    kv_rope[spare] = _nan_of(spec.act_dtype)
    if kv_scale is not None:
        kv_scale[spare] = np.float32(np.nan)
    for b in range(spec.batch):
        L = int(sl[b])
        if L % page:
            p = table[b, L // page]
            lat[p, L % page:] = _nan_of(spec.latent_dtype)
            kv_rope[p, L % page:] = _nan_of(spec.act_dtype)
            if kv_scale is not None:
                kv_scale[p, L % page:] = np.float32(np.nan)

    B, S, H = spec.batch, spec.q_len, spec.n_heads
    q_nope = _store(_normal(rng, (B, S, H, spec.d_nope), spec, spec.d_nope), spec.act_dtype)
    q_rope = _store(_normal(rng, (B, S, H, spec.d_rope), spec, spec.d_rope), spec.act_dtype)
    w_uk = _store(_normal(rng, (H, spec.d_nope, spec.d_c), spec, spec.d_c), spec.act_dtype)
    w_uv = _store(_normal(rng, (H, spec.d_v, spec.d_c), spec, spec.d_c), spec.act_dtype)
    return Workload(spec=spec, seqlens=sl, block_table=table, num_pages=num_pages,
                    poison_page=poison, kv_latent=lat, kv_scale=kv_scale,
                    kv_rope=kv_rope, q_nope=q_nope, q_rope=q_rope, w_uk=w_uk,
                    w_uv=w_uv)


def cache_bytes_per_token(spec):
    """Bytes one cached token occupies: latent (+ its scale) plus rotary key."""
    lat = {"f32": 4, "bf16": 2, "e4m3": 1}[spec.latent_dtype] * spec.d_c
    sc = 4 if spec.latent_dtype == "e4m3" else 0
    rope = {"f32": 4, "bf16": 2}[spec.act_dtype] * spec.d_rope
    return lat + sc + rope
