// C ABI of the MLA paged-decode library: argument checks, workspace layout and
// kernel launches.  Every check runs on the host before anything is enqueued.
#include "mla_decode.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "mla_common.hpp"
#include "mla_internal.hpp"

#define MLA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using mla::AbsorbArgs;
using mla::CombineArgs;
using mla::DecodeArgs;

constexpr int kMaxQLen = 8;
constexpr int kMaxDevices = 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Supported (act, latent) combinations and shapes.
mla_status_t check_dims(const mla_dims_t* d) {
  if (d == nullptr) return MLA_ERR_NULL_POINTER;
  if (d->n_heads < 1 || d->d_latent < 1 || d->d_rope < 0 || d->d_nope < 1 || d->d_v < 1 ||
      d->page_size < 1)
    return MLA_ERR_BAD_SHAPE;
  if (d->d_rope % 2 != 0 || d->d_latent % 8 != 0) return MLA_ERR_BAD_SHAPE;
  if (!(d->softmax_scale > 0.f) || !(d->rope_base > 0.f)) return MLA_ERR_BAD_SHAPE;
  const int act = d->act_dtype, lat = d->latent_dtype;
  if (act < MLA_F32 || act > MLA_FP8_E4M3 || lat < MLA_F32 || lat > MLA_FP8_E4M3)
    return MLA_ERR_BAD_DTYPE;
  if (act == MLA_F32) {
    if (lat != MLA_F32) return MLA_ERR_BAD_DTYPE;
    if (d->page_size != mla::kPage || d->d_latent > 128 || d->d_latent % 16 != 0 ||
        d->d_rope > 32 || d->d_nope > 128 || d->d_v > 128)
      return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
  }
  if (act == MLA_BF16) {
    if (lat != MLA_BF16 && lat != MLA_FP8_E4M3) return MLA_ERR_BAD_DTYPE;
    if (d->page_size != mla::kPage || d->d_latent != 512 || d->d_rope != 64 ||
        d->d_nope != 128 || d->d_v != 128)
      return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
  }
  return MLA_ERR_BAD_DTYPE;  // fp8 activations are not a supported combination
}

mla_status_t check_batch(int32_t batch, int32_t q_len) {
  if (batch < 0) return MLA_ERR_BAD_SHAPE;
  if (q_len < 1 || q_len > kMaxQLen) return MLA_ERR_BAD_SHAPE;
  return MLA_OK;
}


// Compute units of the current device (cached).  This is the first HIP call
// of any entry point and runs only after the argument checks.
mla_status_t device_cus(int* cus) {
  static int cache[kMaxDevices] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      return MLA_ERR_HIP;
    cache[dev] = v;
  }
  *cus = cache[dev];
  return MLA_OK;
}

// Workspace layout for a launch shape, given the device's compute units.
struct Layout {
  int row_groups;
  int num_wg;      // target workgroups G of the split plan
  int grid;        // launched workgroups (>= number of chunks)
  size_t off_o, off_lse, off_units, bytes;
};

Layout layout_for(const mla_dims_t* d, int32_t batch, int32_t q_len, int cus) {
  Layout L;
  L.row_groups = (q_len * d->n_heads + mla::kRowsPerWG - 1) / mla::kRowsPerWG;
  L.num_wg = cus;
  const int64_t units = (int64_t)batch * L.row_groups;
  L.grid = (int)align_up((size_t)(L.num_wg + units), 8);
  const size_t slots = (size_t)L.grid;
  const size_t part_elt = d->act_dtype == MLA_F32 ? 4 : 2;
  const size_t o_bytes = slots * mla::kRowsPerWG * (size_t)d->d_latent * part_elt;
  L.off_o = 0;
  L.off_lse = align_up(o_bytes, 256);
  L.off_units = align_up(L.off_lse + slots * mla::kRowsPerWG * 4, 256);
  L.bytes = align_up(L.off_units + (size_t)units * 2 * 4, 256);
  return L;
}

mla_status_t launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

}  // namespace

MLA_EXPORT const char* mla_status_string(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL_POINTER: return "MLA_ERR_NULL_POINTER: a required pointer is NULL";
    case MLA_ERR_BAD_SHAPE: return "MLA_ERR_BAD_SHAPE: a size or scalar argument is out of range";
    case MLA_ERR_BAD_DTYPE: return "MLA_ERR_BAD_DTYPE: unsupported dtype combination";
    case MLA_ERR_MISALIGNED: return "MLA_ERR_MISALIGNED: a device pointer is not 16-byte aligned";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL: workspace below mla_decode_workspace_size()";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: shape not built into this library";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP runtime call or kernel launch failed";
  }
  return "MLA_ERR_UNKNOWN";
}

MLA_EXPORT mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                     const void* q_nope, const void* q_rope,
                                     const int32_t* seqlens, const void* w_uk, void* q_latent,
                                     float* q_latent_scale, void* q_pe, void* stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_batch(batch, q_len)) != MLA_OK) return st;
  const bool fp8 = dims->latent_dtype == MLA_FP8_E4M3;
  if (!q_nope || !q_rope || !seqlens || !w_uk || !q_latent || !q_pe) return MLA_ERR_NULL_POINTER;
  if (fp8 != (q_latent_scale != nullptr)) return fp8 ? MLA_ERR_NULL_POINTER : MLA_ERR_BAD_DTYPE;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(seqlens) || !aligned16(w_uk) ||
      !aligned16(q_latent) || !aligned16(q_pe) || (fp8 && !aligned16(q_latent_scale)))
    return MLA_ERR_MISALIGNED;
  if (batch == 0) return MLA_OK;
  AbsorbArgs a;
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.seqlens = seqlens;
  a.w_uk = w_uk;
  a.q_lat = q_latent;
  a.q_lat_scale = q_latent_scale;
  a.q_pe = q_pe;
  a.batch = batch;
  a.q_len = q_len;
  a.n_heads = dims->n_heads;
  a.d_nope = dims->d_nope;
  a.d_lat = dims->d_latent;
  a.d_rope = dims->d_rope;
  a.rope_base = dims->rope_base;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dims->act_dtype == MLA_F32) return launch_status(mla::launch_absorb_f32(a, s));
  return launch_status(mla::launch_absorb_bf16(a, fp8, s));
}

MLA_EXPORT mla_status_t mla_decode_workspace_size(const mla_dims_t* dims, int32_t batch,
                                                  int32_t q_len, int32_t max_seqlen,
                                                  size_t* bytes) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_batch(batch, q_len)) != MLA_OK) return st;
  if (bytes == nullptr) return MLA_ERR_NULL_POINTER;
  if (max_seqlen < 0) return MLA_ERR_BAD_SHAPE;
  int cus = 0;
  if ((st = device_cus(&cus)) != MLA_OK) return st;
  *bytes = layout_for(dims, batch, q_len, cus).bytes;
  return MLA_OK;
}

MLA_EXPORT mla_status_t mla_decode_paged(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                         int32_t causal, const void* q_latent,
                                         const float* q_latent_scale, const void* q_pe,
                                         const void* kv_latent, const float* kv_scale,
                                         const void* kv_rope, int32_t num_pages,
                                         const int32_t* block_table, int32_t max_pages_per_seq,
                                         const int32_t* seqlens, int32_t max_seqlen,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_batch(batch, q_len)) != MLA_OK) return st;
  const bool fp8 = dims->latent_dtype == MLA_FP8_E4M3;
  if (!q_latent || !q_pe || !kv_latent || !kv_rope || !block_table || !seqlens || !workspace)
    return MLA_ERR_NULL_POINTER;
  if (fp8 && (!q_latent_scale || !kv_scale)) return MLA_ERR_NULL_POINTER;
  if (!fp8 && (q_latent_scale || kv_scale)) return MLA_ERR_BAD_DTYPE;
  if (num_pages < 1 || max_pages_per_seq < 1 || max_seqlen < 0) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)max_pages_per_seq * dims->page_size < (int64_t)max_seqlen) return MLA_ERR_BAD_SHAPE;
  if (!aligned16(q_latent) || !aligned16(q_pe) || !aligned16(kv_latent) || !aligned16(kv_rope) ||
      !aligned16(block_table) || !aligned16(seqlens) || !aligned16(workspace) ||
      (fp8 && (!aligned16(q_latent_scale) || !aligned16(kv_scale))))
    return MLA_ERR_MISALIGNED;
  int cus = 0;
  if ((st = device_cus(&cus)) != MLA_OK) return st;
  const Layout L = layout_for(dims, batch, q_len, cus);
  if (workspace_bytes < L.bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (batch == 0) return MLA_OK;
  DecodeArgs a;
  a.q_lat = q_latent;
  a.q_scale = q_latent_scale;
  a.q_pe = q_pe;
  a.kv_lat = kv_latent;
  a.kv_scale = kv_scale;
  a.kv_rope = kv_rope;
  a.block_table = block_table;
  a.seqlens = seqlens;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.part_o = ws + L.off_o;
  a.part_lse = reinterpret_cast<float*>(ws + L.off_lse);
  a.unit_chunks = reinterpret_cast<int32_t*>(ws + L.off_units);
  a.max_pages = max_pages_per_seq;
  a.batch = batch;
  a.q_len = q_len;
  a.n_heads = dims->n_heads;
  a.causal = causal != 0;
  a.d_lat = dims->d_latent;
  a.d_rope = dims->d_rope;
  a.num_wg = L.num_wg;
  a.row_groups = L.row_groups;
  a.scale_log2 = dims->softmax_scale * mla::kLog2e;
  (void)num_pages;
  DecodeArgs la = a;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // the launch grid is the chunk-count bound; the kernels read num_wg as G
  hipError_t e;
  if (dims->act_dtype == MLA_F32) {
    e = mla::launch_decode_f32(la, s, L.grid);
  } else if (fp8) {
    e = mla::launch_decode_fp8(la, s, L.grid);
  } else {
    e = mla::launch_decode_bf16(la, s, L.grid);
  }
  return launch_status(e);
}

MLA_EXPORT mla_status_t mla_append_kv(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                      const void* kv_c, const void* k_rope,
                                      const void* norm_weight, float norm_eps,
                                      const int32_t* seqlens, const int32_t* block_table,
                                      int32_t max_pages_per_seq, void* kv_latent,
                                      float* kv_scale, void* kv_rope, int32_t num_pages,
                                      void* stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_batch(batch, q_len)) != MLA_OK) return st;
  const bool fp8 = dims->latent_dtype == MLA_FP8_E4M3;
  if (!kv_c || !k_rope || !norm_weight || !seqlens || !block_table || !kv_latent || !kv_rope)
    return MLA_ERR_NULL_POINTER;
  if (fp8 && !kv_scale) return MLA_ERR_NULL_POINTER;
  if (!fp8 && kv_scale) return MLA_ERR_BAD_DTYPE;
  if (num_pages < 1 || max_pages_per_seq < 1 || !(norm_eps > 0.f)) return MLA_ERR_BAD_SHAPE;
  if (!aligned16(kv_c) || !aligned16(k_rope) || !aligned16(norm_weight) || !aligned16(seqlens) ||
      !aligned16(block_table) || !aligned16(kv_latent) || !aligned16(kv_rope) ||
      (fp8 && !aligned16(kv_scale)))
    return MLA_ERR_MISALIGNED;
  if (batch == 0) return MLA_OK;
  mla::AppendArgs a;
  a.kv_c = kv_c;
  a.k_rope = k_rope;
  a.norm_weight = norm_weight;
  a.seqlens = seqlens;
  a.block_table = block_table;
  a.kv_lat = kv_latent;
  a.kv_scale = kv_scale;
  a.kv_rope = kv_rope;
  a.batch = batch;
  a.q_len = q_len;
  a.d_lat = dims->d_latent;
  a.d_rope = dims->d_rope;
  a.page_size = dims->page_size;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  a.act_dtype = dims->act_dtype;
  a.lat_dtype = dims->latent_dtype;
  a.eps = norm_eps;
  a.rope_base = dims->rope_base;
  return launch_status(mla::launch_append(a, reinterpret_cast<hipStream_t>(stream)));
}

MLA_EXPORT mla_status_t mla_combine(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                    const void* workspace, size_t workspace_bytes,
                                    const int32_t* seqlens, int32_t max_seqlen, const void* w_uv,
                                    void* out, float* lse, void* stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_batch(batch, q_len)) != MLA_OK) return st;
  if (!workspace || !seqlens || !out) return MLA_ERR_NULL_POINTER;
  if (max_seqlen < 0) return MLA_ERR_BAD_SHAPE;
  if (!aligned16(workspace) || !aligned16(seqlens) || !aligned16(out) ||
      (w_uv && !aligned16(w_uv)) || (lse && !aligned16(lse)))
    return MLA_ERR_MISALIGNED;
  int cus = 0;
  if ((st = device_cus(&cus)) != MLA_OK) return st;
  const Layout L = layout_for(dims, batch, q_len, cus);
  if (workspace_bytes < L.bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (batch == 0) return MLA_OK;
  CombineArgs a;
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  a.part_o = ws + L.off_o;
  a.part_lse = reinterpret_cast<const float*>(ws + L.off_lse);
  a.unit_chunks = reinterpret_cast<const int32_t*>(ws + L.off_units);
  a.seqlens = seqlens;
  a.w_uv = w_uv;
  a.out = out;
  a.lse = lse;
  a.batch = batch;
  a.q_len = q_len;
  a.n_heads = dims->n_heads;
  a.d_lat = dims->d_latent;
  a.d_v = dims->d_v;
  a.num_wg = L.num_wg;
  a.row_groups = L.row_groups;
  a.out_dtype = dims->act_dtype;
  return launch_status(mla::launch_combine(a, reinterpret_cast<hipStream_t>(stream)));
}
