// C ABI of the MLA paged-decode library: argument checks, workspace layout and
// kernel launches.  Every check runs on the host before anything is enqueued.
#include "mla_decode.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "mla_common.hpp"
#include "mla_internal.hpp"
#include "mla_validate.hpp"

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
  size_t off_o, off_lse, off_units, off_flag, bytes;
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
  L.off_flag = align_up(L.off_units + (size_t)units * 2 * 4, 256);   // MLA_VALIDATE result
  L.bytes = L.off_flag + 256;
  return L;
}

mla_status_t launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Device scratch of mla_decode_noalloc, in place of a caller workspace: the
// split partials, their log-sum-exps and the unit table of one decode.  Each
// device holds its own copy for the life of the process.  Its device address
// comes from hipGetSymbolAddress, once per device; host code never uses the
// array's own name as an address.
constexpr size_t kScratchBytes = (size_t)80 << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The current device's scratch address (looked up on the first call there).
mla_status_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MLA_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MLA_OK;
}

// MLA_VALIDATE=1 in the environment (read on every call) turns on the device
// check of the decode's preconditions.
bool validation_on() {
  const char* v = std::getenv("MLA_VALIDATE");
  return v != nullptr && v[0] == '1' && v[1] == '\0';
}

// Runs the precondition check on the device, waits for it, and returns
// MLA_ERR_BAD_SHAPE if any sequence breaks one.
mla_status_t validate_on_device(const mla_dims_t* d, int32_t batch, int32_t num_pages,
                                const int32_t* block_table, int32_t max_pages,
                                const int32_t* seqlens, int32_t max_seqlen, int32_t* flag,
                                hipStream_t s) {
  mla::ValidateArgs v;
  v.block_table = block_table;
  v.seqlens = seqlens;
  v.bad = flag;
  v.batch = batch;
  v.max_pages = max_pages;
  v.max_seqlen = max_seqlen;
  v.page_size = d->page_size;
  v.num_pages = num_pages;
  if (mla::launch_validate(v, s) != hipSuccess) return MLA_ERR_HIP;
  int32_t bad = -1;
  if (hipMemcpyAsync(&bad, flag, sizeof(bad), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MLA_ERR_HIP;
  return bad == 0 ? MLA_OK : MLA_ERR_BAD_SHAPE;
}

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
    case MLA_ERR_SCRATCH_TOO_SMALL:
      return "MLA_ERR_SCRATCH_TOO_SMALL: the launch needs more than mla_decode_noalloc's "
             "static scratch (MLA_NOALLOC_SCRATCH_BYTES); use mla_decode_paged with a workspace";
  }
  return "MLA_ERR_UNKNOWN";
}

MLA_EXPORT mla_status_t mla_validate_paged_host(const mla_dims_t* dims, int32_t batch,
                                                int32_t num_pages, const int32_t* block_table,
                                                int32_t max_pages_per_seq,
                                                const int32_t* seqlens, int32_t max_seqlen,
                                                int32_t* bad) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (bad == nullptr || seqlens == nullptr || block_table == nullptr) return MLA_ERR_NULL_POINTER;
  if (batch < 0 || num_pages < 1 || max_pages_per_seq < 1 || max_seqlen < 0)
    return MLA_ERR_BAD_SHAPE;
  if ((int64_t)max_pages_per_seq * dims->page_size < (int64_t)max_seqlen) return MLA_ERR_BAD_SHAPE;
  int32_t n = 0;
  for (int32_t b = 0; b < batch; ++b)
    n += mla::sequence_ok(block_table + (int64_t)b * max_pages_per_seq, seqlens[b], max_seqlen,
                          max_pages_per_seq, dims->page_size, num_pages) ? 0 : 1;
  *bad = n;
  return n == 0 ? MLA_OK : MLA_ERR_BAD_SHAPE;
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
  DecodeArgs la = a;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (validation_on()) {
    st = validate_on_device(dims, batch, num_pages, block_table, max_pages_per_seq, seqlens,
                            max_seqlen, reinterpret_cast<int32_t*>(ws + L.off_flag), s);
    if (st != MLA_OK) return st;
  }
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

MLA_EXPORT mla_status_t mla_streaming_view(const mla_dims_t* dims, int32_t batch,
                                           const int32_t* seqlens, const int32_t* block_table,
                                           int32_t max_pages_per_seq, int32_t sink_pages,
                                           int32_t window_pages, int32_t* out_seqlens,
                                           int32_t* out_block_table, int32_t max_pages_out,
                                           void* stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || max_pages_per_seq < 1 || sink_pages < 0 || window_pages < 1 ||
      max_pages_out < sink_pages + window_pages + 1)
    return MLA_ERR_BAD_SHAPE;
  if (!seqlens || !block_table || !out_seqlens || !out_block_table) return MLA_ERR_NULL_POINTER;
  if (batch == 0) return MLA_OK;
  mla::StreamingViewArgs a;
  a.seqlens = seqlens;
  a.block_table = block_table;
  a.out_seqlens = out_seqlens;
  a.out_block_table = out_block_table;
  a.batch = batch;
  a.max_pages = max_pages_per_seq;
  a.max_pages_out = max_pages_out;
  a.page_size = dims->page_size;
  a.sink_pages = sink_pages;
  a.window_pages = window_pages;
  return launch_status(mla::launch_streaming_view(a, reinterpret_cast<hipStream_t>(stream)));
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

MLA_EXPORT mla_status_t mla_decode_noalloc(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                           int32_t causal, const void* q_latent,
                                           const float* q_latent_scale, const void* q_pe,
                                           const void* kv_latent, const float* kv_scale,
                                           const void* kv_rope, int32_t num_pages,
                                           const int32_t* block_table,
                                           int32_t max_pages_per_seq, const int32_t* seqlens,
                                           int32_t max_seqlen, const void* w_uv, void* out,
                                           float* lse, void* stream) {
  static_assert(kScratchBytes == (size_t)MLA_NOALLOC_SCRATCH_BYTES, "header and library agree");
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_batch(batch, q_len)) != MLA_OK) return st;
  if (!out) return MLA_ERR_NULL_POINTER;
  int cus = 0;
  if ((st = device_cus(&cus)) != MLA_OK) return st;
  const Layout L = layout_for(dims, batch, q_len, cus);
  if (L.bytes > kScratchBytes) return MLA_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MLA_OK) return st;
  // the same two calls a caller makes with a workspace, on the scratch: the
  // decode writes every partial, log-sum-exp and unit-table entry the merge
  // reads, so nothing in the scratch needs clearing between calls
  st = mla_decode_paged(dims, batch, q_len, causal, q_latent, q_latent_scale, q_pe, kv_latent,
                        kv_scale, kv_rope, num_pages, block_table, max_pages_per_seq, seqlens,
                        max_seqlen, ws, kScratchBytes, stream);
  if (st != MLA_OK) return st;
  return mla_combine(dims, batch, q_len, ws, kScratchBytes, seqlens, max_seqlen, w_uv, out, lse,
                     stream);
}

namespace {
constexpr int kMaxPrefillQ = 1 << 16;

// K^C and V rows of every sequence, padded to whole pages
size_t prefill_bytes(const mla_dims_t* d, int32_t batch, int32_t max_seqlen, int32_t* lpad) {
  const int32_t lp = (max_seqlen + mla::kPage - 1) / mla::kPage * mla::kPage;
  if (lpad) *lpad = lp;
  return align_up(2 * (size_t)batch * d->n_heads * lp * 128 * 2, 256);
}

mla_status_t check_prefill_dims(const mla_dims_t* d) {
  mla_status_t st = check_dims(d);
  if (st != MLA_OK) return st;
  if (d->act_dtype != MLA_BF16 || d->latent_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}
}  // namespace

MLA_EXPORT mla_status_t mla_prefill_workspace_size(const mla_dims_t* dims, int32_t batch,
                                                   int32_t max_seqlen, size_t* bytes) {
  mla_status_t st = check_prefill_dims(dims);
  if (st != MLA_OK) return st;
  if (bytes == nullptr) return MLA_ERR_NULL_POINTER;
  if (batch < 0 || max_seqlen < 0) return MLA_ERR_BAD_SHAPE;
  *bytes = prefill_bytes(dims, batch, max_seqlen, nullptr);
  return MLA_OK;
}

MLA_EXPORT mla_status_t mla_prefill_paged(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                          const void* q_nope, const void* q_rope,
                                          const void* kv_latent, const void* kv_rope,
                                          int32_t num_pages, const int32_t* block_table,
                                          int32_t max_pages_per_seq, const int32_t* seqlens,
                                          int32_t max_seqlen, const void* w_uk, const void* w_uv,
                                          void* workspace, size_t workspace_bytes, void* out,
                                          float* lse, void* stream) {
  mla_status_t st = check_prefill_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || q_len < 1 || q_len > kMaxPrefillQ) return MLA_ERR_BAD_SHAPE;
  if (!q_nope || !q_rope || !kv_latent || !kv_rope || !block_table || !seqlens || !w_uk ||
      !w_uv || !workspace || !out)
    return MLA_ERR_NULL_POINTER;
  if (num_pages < 1 || max_pages_per_seq < 1 || max_seqlen < 0) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)max_pages_per_seq * dims->page_size < (int64_t)max_seqlen) return MLA_ERR_BAD_SHAPE;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(kv_latent) || !aligned16(kv_rope) ||
      !aligned16(block_table) || !aligned16(seqlens) || !aligned16(w_uk) || !aligned16(w_uv) ||
      !aligned16(workspace) || !aligned16(out) || (lse && !aligned16(lse)))
    return MLA_ERR_MISALIGNED;
  int32_t lpad = 0;
  const size_t need = prefill_bytes(dims, batch, max_seqlen, &lpad);
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (batch == 0 || max_seqlen == 0) return MLA_OK;
  mla::PrefillArgs a;
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.kv_lat = kv_latent;
  a.kv_rope = kv_rope;
  a.block_table = block_table;
  a.seqlens = seqlens;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.kexp = ws;
  a.vexp = ws + (size_t)batch * dims->n_heads * lpad * 128 * 2;
  a.out = out;
  a.lse = lse;
  a.batch = batch;
  a.q_len = q_len;
  a.n_heads = dims->n_heads;
  a.max_pages = max_pages_per_seq;
  a.lpad = lpad;
  a.scale_log2 = dims->softmax_scale * mla::kLog2e;
  a.rope_base = dims->rope_base;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (validation_on()) {
    // (the flag goes in the output's first word, rewritten by the kernels)
    st = validate_on_device(dims, batch, num_pages, block_table, max_pages_per_seq, seqlens,
                            max_seqlen, reinterpret_cast<int32_t*>(workspace), s);
    if (st != MLA_OK) return st;
  }
  return launch_status(mla::launch_prefill(a, s));
}

namespace {
bool fits_i32(int64_t v) { return v >= 0 && v <= INT32_MAX; }

mla_status_t gemm(int32_t batch, int32_t m, int32_t n, int32_t k, const void* a, int64_t lda,
                  int64_t sa, const void* b, int64_t ldb, int64_t sb, void* c, int32_t c_f32,
                  int64_t ldc, int64_t sc, hipStream_t s) {
  mla::GemmArgs g;
  g.a = a; g.b = b; g.c = c;
  g.lda = lda; g.ldb = ldb; g.ldc = ldc;
  g.stride_a = sa; g.stride_b = sb; g.stride_c = sc;
  g.batch = batch; g.m = m; g.n = n; g.k = k; g.c_f32 = c_f32;
  return launch_status(mla::launch_gemm_nt(g, s));
}

mla_status_t transpose(int32_t batch, int32_t rows, int32_t cols, const void* src, void* dst,
                       hipStream_t s) {
  mla::TransposeArgs t;
  t.src = src; t.dst = dst; t.batch = batch; t.rows = rows; t.cols = cols;
  return launch_status(mla::launch_transpose(t, s));
}

mla_status_t check_bf16_dims(const mla_dims_t* d) {
  mla_status_t st = check_dims(d);
  if (st != MLA_OK) return st;
  return d->act_dtype == MLA_BF16 ? MLA_OK : MLA_ERR_UNSUPPORTED;
}
}  // namespace

MLA_EXPORT mla_status_t mla_gemm_bf16(int32_t batch, int32_t m, int32_t n, int32_t k,
                                      const void* a, int64_t lda, int64_t stride_a,
                                      const void* b, int64_t ldb, int64_t stride_b, void* c,
                                      int32_t c_dtype, int64_t ldc, int64_t stride_c,
                                      void* stream) {
  if (batch < 0 || m < 0 || n < 0 || k < 0 || k % 8 != 0) return MLA_ERR_BAD_SHAPE;
  if (batch > 65535) return MLA_ERR_BAD_SHAPE;
  if (c_dtype != MLA_F32 && c_dtype != MLA_BF16) return MLA_ERR_BAD_DTYPE;
  if (batch == 0 || m == 0 || n == 0) return MLA_OK;
  if (!a || !b || !c) return MLA_ERR_NULL_POINTER;
  if (lda < k || ldb < k || ldc < n || lda % 8 != 0 || ldb % 8 != 0) return MLA_ERR_BAD_SHAPE;
  if (stride_a < 0 || stride_b < 0 || stride_c < 0) return MLA_ERR_BAD_SHAPE;
  if (!aligned16(a) || !aligned16(b) || ((uintptr_t)c & 3u) != 0) return MLA_ERR_MISALIGNED;
  return gemm(batch, m, n, k, a, lda, stride_a, b, ldb, stride_b, c, c_dtype == MLA_F32, ldc,
              stride_c, reinterpret_cast<hipStream_t>(stream));
}

MLA_EXPORT mla_status_t mla_absorb_weights_workspace_size(const mla_dims_t* dims, int32_t d_cq,
                                                          size_t* bytes) {
  mla_status_t st = check_bf16_dims(dims);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_NULL_POINTER;
  if (d_cq < 8 || d_cq % 8 != 0) return MLA_ERR_BAD_SHAPE;
  const size_t H = (size_t)dims->n_heads;
  const size_t q = align_up(H * dims->d_nope * (dims->d_latent + (size_t)d_cq) * 2, 256);
  const size_t o = align_up(H * dims->d_v * (size_t)dims->d_latent * 2, 256);
  *bytes = q > o ? q : o;
  return MLA_OK;
}

MLA_EXPORT mla_status_t mla_absorb_query_weights(const mla_dims_t* dims, int32_t d_cq,
                                                 const void* w_uq, const void* w_uk,
                                                 void* w_q_absorbed, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  size_t need = 0;
  mla_status_t st = mla_absorb_weights_workspace_size(dims, d_cq, &need);
  if (st != MLA_OK) return st;
  if (!w_uq || !w_uk || !w_q_absorbed || !workspace) return MLA_ERR_NULL_POINTER;
  if (!aligned16(w_uq) || !aligned16(w_uk) || !aligned16(w_q_absorbed) || !aligned16(workspace))
    return MLA_ERR_MISALIGNED;
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (dims->d_nope % 8 != 0) return MLA_ERR_UNSUPPORTED;
  const int H = dims->n_heads, dn = dims->d_nope, dc = dims->d_latent;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  void* uk_t = ws;                                        // [H, d_c, d_nope]
  void* uq_t = ws + (size_t)H * dc * dn * 2;              // [H, d_cq, d_nope]
  if ((st = transpose(H, dn, dc, w_uk, uk_t, s)) != MLA_OK) return st;
  if ((st = transpose(H, dn, d_cq, w_uq, uq_t, s)) != MLA_OK) return st;
  // W~_h[c, q] = sum_n W_UK_h^T[c, n] W_UQ_h^T[q, n]
  return gemm(H, dc, d_cq, dn, uk_t, dn, (int64_t)dc * dn, uq_t, dn, (int64_t)d_cq * dn,
              w_q_absorbed, 0, d_cq, (int64_t)dc * d_cq, s);
}

MLA_EXPORT mla_status_t mla_absorb_output_weights(const mla_dims_t* dims, int32_t d_model,
                                                  const void* w_o, const void* w_uv,
                                                  void* w_o_absorbed, void* workspace,
                                                  size_t workspace_bytes, void* stream) {
  size_t need = 0;
  mla_status_t st = mla_absorb_weights_workspace_size(dims, 8, &need);
  if (st != MLA_OK) return st;
  if (d_model < 1) return MLA_ERR_BAD_SHAPE;
  if (!w_o || !w_uv || !w_o_absorbed || !workspace) return MLA_ERR_NULL_POINTER;
  if (!aligned16(w_o) || !aligned16(w_uv) || !aligned16(w_o_absorbed) || !aligned16(workspace))
    return MLA_ERR_MISALIGNED;
  const int H = dims->n_heads, dv = dims->d_v, dc = dims->d_latent;
  if (dv % 8 != 0) return MLA_ERR_UNSUPPORTED;
  if (workspace_bytes < align_up((size_t)H * dv * dc * 2, 256)) return MLA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* uv_t = workspace;                                 // [H, d_c, d_v]
  if ((st = transpose(H, dv, dc, w_uv, uv_t, s)) != MLA_OK) return st;
  // W~O[m, h d_c + c] = sum_v W_O[m, h d_v + v] W_UV_h^T[c, v]
  return gemm(H, d_model, dc, dv, w_o, (int64_t)H * dv, dv, uv_t, dv, (int64_t)dc * dv,
              w_o_absorbed, 0, (int64_t)H * dc, dc, s);
}

MLA_EXPORT mla_status_t mla_query_from_latent(const mla_dims_t* dims, int32_t batch,
                                              int32_t q_len, int32_t d_cq, const void* c_q,
                                              const void* w_q_absorbed, const void* w_qr,
                                              const int32_t* seqlens, void* q_latent,
                                              void* q_pe, void* stream) {
  mla_status_t st = check_bf16_dims(dims);
  if (st != MLA_OK) return st;
  if (dims->latent_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if ((st = check_batch(batch, q_len)) != MLA_OK) return st;
  if (d_cq < 8 || d_cq % 8 != 0) return MLA_ERR_BAD_SHAPE;
  if (!c_q || !w_q_absorbed || !w_qr || !seqlens || !q_latent || !q_pe)
    return MLA_ERR_NULL_POINTER;
  if (!aligned16(c_q) || !aligned16(w_q_absorbed) || !aligned16(w_qr) || !aligned16(seqlens) ||
      !aligned16(q_latent) || !aligned16(q_pe))
    return MLA_ERR_MISALIGNED;
  if (batch == 0) return MLA_OK;
  const int H = dims->n_heads, dc = dims->d_latent, dr = dims->d_rope;
  const int T = batch * q_len;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // q~[t, h, :] = W~_h c^Q_t: batch over heads, c^Q shared (stride 0)
  if ((st = gemm(H, T, dc, d_cq, c_q, d_cq, 0, w_q_absorbed, d_cq, (int64_t)dc * d_cq, q_latent,
                 0, (int64_t)H * dc, dc, s)) != MLA_OK)
    return st;
  // q^R = W_QR c^Q into q_pe, then rotated in place
  if ((st = gemm(1, T, H * dr, d_cq, c_q, d_cq, 0, w_qr, d_cq, 0, q_pe, 0, (int64_t)H * dr, 0,
                 s)) != MLA_OK)
    return st;
  mla::RopeArgs r;
  r.src = q_pe; r.dst = q_pe; r.seqlens = seqlens;
  r.batch = batch; r.q_len = q_len; r.n_heads = H; r.d_rope = dr; r.rope_base = dims->rope_base;
  return launch_status(mla::launch_rope_query(r, s));
}
