// StreamingLLM-style eviction view of the paged latent cache, gfx950.
//
// The related-papers page ("Related papers: SnapMLA: Efficient Long-Context
// MLA Decoding via H…", scifaro.com) names eviction techniques (StreamingLLM,
// SnapKV) that bound a long context's KV cache.  Here a sequence of L tokens
// keeps its first sink_pages pages (the attention sinks) and its most recent
// tokens from the page boundary at or below L - window_pages * page on; a
// sequence whose window would reach back into its sinks keeps everything.
// Kept tokens stay where they are in HBM and at the positions they were cached
// at (their rotary keys are stored already rotated), so the view is only a new
// block table and new lengths: the decode then runs unchanged over it, while
// the absorb pass still takes the true lengths for the query positions.
//
// One wave per sequence; lane j writes output pages j, j + 64, ...
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

__global__ __launch_bounds__(64) void streaming_view_kernel(StreamingViewArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int L = a.seqlens[b];
  const int page = a.page_size;
  const int sink = a.sink_pages * page;
  const int window = a.window_pages * page;
  const int start = L > window ? (L - window) / page * page : 0;
  const bool keep_all = start <= sink;
  const int kept_len = keep_all ? L : sink + (L - start);
  const int pages_in = (L + page - 1) / page;
  const int32_t* src = a.block_table + (int64_t)b * a.max_pages;
  int32_t* dst = a.out_block_table + (int64_t)b * a.max_pages_out;
  for (int j = lane; j < a.max_pages_out; j += 64) {
    int v = 0;
    if (keep_all) {
      if (j < pages_in) v = src[j];
    } else if (j < a.sink_pages) {
      v = src[j];
    } else {
      const int pj = start / page + (j - a.sink_pages);
      if (pj < pages_in) v = src[pj];
    }
    dst[j] = v;
  }
  if (lane == 0) a.out_seqlens[b] = kept_len;
}

}  // namespace

hipError_t launch_streaming_view(const StreamingViewArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(streaming_view_kernel, dim3(a.batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
