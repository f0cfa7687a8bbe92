// Device check of the paged decode's preconditions (MLA_VALIDATE=1): one
// workgroup; thread t checks sequences t, t + 256, ... with the predicate the
// host check uses, and thread 0 stores the number of sequences that break it
// (a plain store: nothing needs clearing beforehand).
#include "mla_internal.hpp"
#include "mla_validate.hpp"

namespace mla {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void validate_paged_kernel(ValidateArgs a) {
  __shared__ int s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  int bad = 0;
  for (int b = threadIdx.x; b < a.batch; b += kThreads)
    bad += sequence_ok(a.block_table + (int64_t)b * a.max_pages, a.seqlens[b], a.max_seqlen,
                       a.max_pages, a.page_size, a.num_pages) ? 0 : 1;
  if (bad) atomicAdd(&s_bad, bad);
  __syncthreads();
  if (threadIdx.x == 0) *a.bad = s_bad;
}

}  // namespace

hipError_t launch_validate(const ValidateArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(validate_paged_kernel, dim3(1), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
