// kda_plan.hip -- device-side scheduling of a varlen batch.
//
// cu_seqlens stays on the device (the call never synchronises with the host,
// so it can be captured in a graph), so the processing order of the sequences
// is computed here: longest first, ties by index.  Workgroups of the main
// kernels take their sequence from this table, so the longest recurrences
// start first and the short ones fill in behind them.
#include "kda_internal.h"

namespace kda {
namespace {

__global__ __launch_bounds__(256) void plan_kernel(const int32_t* __restrict__ cu, int N, int32_t* __restrict__ order) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  const int li = cu[i + 1] - cu[i];
  int rank = 0;
  for (int m = 0; m < N; ++m) {
    const int lm = cu[m + 1] - cu[m];
    rank += (lm > li) || (lm == li && m < i);
  }
  order[rank] = i;  // (length desc, index asc) is a strict order: a permutation
}

}  // namespace

hipError_t launch_plan(const Params& p, hipStream_t stream) {
  const int threads = 256;
  const int blocks = (p.N + threads - 1) / threads;
  const int32_t* cu = p.cu;
  int N = p.N;
  int32_t* order = p.order;
  void* args[] = {&cu, &N, &order};
  return hipLaunchKernel(reinterpret_cast<const void*>(&plan_kernel), dim3(blocks), dim3(threads),
                         args, 0, stream);
}

}  // namespace kda
