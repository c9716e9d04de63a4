// Top-k weighted combine ("Pushing the Limits of Serving DeepSeek-V4-Pro",
// section 3.2: the top-k reduction is fused with the shared-expert add):
//   y[t, :] = bf16( sum_j w[t, j] * o[t*K + j, :]  (+ shared[t, :]) )
// Atomic-free gather: each lane owns 8 columns of one token, reads the K per-pair
// rows (contiguous, token-major slots; fp16 codes with a power-of-two scale per 32
// columns, decoded exactly to fp32), accumulates in fp32 in pick order, adds the
// shared expert last and rounds once to bf16. Dropped picks (pair_rows == -1)
// contribute nothing. HBM-bound.
#include "combine_group.h"
#include "host_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_combine(const uint16_t* __restrict__ o, const uint8_t* __restrict__ os,
                                                       const float* __restrict__ w,
                                                       const int32_t* __restrict__ pair_rows,
                                                       const uint16_t* __restrict__ so,
                                                       const uint8_t* __restrict__ sos, uint16_t* __restrict__ y,
                                                       int64_t n_groups, int groups_per_row, int K) {
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < n_groups; g += (int64_t)gridDim.x * kThreads) {
    const int64_t t = g / groups_per_row;
    combine_group(o, os, w, pair_rows, so, sos, y, t, (int)(g - t * groups_per_row), groups_per_row, K);
  }
}

}  // namespace

hipError_t launch_combine(const uint16_t* o, const uint8_t* os, const float* topk_weights, const int32_t* pair_rows,
                          const uint16_t* so, const uint8_t* sos, uint16_t* y, int T, int H, int K, hipStream_t s) {
  const int64_t n_groups = (int64_t)T * (H / 8);
  if (n_groups == 0) return hipSuccess;
  // one 8-column group per thread (measured at 32K tokens: 0.78 ms against 0.84 ms
  // with the grid capped at 8192 workgroups and a grid-stride loop)
  const int64_t ctas = ceil_div(n_groups, kThreads);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)ctas), dim3(kThreads), 0, s, o, os, topk_weights, pair_rows, so, sos, y,
                     n_groups, H / 8, K);
  return hipGetLastError();
}

}  // namespace moe
