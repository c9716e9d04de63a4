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
constexpr int kUniformMaxTokens = 4096;

// UNIFORM: groups_per_row is a multiple of 64, so the 64 lanes of a wave serve one
// token; its index is then made wave-uniform, and the token's pick weights and pair
// rows come through scalar loads instead of one vector load per lane and pick. Used
// for batches of at most kUniformMaxTokens, where the combine is a few waves bound
// by load latency (decode7 0.2206 vs 0.2221 ms per step, 256 tokens 1.930 vs 1.932
// ms); at 32K tokens, bound by streaming 4 GB of rows, it measured 0.6% slower.
template <bool UNIFORM>
__global__ __launch_bounds__(kThreads) void k_combine(const uint16_t* __restrict__ o, const uint8_t* __restrict__ os,
                                                       const float* __restrict__ w,
                                                       const int32_t* __restrict__ pair_rows,
                                                       const uint16_t* __restrict__ so,
                                                       const uint8_t* __restrict__ sos, uint16_t* __restrict__ y,
                                                       int64_t n_groups, int groups_per_row, int K) {
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < n_groups; g += (int64_t)gridDim.x * kThreads) {
    int64_t t = g / groups_per_row;
    if constexpr (UNIFORM) t = __builtin_amdgcn_readfirstlane((int)t);
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
  if ((H / 8) % 64 == 0 && T <= kUniformMaxTokens)   // kThreads and the grid stride are multiples of 64 too
    hipLaunchKernelGGL(k_combine<true>, dim3((unsigned)ctas), dim3(kThreads), 0, s, o, os, topk_weights, pair_rows,
                       so, sos, y, n_groups, H / 8, K);
  else
    hipLaunchKernelGGL(k_combine<false>, dim3((unsigned)ctas), dim3(kThreads), 0, s, o, os, topk_weights, pair_rows,
                       so, sos, y, n_groups, H / 8, K);
  return hipGetLastError();
}

}  // namespace moe
