// Top-k weighted combine ("Pushing the Limits of Serving DeepSeek-V4-Pro",
// section 3.2: the top-k reduction is fused with the shared-expert add):
//   y[t, :] = bf16( sum_j w[t, j] * o[t*K + j, :]  (+ shared[t, :]) )
// Atomic-free gather: each lane owns 4 columns of one token, reads the K per-pair
// fp32 rows (contiguous, token-major slots), accumulates in fp32 in pick order,
// adds the shared expert last and rounds once to bf16. Dropped picks
// (pair_rows == -1) contribute nothing. HBM-bound.
#include "device_common.h"
#include "host_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_combine(const float* __restrict__ o, const float* __restrict__ w,
                                                       const int32_t* __restrict__ pair_rows,
                                                       const float* __restrict__ so, uint16_t* __restrict__ y,
                                                       int64_t n_groups, int groups_per_row, int K) {
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < n_groups; g += (int64_t)gridDim.x * kThreads) {
    const int64_t t = g / groups_per_row;
    const int64_t c4 = g - t * groups_per_row;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // j in order; batches of 8 pairs issue all their loads before the first add (a
    // dropped pair's row is loaded but not added: its slot was never written)
    for (int j0 = 0; j0 < K; j0 += 8) {
      float4 v[8];
      float wt[8];
      bool ok[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int64_t p = t * K + min(j0 + jj, K - 1);
        ok[jj] = j0 + jj < K && pair_rows[p] >= 0;
        wt[jj] = w[p];
        v[jj] = reinterpret_cast<const float4*>(o)[p * groups_per_row + c4];
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (ok[jj]) {
          acc.x = fmaf(wt[jj], v[jj].x, acc.x);
          acc.y = fmaf(wt[jj], v[jj].y, acc.y);
          acc.z = fmaf(wt[jj], v[jj].z, acc.z);
          acc.w = fmaf(wt[jj], v[jj].w, acc.w);
        }
      }
    }
    if (so) {
      const float4 v = reinterpret_cast<const float4*>(so)[g];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const uint32_t lo = (uint32_t)bf16_rne(acc.x) | ((uint32_t)bf16_rne(acc.y) << 16);
    const uint32_t hi = (uint32_t)bf16_rne(acc.z) | ((uint32_t)bf16_rne(acc.w) << 16);
    reinterpret_cast<uint2*>(y)[g] = make_uint2(lo, hi);
  }
}

}  // namespace

hipError_t launch_combine(const float* o, const float* topk_weights, const int32_t* pair_rows, const float* so,
                          uint16_t* y, int T, int H, int K, hipStream_t s) {
  const int64_t n_groups = (int64_t)T * (H / 4);
  if (n_groups == 0) return hipSuccess;
  int64_t ctas = ceil_div(n_groups, kThreads);
  if (ctas > 256 * 32) ctas = 256 * 32;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)ctas), dim3(kThreads), 0, s, o, topk_weights, pair_rows, so, y,
                     n_groups, H / 4, K);
  return hipGetLastError();
}

}  // namespace moe
