// Top-k weighted combine ("Pushing the Limits of Serving DeepSeek-V4-Pro",
// section 3.2: the top-k reduction is fused with the shared-expert add):
//   y[t, :] = bf16( sum_j w[t, j] * o[t*K + j, :]  (+ shared[t, :]) )
// Atomic-free gather: each lane owns 8 columns of one token, reads the K per-pair
// rows (contiguous, token-major slots; fp16 codes with a power-of-two scale per 32
// columns, decoded exactly to fp32), accumulates in fp32 in pick order, adds the
// shared expert last and rounds once to bf16. Dropped picks (pair_rows == -1)
// contribute nothing. HBM-bound.
#include "device_common.h"
#include "host_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float f16_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu)); }
__device__ __forceinline__ float f16_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

__global__ __launch_bounds__(kThreads) void k_combine(const uint16_t* __restrict__ o, const uint8_t* __restrict__ os,
                                                       const float* __restrict__ w,
                                                       const int32_t* __restrict__ pair_rows,
                                                       const uint16_t* __restrict__ so,
                                                       const uint8_t* __restrict__ sos, uint16_t* __restrict__ y,
                                                       int64_t n_groups, int groups_per_row, int K) {
  const int scales_per_row = groups_per_row / 4;   // one scale per 32 columns = 4 groups of 8
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < n_groups; g += (int64_t)gridDim.x * kThreads) {
    const int64_t t = g / groups_per_row;
    const int64_t c8 = g - t * groups_per_row;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // j in order; batches of 8 pairs issue all their loads before the first add (a
    // dropped pair's row is loaded but not added: its slot was never written)
    for (int j0 = 0; j0 < K; j0 += 8) {
      uint4 v[8];
      int ex[8];
      float wt[8];
      bool ok[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int64_t p = t * K + min(j0 + jj, K - 1);
        ok[jj] = j0 + jj < K && pair_rows[p] >= 0;
        wt[jj] = w[p];
        const v4i r = load16_nt(reinterpret_cast<const uint4*>(o) + p * groups_per_row + c8);
        v[jj] = make_uint4((uint32_t)r.x, (uint32_t)r.y, (uint32_t)r.z, (uint32_t)r.w);
        ex[jj] = (int)os[p * scales_per_row + (c8 >> 2)] - 127;
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (ok[jj]) {
          const uint32_t u[4] = {v[jj].x, v[jj].y, v[jj].z, v[jj].w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            acc[2 * k] = fmaf(wt[jj], __builtin_amdgcn_ldexpf(f16_lo(u[k]), ex[jj]), acc[2 * k]);
            acc[2 * k + 1] = fmaf(wt[jj], __builtin_amdgcn_ldexpf(f16_hi(u[k]), ex[jj]), acc[2 * k + 1]);
          }
        }
      }
    }
    if (so) {   // the shared expert's row, same storage as the per-pair rows, added last
      const v4i r = load16_nt(reinterpret_cast<const uint4*>(so) + g);
      const uint4 v = make_uint4((uint32_t)r.x, (uint32_t)r.y, (uint32_t)r.z, (uint32_t)r.w);
      const int ex = (int)sos[t * scales_per_row + (c8 >> 2)] - 127;
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] += __builtin_amdgcn_ldexpf(f16_lo(u[k]), ex);
        acc[2 * k + 1] += __builtin_amdgcn_ldexpf(f16_hi(u[k]), ex);
      }
    }
    uint4 r;
    r.x = (uint32_t)bf16_rne(acc[0]) | ((uint32_t)bf16_rne(acc[1]) << 16);
    r.y = (uint32_t)bf16_rne(acc[2]) | ((uint32_t)bf16_rne(acc[3]) << 16);
    r.z = (uint32_t)bf16_rne(acc[4]) | ((uint32_t)bf16_rne(acc[5]) << 16);
    r.w = (uint32_t)bf16_rne(acc[6]) | ((uint32_t)bf16_rne(acc[7]) << 16);
    reinterpret_cast<uint4*>(y)[g] = r;
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
