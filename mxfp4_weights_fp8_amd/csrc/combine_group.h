// The top-k weighted combine of one group of 8 output columns of one token,
// shared by the combine kernel and the decode chain:
//   y[t, 8 c8 .. 8 c8 + 7] = bf16( sum_j w[t, j] * o[t*K + j, ...]  (+ shared[t, ...]) )
// Per-pair rows are fp16 codes with one power-of-two scale per 32 columns (token-
// major slots p = t*K + j), decoded exactly to fp32 and accumulated in fp32 in pick
// order; the shared expert's row (same storage) is added last; one rounding to
// bf16. Dropped picks (pair_rows == -1) contribute nothing.
// COH: the per-pair rows were written by other workgroups of the same launch with
// device-scope coherent stores. Their scale bytes are then read with device-scope
// coherent (sc1) loads: a cache line of scales holds several column blocks' bytes,
// and another column block's combine may have cached it before these were
// written. The fp16 rows keep the default policy: the 256-column block a combine
// reads is whole cache lines that nothing in the launch read before.
#pragma once

#include "device_common.h"

namespace moe {

__device__ __forceinline__ float f16_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu)); }
__device__ __forceinline__ float f16_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

template <bool COH = false>
__device__ __forceinline__ void combine_group(const uint16_t* __restrict__ o, const uint8_t* __restrict__ os,
                                              const float* __restrict__ w, const int32_t* __restrict__ pair_rows,
                                              const uint16_t* __restrict__ so, const uint8_t* __restrict__ sos,
                                              uint16_t* __restrict__ y, int64_t t, int c8, int groups_per_row,
                                              int K) {
  const int scales_per_row = groups_per_row / 4;   // one scale per 32 columns = 4 groups of 8
  const int64_t g = t * groups_per_row + c8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // the shared expert's row (same storage as the per-pair rows) is loaded with the
  // first batch and added last
  v4i sr = {0, 0, 0, 0};
  int sex = 0;
  if (so) {
    sr = load16_nt(reinterpret_cast<const uint4*>(so) + g);
    sex = (int)sos[t * scales_per_row + (c8 >> 2)] - 127;
  }
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
      if constexpr (COH)
        ex[jj] = buf_load1<16>(make_rsrc(os, 0xFFFFFFFFu), (int)(p * scales_per_row + (c8 >> 2)), 0) - 127;
      else
        ex[jj] = (int)os[p * scales_per_row + (c8 >> 2)] - 127;
      v[jj] = make_uint4((uint32_t)r.x, (uint32_t)r.y, (uint32_t)r.z, (uint32_t)r.w);
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
  if (so) {
    const uint32_t u[4] = {(uint32_t)sr.x, (uint32_t)sr.y, (uint32_t)sr.z, (uint32_t)sr.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] += __builtin_amdgcn_ldexpf(f16_lo(u[k]), sex);
      acc[2 * k + 1] += __builtin_amdgcn_ldexpf(f16_hi(u[k]), sex);
    }
  }
  uint4 r;
  r.x = (uint32_t)bf16_rne(acc[0]) | ((uint32_t)bf16_rne(acc[1]) << 16);
  r.y = (uint32_t)bf16_rne(acc[2]) | ((uint32_t)bf16_rne(acc[3]) << 16);
  r.z = (uint32_t)bf16_rne(acc[4]) | ((uint32_t)bf16_rne(acc[5]) << 16);
  r.w = (uint32_t)bf16_rne(acc[6]) | ((uint32_t)bf16_rne(acc[7]) << 16);
  reinterpret_cast<uint4*>(y)[g] = r;
}

}  // namespace moe
