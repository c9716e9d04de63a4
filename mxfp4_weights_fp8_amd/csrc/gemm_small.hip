// Small-M grouped GEMMs (decode shapes, at most 16 routed rows per tile), on the
// gfx950 block-scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4.
//
// A 7-token verify leaves each expert a handful of rows, so generic tiles of 16+
// token rows mostly compute padding ("Optimization progress report",
// Optimization 06). Here the weights take the MFMA's 16-row A side (E2M1, one
// E8M0 scale per 32 K) and the routed tokens its 16-column B side (E4M3, the
// per-128 activation scale replicated over the four 32-blocks). The work is a
// stream of the expert's weights: each lane loads one 16-byte run of 32 E2M1
// codes per fragment and K step straight from HBM into registers (no reuse
// across waves, so no LDS staging), four fragments per wave in flight.
//
// W13 (gate/up, "Pushing the Limits of Serving DeepSeek-V4-Pro", section 3.3):
// a workgroup owns 128 columns of h = silu(gate) * up, i.e. gate rows
// [n0, n0+128) and up rows [I+n0, I+n0+128) of the expert, so the fused SwiGLU +
// FP8 requantization epilogue (same blog, section 4.3) sees a whole 128-column
// scale block per routed row and writes W2's E4M3 operand and E8M0 scales
// directly.
// W2 (down): a workgroup owns 256 output columns; the epilogue writes each routed
// pair's fp32 row to its token-major slot p = t*K + j for the top-k combine.
#include "device_common.h"
#include "host_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ v8i act_operand(const uint8_t* p) {
  // 8-bit B operand of one 128-long K step: bytes [16q, 16q+16) and [64+16q, 64+16q+16)
  const v4i lo = load16(p), hi = load16(p + 64);
  v8i b;
  b[0] = lo[0]; b[1] = lo[1]; b[2] = lo[2]; b[3] = lo[3];
  b[4] = hi[0]; b[5] = hi[1]; b[6] = hi[2]; b[7] = hi[3];
  return b;
}

__device__ __forceinline__ v8i fp4_operand(const uint8_t* p) {
  const v4i w = load16(p);
  v8i a;
  a[0] = w[0]; a[1] = w[1]; a[2] = w[2]; a[3] = w[3];
  a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
  return a;
}

__global__ __launch_bounds__(kThreads) void k_w13_small(
    const int2* __restrict__ items, const int32_t* __restrict__ n_items, int item_rows,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
    const uint8_t* __restrict__ x_q, const uint8_t* __restrict__ x_s, const uint8_t* __restrict__ w13,
    const uint8_t* __restrict__ w13_s, uint8_t* __restrict__ h_q, uint8_t* __restrict__ h_s, int H, int I,
    int K) {
  __shared__ float red[kThreads / 64][16];
  const int item = blockIdx.y;
  if (item >= n_items[0]) return;
  const int2 it = items[item];
  const int e = it.x;
  const int e_begin = offsets[e], e_end = offsets[e + 1];
  const int nb = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  const int KS = H / 128;
  const int64_t wrow = H / 2, srow = H / 32;

  const uint8_t* wp[4];
  const uint8_t* sp[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int64_t n = (int64_t)e * 2 * I + (f >= 2 ? I : 0) + nb * 128 + wave * 32 + (f & 1) * 16 + c;
    wp[f] = w13 + n * wrow + q * 16;
    sp[f] = w13_s + n * srow + q;
  }

  for (int m0 = it.y; m0 < it.y + item_rows && e_begin + m0 < e_end; m0 += kSmallRows) {
    const int row0 = e_begin + m0;
    const int mcount = min(kSmallRows, e_end - row0);
    const bool has = c < mcount;
    const int tok = has ? sorted_pairs[row0 + c] / K : 0;
    const uint8_t* xp = x_q + (int64_t)tok * H + q * 16;
    const uint8_t* xsp = x_s + (int64_t)tok * KS;

    v4f acc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int ks = 0; ks < KS; ++ks) {
      v8i b = {0, 0, 0, 0, 0, 0, 0, 0};
      int sb = 127;
      if (has) {
        b = act_operand(xp + ks * 128);
        sb = xsp[ks];
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const v8i a = fp4_operand(wp[f] + ks * 64);
        acc[f] = mfma_scale_16x16x128<kFmtE2M1, kFmtE4M3>(a, b, acc[f], sp[f][ks * 4], sb);
      }
    }

    // SwiGLU + FP8 requantization: lane (c, q) holds h columns 4q..4q+3 of each
    // 16-column fragment pair, for routed row c.
    float h[2][4];
    float amax = 0.f;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[g][j] = silu_mul(acc[g][j], acc[g + 2][j]);
        amax = fmaxf(amax, fabsf(h[g][j]));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (q == 0) red[wave][c] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
    __syncthreads();
    const int ex = e8m0_exponent(amax);
    const float inv = exp2_neg(ex);
    if (has) {
      uint8_t* dst = h_q + (int64_t)(row0 + c) * I + nb * 128 + wave * 32 + q * 4;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint32_t packed = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) packed |= e4m3_encode(h[g][j] * inv) << (8 * j);
        *reinterpret_cast<uint32_t*>(dst + g * 16) = packed;
      }
      if (wave == 0 && q == 0) h_s[(int64_t)(row0 + c) * (I / 128) + nb] = (uint8_t)(ex + 127);
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_w2_small(
    const int2* __restrict__ items, const int32_t* __restrict__ n_items, int item_rows,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
    const uint8_t* __restrict__ h_q, const uint8_t* __restrict__ h_s, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ w2_s, float* __restrict__ o, int H, int I) {
  const int item = blockIdx.y;
  if (item >= n_items[0]) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  const int n_wave = blockIdx.x * 256 + wave * 64;
  if (n_wave >= H) return;
  const int2 it = items[item];
  const int e = it.x;
  const int e_begin = offsets[e], e_end = offsets[e + 1];
  const int KS = I / 128;
  const int64_t wrow = I / 2, srow = I / 32;

  const uint8_t* wp[4];
  const uint8_t* sp[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int64_t n = (int64_t)e * H + n_wave + f * 16 + c;
    wp[f] = w2 + n * wrow + q * 16;
    sp[f] = w2_s + n * srow + q;
  }

  for (int m0 = it.y; m0 < it.y + item_rows && e_begin + m0 < e_end; m0 += kSmallRows) {
    const int row0 = e_begin + m0;
    const int mcount = min(kSmallRows, e_end - row0);
    const bool has = c < mcount;
    const uint8_t* hp = h_q + (int64_t)(has ? row0 + c : row0) * I + q * 16;
    const uint8_t* hsp = h_s + (int64_t)(has ? row0 + c : row0) * KS;

    v4f acc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int ks = 0; ks < KS; ++ks) {
      v8i b = {0, 0, 0, 0, 0, 0, 0, 0};
      int sb = 127;
      if (has) {
        b = act_operand(hp + ks * 128);
        sb = hsp[ks];
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const v8i a = fp4_operand(wp[f] + ks * 64);
        acc[f] = mfma_scale_16x16x128<kFmtE2M1, kFmtE4M3>(a, b, acc[f], sp[f][ks * 4], sb);
      }
    }
    if (has) {
      const int64_t slot = sorted_pairs[row0 + c];
      float* dst = o + slot * H + n_wave + q * 4;
#pragma unroll
      for (int f = 0; f < 4; ++f)
        *reinterpret_cast<float4*>(dst + f * 16) = make_float4(acc[f][0], acc[f][1], acc[f][2], acc[f][3]);
    }
  }
}

}  // namespace

hipError_t launch_w13_small(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                            int item_rows, const int32_t* offsets, const int32_t* sorted_pairs,
                            const uint8_t* x_q, const uint8_t* x_s, const uint8_t* w13, const uint8_t* w13_s,
                            uint8_t* h_q, uint8_t* h_s, hipStream_t s) {
  if (max_items <= 0) return hipSuccess;
  dim3 grid(d.I / 128, (unsigned)max_items);
  hipLaunchKernelGGL(k_w13_small, grid, dim3(kThreads), 0, s, items, n_items, item_rows, offsets, sorted_pairs,
                     x_q, x_s, w13, w13_s, h_q, h_s, d.H, d.I, d.K);
  return hipGetLastError();
}

hipError_t launch_w2_small(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                           int item_rows, const int32_t* offsets, const int32_t* sorted_pairs,
                           const uint8_t* h_q, const uint8_t* h_s, const uint8_t* w2, const uint8_t* w2_s,
                           float* o, hipStream_t s) {
  if (max_items <= 0) return hipSuccess;
  dim3 grid((unsigned)ceil_div(d.H, 256), (unsigned)max_items);
  hipLaunchKernelGGL(k_w2_small, grid, dim3(kThreads), 0, s, items, n_items, item_rows, offsets, sorted_pairs,
                     h_q, h_s, w2, w2_s, o, d.H, d.I);
  return hipGetLastError();
}

}  // namespace moe
