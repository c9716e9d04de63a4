// Online FP8 activation quantization ("Pushing the Limits of Serving
// DeepSeek-V4-Pro", section 2.2): bf16 x [T, H] -> E4M3 codes [T, H] and one E8M0
// scale per token per 128 columns. HBM-bound: 16 lanes own one 128-column block,
// each loads 8 bf16 (16 B) and stores 8 codes (8 B); the block amax is a 16-lane
// butterfly. The scale is the smallest power of two with amax <= 448 * scale, so
// x / scale is exact and no code saturates; codes round to nearest-even.
// Optionally the quantized values themselves, E4M3(code) * scale, are written as
// bf16 too (exact: at most 4 significant bits, inside bf16's range for every
// scale a finite bf16 block below 2^127 can take): the operand of the shared
// expert's bf16 gate/up GEMM.
#include "device_common.h"
#include "host_internal.h"

namespace moe {
namespace {

constexpr int kQuantThreads = 256;

__global__ __launch_bounds__(kQuantThreads) void k_quant_act(const uint16_t* __restrict__ x,
                                                              uint8_t* __restrict__ x_q,
                                                              uint8_t* __restrict__ x_s,
                                                              uint16_t* __restrict__ x_hat,
                                                              int32_t* __restrict__ zero, int n_zero,
                                                              int64_t n_blocks) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_zero; i += kQuantThreads) zero[i] = 0;
  const int sub = threadIdx.x & 15;
  const int64_t groups_per_cta = kQuantThreads / 16;
  for (int64_t blk = (int64_t)blockIdx.x * groups_per_cta + (threadIdx.x >> 4); blk < n_blocks;
       blk += (int64_t)gridDim.x * groups_per_cta) {
    const int64_t base = blk * 128 + sub * 8;   // element index of this lane's 8 values
    const v4i raw = load16_nt(x + base);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_float((uint16_t)(raw[i] & 0xFFFF));
      v[2 * i + 1] = bf16_to_float((uint16_t)((uint32_t)raw[i] >> 16));
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    const int e = e8m0_exponent(amax);
    const float inv = exp2_neg(e);
    const uint32_t lo = e4m3_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    const uint32_t hi = e4m3_pack4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    *reinterpret_cast<uint2*>(x_q + base) = make_uint2(lo, hi);
    if (sub == 0) x_s[blk] = (uint8_t)(e + 127);
    if (x_hat) {
      const uint2 a = e4m3x4_to_bf16(lo, e), b = e4m3x4_to_bf16(hi, e);
      *reinterpret_cast<uint4*>(x_hat + base) = make_uint4(a.x, a.y, b.x, b.y);
    }
  }
}

}  // namespace

hipError_t launch_quant_act(const uint16_t* x, uint8_t* x_q, uint8_t* x_s, int T, int H, hipStream_t s,
                            uint16_t* x_hat, int32_t* zero, int n_zero) {
  const int64_t n_blocks = (int64_t)T * (H / 128);
  if (n_blocks == 0) return hipSuccess;
  // one 128-column block per 16 lanes (at 32K tokens 0.120 ms against 0.127 ms with the
  // grid capped at 4096 workgroups and a grid-stride loop)
  const int64_t ctas = ceil_div(n_blocks, kQuantThreads / 16);
  hipLaunchKernelGGL(k_quant_act, dim3((unsigned)ctas), dim3(kQuantThreads), 0, s, x, x_q, x_s, x_hat, zero,
                     n_zero, n_blocks);
  return hipGetLastError();
}

}  // namespace moe
