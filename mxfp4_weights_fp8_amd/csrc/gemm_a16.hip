// MXFP4 weights x bf16 activations ("MXFP4A16", the variant beside MXFP4AFP8 in
// "Pushing the Limits of Serving DeepSeek-V4-Pro", Appendix D.2, accuracy table):
// the activations are not quantized, the SwiGLU output stays bf16 as W2's operand,
// and the expert weights keep their MXFP4 codes and E8M0 scales.
//
// The block-scaled MFMA takes 8-, 6- and 4-bit operands only, so each E2M1 code is
// expanded with its 32-element block's scale into bf16 in registers (exact: an
// E2M1 value has at most 2 significant bits and the scale is a power of two, inside
// bf16's range for scales 2^-127 .. 2^125) by gfx950's scaled FP4-to-bf16 conversion,
// and multiplied on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//
// The structure of the FP8 small-M kernels (gemm_small.hip): the weights take the
// MFMA's 16-row A side, the routed tokens its 16-column B side, 16 routed rows per
// tile, weight codes streamed from the kernel-native layout (lane (c, q) of a
// fragment holds row c, K 32q .. 32q+31 of the 128-K step), MXFP4 scales staged in
// LDS per wave; the number of fragments per wave is chosen per variant (below). One 128-K step is four bf16 MFMAs; in MFMA u, lane (c, q) supplies K
// 32q + 8u .. +7 for both operands (the instruction sums over K, so any assignment
// of K to its slots that the two operands share gives the same dot product), so the
// lane's weights come from its own 16 code bytes and its activations are 64
// consecutive bytes of the token row. Every item list of the plan is walked in
// 16-row tiles: efficient for decode (HBM-bound weight streams), correct for any
// shape.
//
// NVFP4 weights (template flag NV; "Optimization progress report", Optimization
// 05, runs NVFP4 expert weights as stored): the same E2M1 codes, but one E4M3
// scale per 16 K elements ([rows, K/16] bytes, row-major) and one fp32 scale per
// expert tensor (NVIDIA's published NVFP4 layout; the page names the format
// only). The conversion above takes only the power of two of its scale operand,
// so a block scale v = f * 2^k (f an integer 8 .. 15, 0 for a zero scale) expands
// its codes to fp32 with 2^k, multiplies them by f (exact: at most 6 significant
// bits) and keeps the upper halves as bf16 (exact for the same reason). A lane's
// 32 K of a step span two 16-blocks (MFMAs u = 0, 1 and u = 2, 3); their two scale
// bytes come in one 4-byte load per fragment and step, in the same register ring
// as the codes. The per-tensor scale multiplies the fp32 accumulators before the
// epilogue (it is constant over the contraction).
#include "small_unit.h"

namespace moe {
namespace {

using namespace small;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Work split per variant. Each 128-K step is four bf16 MFMAs per fragment, each
// accumulating into the previous one, so a wave with more fragments has more
// independent MFMA chains to interleave with the codes' expansion. Measured (one box,
// bitwise-equal results, per step): MXFP4 x bf16 with W13 in 4 waves x (2 gate + 2 up
// fragments) and W2 in 2 waves x 4 fragments: decode7 0.226 vs 0.246 ms and the
// 256-token step 2.32 vs 2.80 ms against 8 x (1 + 1) and 4 x 2. NVFP4, whose codes take
// four times the VALU work to expand, keeps 8 x (1 + 1) and 4 x 2 up to kNvWidePairs
// pairs: there its 4 x (2 + 2) W13 ran decode7 4% slower (0.366 vs 0.351 ms) and its
// 2 x 4 W2 1% slower; above, as on the 256-token step, they ran 3% and 2% faster, and
// are used.
constexpr int kW13Waves = 4;      // MXFP4 W13: 4 waves, NG = 2 gate + 2 up fragments each (128 h columns)
constexpr int kW13WavesNV = 8;    // NVFP4 W13: 8 waves, one gate + one up fragment each
constexpr int kW2Waves = 2;       // MXFP4 W2: 2 waves of 4 fragments (128 output columns)
constexpr int kW2Frags = 4;
constexpr int kW2WavesNV = 4;     // NVFP4 W2: 4 waves of 2 fragments (128 output columns)
constexpr int kW2FragsNV = 2;
constexpr int64_t kNvWidePairs = 512;
// K steps of codes in flight per wave: two (the ring then holds 52 registers, so
// the kernels fit 4-5 waves per SIMD instead of 3; the codes' expansion is VALU
// work that more waves hide better). Measured against four on one box, results
// bitwise equal: decode7 NVFP4 0.354 vs 0.362 ms per step, 256 tokens NVFP4 4.14
// vs 4.19 ms, decode7 bf16 activations 0.247 vs 0.249 ms.
constexpr int kQ = 2;

// E8M0 scale byte -> 2^(scale - 127) as a float (byte 0 is the fp32 subnormal 2^-127).
__device__ __forceinline__ float e8m0_float(uint32_t scale) {
  return scale ? __uint_as_float(scale << 23) : __uint_as_float(0x00400000u);
}

// 8 codes (one 32-bit word, low nibble = lower K) times the block scale -> 8 bf16 (4
// words, element 2i in the low half of word i), with gfx950's conversion of two
// FP4 codes with an fp32 scale (v_cvt_scalef32_pk_bf16_fp4, byte i of the word).
__device__ __forceinline__ v4i e2m1x8_bf16(uint32_t w, float scale) {
  v4i r;
  r[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return r;
}

typedef float v2f __attribute__((ext_vector_type(2)));

// NVFP4: 8 codes times the block scale f * 2^k (see above) -> 8 bf16, in the layout
// of e2m1x8_bf16.
__device__ __forceinline__ v4i e2m1x8_bf16_nv(uint32_t w, float pow2, float f) {
  v4i r;
#define NV_PAIR(k)                                                                           \
  {                                                                                          \
    const v2f p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, pow2, k);                      \
    r[k] = (int)__builtin_amdgcn_perm(__float_as_uint(p[1] * f), __float_as_uint(p[0] * f),  \
                                      0x07060302u);                                          \
  }
  NV_PAIR(0) NV_PAIR(1) NV_PAIR(2) NV_PAIR(3)
#undef NV_PAIR
  return r;
}

// An E4M3 block scale (finite, non-negative) as f * 2^k: pow2 = 2^k with
// k = floor(log2 v) - 3 and f = v / 2^k, an integer 8 .. 15 (v >= 2^-9, the smallest
// E4M3 subnormal, so k >= -12). With frexp's exponent x (v = g * 2^x, g in [0.5, 1))
// k = x - 4; for v = 0 frexp gives x = 0, so pow2 = 2^-4 (finite codes) and f = 0,
// and the block expands to zeros, with no test for zero.
__device__ __forceinline__ void nv_scale(float v, float& pow2, float& f) {
  const int x = __builtin_amdgcn_frexp_expf(v);
  pow2 = __builtin_amdgcn_ldexpf(0.0625f, x);   // 2^(x - 4)
  f = __builtin_amdgcn_ldexpf(v, 4 - x);
}

__device__ __forceinline__ v4f mfma_bf16(v4i a, v4i b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// Operands of one K step: NF fragments' codes (and, for NVFP4, scale words), the
// token column's 32 bf16.
template <int NF, bool NV>
struct Step16 {
  v4i w[NF];
  v4i x[4];
  uint32_t sw[NF];
};

// Where a wave's operands live: weight codes (resource + per-fragment lane offsets,
// step s at +1024 s), the token rows (resource + lane offset, step s at +256 s), the
// weight scales: MXFP4 in LDS (sl[f]: the lane's row of fragment f, K/32 bytes),
// NVFP4 in memory (resource + per-fragment lane offsets of the 4-byte word holding
// the lane's two block scales, step s at +8 s).
template <int NF, bool NV>
struct Stream16 {
  rsrc_t w, x, s;
  int wo[NF];
  int so[NF];
  int xo;
  const uint8_t* sl[NF];
};

template <int NF, bool NV>
__device__ __forceinline__ void load16(Step16<NF, NV>& r, const Stream16<NF, NV>& p, int s) {
#pragma unroll
  for (int f = 0; f < NF; ++f) r.w[f] = buf_load16_nt(p.w, p.wo[f], s * 1024);
  if constexpr (NV) {
#pragma unroll
    for (int f = 0; f < NF; ++f) r.sw[f] = (uint32_t)buf_load4(p.s, p.so[f], s * 8);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) r.x[u] = buf_load16(p.x, p.xo, s * 256 + 16 * u);
}

// One K step. MXFP4: sc[f] is the scale (as a float) of fragment f's lane's block.
// NVFP4: the lane's two block scales come from r.sw (bytes 2 (q & 1) and +1).
template <int NF, bool NV>
__device__ __forceinline__ void mma16(const Step16<NF, NV>& r, const float* sc, int q, v4f* acc) {
  if constexpr (NV) {
    float p2[NF][2], fm[NF][2];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint32_t w = r.sw[f] >> (16 * (q & 1));
      nv_scale(__builtin_amdgcn_cvt_f32_fp8((int)w, 0), p2[f][0], fm[f][0]);
      nv_scale(__builtin_amdgcn_cvt_f32_fp8((int)w, 1), p2[f][1], fm[f][1]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f)
        acc[f] = mfma_bf16(e2m1x8_bf16_nv((uint32_t)r.w[f][u], p2[f][u >> 1], fm[f][u >> 1]), r.x[u], acc[f]);
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[f] = mfma_bf16(e2m1x8_bf16((uint32_t)r.w[f][u], sc[f]), r.x[u], acc[f]);
  }
}

template <int NF, bool NV>
__device__ __forceinline__ void step_scales(const Stream16<NF, NV>& p, int s, int q, float* sc) {
  if constexpr (!NV) {
#pragma unroll
    for (int f = 0; f < NF; ++f) sc[f] = e8m0_float(p.sl[f][4 * s + q]);
  }
}

// acc[f] += sum over KS steps of 128 K. kQ steps of codes in flight in a register
// ring (prefetch indices clamped, so the loop is branch-free; KS a multiple of kQ),
// else one step at a time. The weight-scale copies into LDS are waited for first.
template <int NF, bool NV>
__device__ __forceinline__ void stream16(v4f* acc, const Stream16<NF, NV>& p, int KS, int q) {
  float sc[NF];
  if (KS % kQ != 0) {
    wait_vmcnt<0>();
    for (int s = 0; s < KS; ++s) {
      Step16<NF, NV> r;
      load16(r, p, s);
      step_scales(p, s, q, sc);
      mma16(r, sc, q, acc);
    }
    return;
  }
  Step16<NF, NV> buf[kQ];
#pragma unroll
  for (int d = 0; d < kQ; ++d) load16(buf[d], p, d);
  wait_vmcnt<0>();
  for (int s0 = 0; s0 < KS; s0 += kQ) {
#pragma unroll
    for (int d = 0; d < kQ; ++d) {
      step_scales(p, s0 + d, q, sc);
      mma16(buf[d], sc, q, acc);
      load16(buf[d], p, min(s0 + kQ + d, KS - 1));
    }
  }
}

// W13 unit: 128 h columns (nb) of one item, WAVES waves x (NG gate + NG up fragments),
// NG = 8 / WAVES. gs: NVFP4's per-expert tensor scales (unused for MXFP4).
template <bool NV, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_w13_a16(
    const SmallLists lists, const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w13, const uint8_t* __restrict__ w13_s,
    const float* __restrict__ gs, uint16_t* __restrict__ h, int H, int I, int K) {
  constexpr int NG = 8 / WAVES;
  constexpr int NF = 2 * NG;
  extern __shared__ __attribute__((aligned(16))) uint8_t sS[];   // MXFP4: per wave 2 runs of 16 NG rows x H/32
  const int l = blockIdx.y >= lists.cap0;
  const int item = blockIdx.y - (l ? lists.cap0 : 0);
  if (item >= lists.n_items[l][0]) return;
  const int2 it = lists.items[l][item];
  const int item_rows = lists.rows[l];
  const int e = it.x;
  const int e_begin = offsets[e], e_end = offsets[e + 1];
  const int nb = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  const int KS = H / 128;
  const int64_t wrow = H / 2;

  Stream16<NF, NV> p;
  p.w = make_rsrc(w13 + (int64_t)e * 2 * I * wrow, (uint32_t)(2 * I * wrow));
  p.x = make_rsrc(x, 0xFFFFFFFFu);
  const int n_gate = nb * 128 + wave * 16 * NG;   // first gate row of the wave; up row I + n_gate
#pragma unroll
  for (int f = 0; f < NF; ++f) p.wo[f] = ((f < NG ? 0 : I) + n_gate + 16 * (f % NG)) * (int)wrow + lane * 16;
  float g_scale = 1.f;
  if constexpr (NV) {
    const int64_t srow = H / 16;
    p.s = make_rsrc(w13_s + (int64_t)e * 2 * I * srow, (uint32_t)(2 * I * srow));
#pragma unroll
    for (int f = 0; f < NF; ++f)
      p.so[f] = ((f < NG ? 0 : I) + n_gate + 16 * (f % NG) + c) * (int)srow + 4 * (q >> 1);
    g_scale = gs[e];
  } else {
    const int64_t srow = H / 32;
    const int run = staged_bytes(16 * NG * (int)srow);
    stage_scales(w13_s + ((int64_t)e * 2 * I + n_gate) * srow, w13_s + ((int64_t)e * 2 * I + I + n_gate) * srow,
                 16 * NG * (int)srow, sS + wave * 2 * run, lane);
#pragma unroll
    for (int f = 0; f < NF; ++f) p.sl[f] = sS + wave * 2 * run + (f < NG ? 0 : run) + (16 * (f % NG) + c) * srow;
  }

  for (int m0 = it.y; m0 < it.y + item_rows && e_begin + m0 < e_end; m0 += kSmallRows) {
    const int row0 = e_begin + m0;
    const int mcount = min(kSmallRows, e_end - row0);
    const bool has = c < mcount;
    const int tok = sorted_pairs[row0 + (has ? c : 0)] / K;   // an absent column repeats the first row
    p.xo = (tok * H + 32 * q) * 2;
    v4f acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};
    stream16<NF, NV>(acc, p, KS, q);
    if constexpr (NV) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[f][i] *= g_scale;
    }
    // lane (c, q): h columns n_gate + 16 g + 4q .. +3 of routed row c, as bf16
    if (has) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        uint16_t* dst = h + (int64_t)(row0 + c) * I + n_gate + 16 * g + 4 * q;
        const uint32_t lo = (uint32_t)bf16_rne(silu_mul(acc[g][0], acc[NG + g][0])) |
                            ((uint32_t)bf16_rne(silu_mul(acc[g][1], acc[NG + g][1])) << 16);
        const uint32_t hi = (uint32_t)bf16_rne(silu_mul(acc[g][2], acc[NG + g][2])) |
                            ((uint32_t)bf16_rne(silu_mul(acc[g][3], acc[NG + g][3])) << 16);
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
      }
    }
  }
}

// W2 unit: WAVES * 16 * NF output columns of one item, WAVES waves x NF fragments;
// per-pair rows as fp16 codes with one power-of-two scale per 32 columns (a pair of
// the wave's fragments).
template <bool NV, int WAVES, int NF>
__global__ __launch_bounds__(WAVES * 64) void k_w2_a16(
    const SmallLists lists, const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
    const uint16_t* __restrict__ h, const uint8_t* __restrict__ w2, const uint8_t* __restrict__ w2_s,
    const float* __restrict__ gs, uint16_t* __restrict__ o, uint8_t* __restrict__ os, int H, int I) {
  static_assert(NF % 2 == 0, "whole 32-column scale blocks per wave");
  extern __shared__ __attribute__((aligned(16))) uint8_t sS[];   // MXFP4: per wave 16 NF rows x I/32
  const int l = blockIdx.y >= lists.cap0;
  const int item = blockIdx.y - (l ? lists.cap0 : 0);
  if (item >= lists.n_items[l][0]) return;
  const int2 it = lists.items[l][item];
  const int item_rows = lists.rows[l];
  const int e = it.x;
  const int e_begin = offsets[e], e_end = offsets[e + 1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  const int n_wave = (blockIdx.x * WAVES + wave) * 16 * NF;
  if (n_wave >= H) return;
  const int KS = I / 128;
  const int64_t wrow = I / 2;

  Stream16<NF, NV> p;
  p.w = make_rsrc(w2 + (int64_t)e * H * wrow, (uint32_t)(H * wrow));
  p.x = make_rsrc(h, 0xFFFFFFFFu);
#pragma unroll
  for (int f = 0; f < NF; ++f) p.wo[f] = (n_wave + f * 16) * (int)wrow + lane * 16;
  float g_scale = 1.f;
  if constexpr (NV) {
    const int64_t srow = I / 16;
    p.s = make_rsrc(w2_s + (int64_t)e * H * srow, (uint32_t)(H * srow));
#pragma unroll
    for (int f = 0; f < NF; ++f) p.so[f] = (n_wave + f * 16 + c) * (int)srow + 4 * (q >> 1);
    g_scale = gs[e];
  } else {
    const int64_t srow = I / 32;
    const int run = staged_bytes(16 * NF * (int)srow);
    stage_scales(w2_s + ((int64_t)e * H + n_wave) * srow, nullptr, 16 * NF * (int)srow, sS + wave * run, lane);
#pragma unroll
    for (int f = 0; f < NF; ++f) p.sl[f] = sS + wave * run + (f * 16 + c) * srow;
  }

  for (int m0 = it.y; m0 < it.y + item_rows && e_begin + m0 < e_end; m0 += kSmallRows) {
    const int row0 = e_begin + m0;
    const int mcount = min(kSmallRows, e_end - row0);
    const bool has = c < mcount;
    const int hrow = row0 + (has ? c : 0);
    p.xo = (hrow * I + 32 * q) * 2;
    v4f acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};
    stream16<NF, NV>(acc, p, KS, q);
    int ex[NF / 2];
#pragma unroll
    for (int b = 0; b < NF / 2; ++b) {
      float m = 0.f;
#pragma unroll
      for (int f = 2 * b; f < 2 * b + 2; ++f)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if constexpr (NV) acc[f][k] *= g_scale;
          m = fmaxf(m, fabsf(acc[f][k]));
        }
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      ex[b] = o_exponent(m);
    }
    if (has) {
      const int64_t slot = sorted_pairs[row0 + c];
      uint16_t* dst = o + slot * H + n_wave + q * 4;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const float inv = exp2_neg(ex[f / 2]);
        *reinterpret_cast<uint2*>(dst + f * 16) =
            f16_pack4(acc[f][0] * inv, acc[f][1] * inv, acc[f][2] * inv, acc[f][3] * inv);
      }
      if (q == 0) {
#pragma unroll
        for (int b = 0; b < NF / 2; ++b) os[slot * (H / 32) + n_wave / 32 + b] = (uint8_t)(ex[b] + 127);
      }
    }
  }
}

}  // namespace

hipError_t launch_w13_a16(const moe_dims& d, const SmallLists& lists, const int32_t* offsets,
                          const int32_t* sorted_pairs, const uint16_t* x, const uint8_t* w13, const uint8_t* w13_s,
                          const float* w13_gs, uint16_t* h, hipStream_t s) {
  const int64_t max_items = (int64_t)lists.cap0 + lists.cap1;
  if (max_items <= 0) return hipSuccess;
  const dim3 grid(d.I / 128, (unsigned)max_items);
  if (w13_gs && (int64_t)d.T * d.K > kNvWidePairs) {
    hipLaunchKernelGGL((k_w13_a16<true, 4>), grid, dim3(4 * 64), 0, s, lists, offsets, sorted_pairs, x, w13, w13_s,
                       w13_gs, h, d.H, d.I, d.K);
  } else if (w13_gs) {
    hipLaunchKernelGGL((k_w13_a16<true, kW13WavesNV>), grid, dim3(kW13WavesNV * 64), 0, s, lists, offsets,
                       sorted_pairs, x, w13, w13_s, w13_gs, h, d.H, d.I, d.K);
  } else {
    const size_t lds = (size_t)kW13Waves * 2 * staged_bytes(16 * (8 / kW13Waves) * (d.H / 32));
    hipLaunchKernelGGL((k_w13_a16<false, kW13Waves>), grid, dim3(kW13Waves * 64), lds, s, lists, offsets,
                       sorted_pairs, x, w13, w13_s, nullptr, h, d.H, d.I, d.K);
  }
  return hipGetLastError();
}

hipError_t launch_w2_a16(const moe_dims& d, const SmallLists& lists, const int32_t* offsets,
                         const int32_t* sorted_pairs, const uint16_t* h, const uint8_t* w2, const uint8_t* w2_s,
                         const float* w2_gs, uint16_t* o, uint8_t* os, hipStream_t s) {
  const int64_t max_items = (int64_t)lists.cap0 + lists.cap1;
  if (max_items <= 0) return hipSuccess;
  if (w2_gs && (int64_t)d.T * d.K > kNvWidePairs) {
    const dim3 grid((unsigned)ceil_div(d.H, 2 * 16 * 4), (unsigned)max_items);
    hipLaunchKernelGGL((k_w2_a16<true, 2, 4>), grid, dim3(2 * 64), 0, s, lists, offsets, sorted_pairs, h, w2, w2_s,
                       w2_gs, o, os, d.H, d.I);
  } else if (w2_gs) {
    const dim3 grid((unsigned)ceil_div(d.H, kW2WavesNV * 16 * kW2FragsNV), (unsigned)max_items);
    hipLaunchKernelGGL((k_w2_a16<true, kW2WavesNV, kW2FragsNV>), grid, dim3(kW2WavesNV * 64), 0, s, lists, offsets,
                       sorted_pairs, h, w2, w2_s, w2_gs, o, os, d.H, d.I);
  } else {
    const dim3 grid((unsigned)ceil_div(d.H, kW2Waves * 16 * kW2Frags), (unsigned)max_items);
    const size_t lds = (size_t)kW2Waves * staged_bytes(16 * kW2Frags * (d.I / 32));
    hipLaunchKernelGGL((k_w2_a16<false, kW2Waves, kW2Frags>), grid, dim3(kW2Waves * 64), lds, s, lists, offsets,
                       sorted_pairs, h, w2, w2_s, nullptr, o, os, d.H, d.I);
  }
  return hipGetLastError();
}

}  // namespace moe
