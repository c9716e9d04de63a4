// Device-side helpers shared by the gfx950 kernels: block-scaled MFMA operand
// types, FP8 E4M3 encoding, the E8M0 block-scale rule, bf16 rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Operand format selectors of v_mfma_scale_f32_*_f8f6f4 (cbsz / blgp fields).
constexpr int kFmtE4M3 = 0;
constexpr int kFmtE2M1 = 4;

// Lane layout of v_mfma_scale_f32_16x16x128_f8f6f4 on gfx950, lane l, q = l / 16:
//   A (16 x 128): row l % 16.  B (128 x 16): column l % 16.
//   8-bit operand: register bytes 0..15 hold K = 16q + i, bytes 16..31 hold
//     K = 64 + 16q + i (two 16-byte halves of the 128-long K step).
//   4-bit operand: the low 16 bytes hold K = 32q .. 32q+31, low nibble first.
//   scale operand (E8M0 in byte OPSEL of the VGPR): row/column l % 16, K block q
//     (K = 32q .. 32q+31).
//   D (16 x 16 fp32): column l % 16, rows 4q .. 4q+3.
//   OPSEL_A / OPSEL_B (0..3) pick which byte of the 32-bit scale operand is used.
template <int FMT_A, int FMT_B, int OPSEL_A = 0, int OPSEL_B = 0>
__device__ __forceinline__ v4f mfma_scale_16x16x128(v8i a, v8i b, v4f c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT_A, FMT_B, OPSEL_A, scale_a, OPSEL_B, scale_b);
}

// Smallest e with amax <= 448 * 2^e, from the fp32 bit pattern of amax >= 0:
// with amax = m * 2^p, m in [1, 2), e = p - 8 if m <= 1.75 else p - 7; zero and
// fp32 subnormals take the smallest E8M0 exponent, -127.
__device__ __forceinline__ int e8m0_exponent(float amax) {
  uint32_t b = __float_as_uint(amax) & 0x7FFFFFFFu;
  int be = (int)(b >> 23);
  int e = be - 127 - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  e = be == 0 ? -127 : e;
  return e < -127 ? -127 : e;
}

// 2^-e as a float, for e in [-127, 126].
__device__ __forceinline__ float exp2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// Four values to E4M3FN codes (byte i = code of value i): nearest, ties to even,
// sign kept for values that round to zero, for |v| <= 448 (callers scale by the
// block's E8M0 exponent first, which guarantees it). gfx950's v_cvt_pk_fp8_f32
// converts to the OCP E4M3 format and, measured over every fp32 pattern of
// magnitude <= 448 with both signs, gives exactly these codes (round to nearest
// even on the 3-bit mantissa in the normal range, on the 2^-9 grid below 2^-6).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Four E4M3 codes (byte i of `word`) times 2^e, as two packed bf16 pairs (code 0
// in the low half of the first). Exact when the values lie in bf16's range: an
// E4M3 value has at most 4 significant bits.
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t word, int e);

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ __forceinline__ float bf16_to_float(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t word, int e) {
  const int w = (int)word;
  const float v0 = __builtin_amdgcn_ldexpf(__builtin_amdgcn_cvt_f32_fp8(w, 0), e);
  const float v1 = __builtin_amdgcn_ldexpf(__builtin_amdgcn_cvt_f32_fp8(w, 1), e);
  const float v2 = __builtin_amdgcn_ldexpf(__builtin_amdgcn_cvt_f32_fp8(w, 2), e);
  const float v3 = __builtin_amdgcn_ldexpf(__builtin_amdgcn_cvt_f32_fp8(w, 3), e);
  return make_uint2((uint32_t)bf16_rne(v0) | ((uint32_t)bf16_rne(v1) << 16),
                    (uint32_t)bf16_rne(v2) | ((uint32_t)bf16_rne(v3) << 16));
}

// SiLU(g) * u = g * u / (1 + e^-g), with the hardware exp2 and reciprocal (about
// 1 ulp each): the result is requantized to E4M3 (3 mantissa bits), so fp32
// rounding of this order only moves values that sit on a rounding boundary. For
// g << 0, e^-g is +inf and the reciprocal 0, giving a signed zero.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Per-pair W2 outputs are stored as fp16 codes of o * 2^-e with one power-of-two
// scale 2^e per 32 columns (stored as the byte e + 127): e = floor(log2 amax) - 14,
// at least -127, so every scaled value is below 2^15 (the fp16 maximum is 65504)
// and values within 2^28 of the block's amax keep a relative error <= 2^-11.
__device__ __forceinline__ int o_exponent(float amax) {
  const int be = (int)((__float_as_uint(amax) & 0x7FFFFFFFu) >> 23);
  return be - 141 < -127 ? -127 : be - 141;
}

// Four floats to fp16 (round to nearest even), packed low to high.
__device__ __forceinline__ uint2 f16_pack4(float a, float b, float c, float d) {
  const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
  const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)c) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)d) << 16);
  return make_uint2(lo, hi);
}

// One row's 16 NF output columns held by a wave as NF fragments of 16 columns
// (lane (c, q) holds columns 16 i + 4 q .. +3 of its row in r[i]): fp16 codes to
// dst (the row's column 4 q) and the NF / 2 scale bytes of its 32-column blocks to
// sdst (by the q == 0 lanes). Every lane of the wave must call it (the amax goes
// through lane shuffles); `store` masks the writes.
template <int NF>
__device__ __forceinline__ void store_o_rows(const v4f (&r)[NF], bool store, uint16_t* dst, uint8_t* sdst, int q) {
  static_assert(NF == 4 || NF == 8, "64 or 128 columns");
  int ex[NF / 2];
#pragma unroll
  for (int b = 0; b < NF / 2; ++b) {
    float m = 0.f;
#pragma unroll
    for (int i = 2 * b; i < 2 * b + 2; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) m = fmaxf(m, fabsf(r[i][k]));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    ex[b] = o_exponent(m);
  }
  if (store) {
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const float inv = exp2_neg(ex[i >> 1]);
      *reinterpret_cast<uint2*>(dst + 16 * i) = f16_pack4(r[i][0] * inv, r[i][1] * inv, r[i][2] * inv, r[i][3] * inv);
    }
    if (q == 0) {
      if constexpr (NF == 8)
        *reinterpret_cast<uint32_t*>(sdst) = (uint32_t)(ex[0] + 127) | ((uint32_t)(ex[1] + 127) << 8) |
                                             ((uint32_t)(ex[2] + 127) << 16) | ((uint32_t)(ex[3] + 127) << 24);
      else
        *reinterpret_cast<uint16_t*>(sdst) = (uint16_t)((ex[0] + 127) | ((ex[1] + 127) << 8));
    }
  }
}
__device__ __forceinline__ void store_o_row128(const v4f (&r)[8], bool store, uint16_t* dst, uint8_t* sdst, int q) {
  store_o_rows<8>(r, store, dst, sdst, q);
}

__device__ __forceinline__ v4i load16(const void* p) { return *reinterpret_cast<const v4i*>(p); }
// 16 bytes read once per step (activations into the quantizer, per-pair rows into the
// combine), loaded with the nontemporal hint so that they do not displace reused lines.
__device__ __forceinline__ v4i load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

// Buffer loads: a wave-uniform resource (base, size in bytes, kept in SGPRs), a
// 32-bit per-lane offset and a wave-uniform offset. Reads past `bytes` return 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped) buffer access on gfx9-family

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
// POLICY: the instruction's cache-policy bits (0 = default; 16 = sc1, device-scope
// coherent, for data another workgroup of the same launch wrote with sc1 stores).
template <int POLICY = 0>
__device__ __forceinline__ v4i buf_load16(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POLICY));
}
// The same load with the nontemporal cache policy (the `nt` bit, cache-policy value
// 2 on gfx950): for data read once per step, such as the decode weight streams
// (measured on a stream of that shape: 6.0 -> 6.7 TB/s).
__device__ __forceinline__ v4i buf_load16_nt(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}
template <int POLICY = 0>
__device__ __forceinline__ int buf_load4(rsrc_t r, int voff, int soff) {
  return (int)__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, POLICY);
}
template <int POLICY = 0>
__device__ __forceinline__ int buf_load1(rsrc_t r, int voff, int soff) {
  return (int)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, POLICY);
}

}  // namespace moe
