// Test support (not part of the product library): runs single gfx950 MFMA
// instructions on caller-built register images, so that tests can check the
// hardware's dot-product arithmetic against exact sums on the host.
//
// Each wave w of a launch executes ONE MFMA on its own operands:
//   a, b   [waves][64 lanes][8] int32   operand register images (lane-major)
//   sa, sb [waves][64]          int32   E8M0 scale operands (byte 0 used; scaled form only)
//   c      [waves][64][4]       float   accumulator input
//   d      [waves][64][4]       float   result
// The caller lays values out in the instruction's lane order; nothing here
// interprets them. probe_cvt_fp4_bf16 runs gfx950's scaled FP4 -> bf16 conversion
// on n words (one thread per word, guarded by n); probe_cvt_fp4_f32 its
// fp32-output form. Every pointer is a device pointer; `waves` >= 1; the launch
// is one 64-lane workgroup per wave, so every access stays inside the arrays.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace {

// Format codes of the scaled MFMA's cbsz (A) / blgp (B) fields.
constexpr int kE4M3 = 0, kE2M1 = 4;

template <int FA, int FB>
__global__ __launch_bounds__(64) void k_scaled(const int* __restrict__ a, const int* __restrict__ b,
                                               const int* __restrict__ sa, const int* __restrict__ sb,
                                               const float* __restrict__ c, float* __restrict__ d) {
  const int w = blockIdx.x, l = threadIdx.x;
  const int64_t r = (int64_t)w * 64 + l;
  v8i A, B;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    A[i] = a[r * 8 + i];
    B[i] = b[r * 8 + i];
  }
  v4f C = {c[r * 4 + 0], c[r * 4 + 1], c[r * 4 + 2], c[r * 4 + 3]};
  v4f D = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, C, FA, FB, 0, sa[r], 0, sb[r]);
#pragma unroll
  for (int i = 0; i < 4; ++i) d[r * 4 + i] = D[i];
}

__global__ __launch_bounds__(64) void k_bf16(const int* __restrict__ a, const int* __restrict__ b,
                                             const float* __restrict__ c, float* __restrict__ d) {
  const int w = blockIdx.x, l = threadIdx.x;
  const int64_t r = (int64_t)w * 64 + l;
  v8i A, B;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    A[i] = a[r * 8 + i];
    B[i] = b[r * 8 + i];
  }
  v8bf Ab = __builtin_bit_cast(v8bf, (int __attribute__((ext_vector_type(4)))){A[0], A[1], A[2], A[3]});
  v8bf Bb = __builtin_bit_cast(v8bf, (int __attribute__((ext_vector_type(4)))){B[0], B[1], B[2], B[3]});
  v4f C = {c[r * 4 + 0], c[r * 4 + 1], c[r * 4 + 2], c[r * 4 + 3]};
  v4f D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ab, Bb, C, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) d[r * 4 + i] = D[i];
}

__global__ __launch_bounds__(64) void k_cvt_fp4_bf16(const uint32_t* __restrict__ w, const float* __restrict__ sc,
                                                     uint32_t* __restrict__ out, int n) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= n) return;
  const uint32_t v = w[i];
  const float s = sc[i];
  out[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 0));
  out[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 1));
  out[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 2));
  out[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 3));
}

__global__ __launch_bounds__(64) void k_cvt_fp4_f32(const uint32_t* __restrict__ w, const float* __restrict__ sc,
                                                    float* __restrict__ out, int n) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= n) return;
  const uint32_t v = w[i];
  const float s = sc[i];
  typedef float v2f __attribute__((ext_vector_type(2)));
  const v2f r0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, s, 0);
  const v2f r1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, s, 1);
  const v2f r2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, s, 2);
  const v2f r3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, s, 3);
  out[8 * i + 0] = r0[0];
  out[8 * i + 1] = r0[1];
  out[8 * i + 2] = r1[0];
  out[8 * i + 3] = r1[1];
  out[8 * i + 4] = r2[0];
  out[8 * i + 5] = r2[1];
  out[8 * i + 6] = r3[0];
  out[8 * i + 7] = r3[1];
}

}  // namespace

extern "C" {

// v_mfma_scale_f32_16x16x128_f8f6f4 with A format fmt_a and B format fmt_b
// (0 = E4M3, 4 = E2M1; other values return -1). Returns 0 or the HIP error code.
int probe_mfma_scaled(int fmt_a, int fmt_b, const int* a, const int* b, const int* sa, const int* sb,
                      const float* c, float* d, int waves, void* stream) {
  if (waves < 1) return -1;
  hipStream_t s = (hipStream_t)stream;
  if (fmt_a == kE2M1 && fmt_b == kE4M3)
    hipLaunchKernelGGL((k_scaled<kE2M1, kE4M3>), dim3(waves), dim3(64), 0, s, a, b, sa, sb, c, d);
  else if (fmt_a == kE4M3 && fmt_b == kE4M3)
    hipLaunchKernelGGL((k_scaled<kE4M3, kE4M3>), dim3(waves), dim3(64), 0, s, a, b, sa, sb, c, d);
  else if (fmt_a == kE2M1 && fmt_b == kE2M1)
    hipLaunchKernelGGL((k_scaled<kE2M1, kE2M1>), dim3(waves), dim3(64), 0, s, a, b, sa, sb, c, d);
  else
    return -1;
  return (int)hipGetLastError();
}

// v_mfma_f32_16x16x32_bf16: a and b carry 8 bf16 per lane in ints 0..3 of each
// lane's 8-int slot (ints 4..7 unused).
int probe_mfma_bf16(const int* a, const int* b, const float* c, float* d, int waves, void* stream) {
  if (waves < 1) return -1;
  hipLaunchKernelGGL(k_bf16, dim3(waves), dim3(64), 0, (hipStream_t)stream, a, b, c, d);
  return (int)hipGetLastError();
}

// v_cvt_scalef32_pk_bf16_fp4 on words[i] with scales[i], byte selects 0..3:
// out[4i + k] = the two bf16 of byte k (n >= 0 words; device pointers).
int probe_cvt_fp4_bf16(const uint32_t* words, const float* scales, uint32_t* out, int n, void* stream) {
  if (n < 0) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_cvt_fp4_bf16, dim3((n + 63) / 64), dim3(64), 0, (hipStream_t)stream, words, scales, out, n);
  return (int)hipGetLastError();
}

// v_cvt_scalef32_pk_f32_fp4 on words[i] with scales[i]: out[8i + 2k + h] = value
// h (0 = low nibble) of byte k.
int probe_cvt_fp4_f32(const uint32_t* words, const float* scales, float* out, int n, void* stream) {
  if (n < 0) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_cvt_fp4_f32, dim3((n + 63) / 64), dim3(64), 0, (hipStream_t)stream, words, scales, out, n);
  return (int)hipGetLastError();
}

}  // extern "C"
