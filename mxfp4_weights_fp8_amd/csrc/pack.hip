// Kernel-native layout of MXFP4 expert weights (a one-time conversion when the
// weights are loaded).
//
// Row-major E2M1 codes w[R][K/2] (R rows of K weights, two per byte) become
// blocks of 16 rows x 128 K: block (g, s) covers rows 16g .. 16g+15 and code bytes
// 64s .. 64s+63 of each row and is 1 KB at offset g * 16 * K/2 + s * 1024; inside a
// block, byte 16 * (16q + c) + b is w[16g + c][64s + 16q + b]. That is the order in
// which the 64 lanes of a wave hold a 16-row weight fragment of one 128-K step on
// v_mfma_scale_f32_16x16x128_f8f6f4 (lane 16q + c: row c, 32 codes of K block q),
// so one 16-byte-per-lane load or copy moves a whole fragment as 1 KB of
// consecutive bytes (full cache lines, one stream per fragment).
#include "device_common.h"
#include "host_internal.h"

namespace moe {
namespace {

// one thread per 16-byte chunk of the output
__global__ __launch_bounds__(256) void k_pack_weights(const uint4* __restrict__ w, uint4* __restrict__ out,
                                                      int64_t n_chunks, int kb) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_chunks) return;
  const int64_t block = i >> 6;                 // 64 chunks of 16 bytes per 1 KB block
  const int lane = (int)(i & 63), q = lane >> 4, c = lane & 15;
  const int steps = kb / 64;                    // 128-K steps per row
  const int64_t g = block / steps;
  const int s = (int)(block - g * steps);
  const int64_t src = ((16 * g + c) * kb + 64 * s + 16 * q) / 16;
  out[i] = w[src];
}

}  // namespace

hipError_t launch_pack_weights(const uint8_t* w, uint8_t* out, int64_t rows, int K, hipStream_t s) {
  const int64_t n_chunks = rows * (K / 2) / 16;
  if (n_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_weights, dim3((unsigned)ceil_div(n_chunks, 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(w), reinterpret_cast<uint4*>(out), n_chunks, K / 2);
  return hipGetLastError();
}

}  // namespace moe
