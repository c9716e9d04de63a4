// Large-M grouped GEMMs (prefill shapes: experts with more routed rows than the
// small-M threshold), on the gfx950 block-scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4.
//
// Prefill routing spreads a 32K chunk unevenly over 384 experts, so per-expert M
// clusters on a few values and W13 and W2 have different shapes ("Pushing the
// Limits of Serving DeepSeek-V4-Pro", section 3.3); both are MFMA-bound here.
//
// Tile: 128 routed rows (one large work item from the planner) x 256 weight rows,
// full K, no split-K (ascending K, one accumulation order). Four waves in a 2x2
// grid; each wave owns 128 weight rows (8 fragments of 16) x 64 routed rows (4
// fragments), i.e. 32 accumulator tiles. The weights are the MFMA A side (E2M1,
// one E8M0 scale per 32 K), the routed rows the B side (E4M3, the per-128 scale).
//   W13: the 256 weight rows are gate rows [n0, n0+128) and up rows
//        [I+n0, I+n0+128); a wave's gate fragment i and up fragment i cover the same
//        16 h columns, so SwiGLU pairs registers of one lane, and the workgroup
//        sees whole 128-column scale blocks for the fused FP8 requantization (same
//        blog, section 4.3).
//   W2:  256 output columns; the epilogue writes fp32 rows to token-major slots.
//
// Data movement: the codes of each 128-K step are copied HBM -> LDS with
// direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds): a wave's load of one
// 16-row fragment lands in LDS in exactly the MFMA lane order (lane l's 16 bytes at
// l*16), so the LDS reads of the MFMA operands are conflict-free and no VGPRs
// stage the copy. Two LDS stages: the copy of step k+2 is issued as soon as step k
// has been consumed. The E8M0 scales of four K steps are fetched together through
// VGPRs one chunk ahead and stored to LDS.
#include "device_common.h"
#include "host_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokTile = kLargeRows;      // 128 routed rows per tile
constexpr int kAFrags = 16;               // 256 weight rows
constexpr int kBFrags = kTokTile / 16;    // 8 fragments of 16 routed rows
constexpr int kStageA = kAFrags * 1024;   // bytes of A codes per K step
constexpr int kStageB = kBFrags * 2048;   // bytes of B codes per K step
constexpr int kStages = 3;                // K steps of codes in flight in LDS
constexpr int kCodeDma = 4 + 4;           // direct-to-LDS code loads per wave per K step
constexpr int kMaxKS = 64;                // K steps whose activation scales fit the tile's LDS

typedef int v4i_s __attribute__((ext_vector_type(4)));

// Buffer resource as four SGPRs (base, stride 0, size, raw access) for inline asm.
__device__ __forceinline__ v4i_s rsrc4(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  v4i_s r;
  r[0] = (int)(uint32_t)b;
  r[1] = (int)(uint32_t)(b >> 32);
  r[2] = (int)bytes;
  r[3] = kRsrcWord3;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct-to-LDS buffer loads: lane l's data lands at M0 + l*size. Issued from
// inline asm so the compiler does not serialize later LDS reads against these
// writes; every use of the copied data is preceded by an explicit vmcnt wait and
// a barrier.
__device__ __forceinline__ void dma16(v4i_s r, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(r),
               "s"(soff)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(v4i_s r, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(r),
               "s"(soff)
               : "memory", "m0");
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

struct LargeArgs {
  const int2* items;
  const int32_t* n_items;
  const int32_t* offsets;
  const int32_t* sorted_pairs;
  const uint8_t* act;      // W13: x_q [T, H]; W2: h_q [P, I]
  const uint8_t* act_s;    // scales of act
  const uint8_t* w;        // W13 [E, 2I, H/2] or W2 [E, H, I/2]
  const uint8_t* w_s;
  uint8_t* h_q;            // W13 out
  uint8_t* h_s;
  float* o;                // W2 out
  int H, I, K;
};

template <bool W13>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_large(LargeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA[kStages][kStageA];
  __shared__ __attribute__((aligned(1024))) uint8_t sB[kStages][kStageB];
  __shared__ __attribute__((aligned(16))) uint32_t sSa[2][4][kAFrags * 16];   // [chunk buf][step][row]
  __shared__ __attribute__((aligned(16))) uint8_t sSb[kTokTile][kMaxKS];     // [row][step]
  __shared__ int sTok[kTokTile];
  __shared__ float sRed[2][kTokTile];

  const int item = blockIdx.y;
  if (item >= a.n_items[0]) return;
  const int2 it = a.items[item];
  const int e = it.x;
  const int e_begin = a.offsets[e], e_end = a.offsets[e + 1];
  const int row0 = e_begin + it.y;                      // first sorted row of the tile
  const int nrows = min(kTokTile, e_end - row0);
  const int nb = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  const int Kdim = W13 ? a.H : a.I;                     // reduction length
  const int N = W13 ? 2 * a.I : a.H;                    // weight rows per expert
  const int KS = Kdim / 128;
  const int wrow = Kdim / 2, srow = Kdim / 32, arow = Kdim;

  // routed rows of the tile -> activation row index (padding repeats the first row)
  if (tid < kTokTile) {
    const int r = row0 + (tid < nrows ? tid : 0);
    sTok[tid] = W13 ? a.sorted_pairs[r] / a.K : r;
  }
  __syncthreads();
  // activation scales of the whole tile (KS bytes per routed row): two threads per
  // row, 32 steps each, every load issued before the first LDS store
  {
    const int r = tid >> 1, s0 = (tid & 1) * (kMaxKS / 2);
    const uint8_t* src = a.act_s + (int64_t)sTok[r] * KS;
    uint32_t v[kMaxKS / 8];
#pragma unroll
    for (int i = 0; i < kMaxKS / 8; ++i) {
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int st = s0 + 4 * i + b;
        const uint32_t byte = src[min(st, KS - 1)];   // unconditional load, masked below
        w |= (st < KS ? byte : 0u) << (8 * b);
      }
      v[i] = w;
    }
#pragma unroll
    for (int i = 0; i < kMaxKS / 8; ++i) *reinterpret_cast<uint32_t*>(&sSb[r][s0 + 4 * i]) = v[i];
  }

  const v4i_s rw = rsrc4(a.w + (int64_t)e * N * wrow, (uint32_t)(N * wrow));
  const v4i_s rws = rsrc4(a.w_s + (int64_t)e * N * srow, (uint32_t)(N * srow));
  const v4i_s ra = rsrc4(a.act, 0xFFFFFFFFu);

  // weight row of LDS A fragment f (0..15)
  auto a_row = [&](int f) -> int {
    if (W13) return (f < 8 ? 0 : a.I) + nb * 128 + (f & 7) * 16;
    return nb * 256 + f * 16;
  };
  // this wave copies A fragments wave + 4i (i < 4) and B fragments wave + 4i (i < 2)
  int dA[4], dB[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) dA[i] = (a_row(wave + 4 * i) + c) * wrow + q * 16;
#pragma unroll
  for (int i = 0; i < 2; ++i) dB[i] = sTok[(wave + 4 * i) * 16 + c] * arow + q * 16;
  // A scales: lane l of this wave fetches LDS row wave*64 + l = fragment (wave*4 + l/16), row l%16
  const int dS = (a_row(wave * 4 + (lane >> 4)) + c) * srow;

  auto issue_codes = [&](int stage, int ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(rw, lds_addr(&sA[stage][(wave + 4 * i) * 1024]), dA[i], ks * 64);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      dma16(ra, lds_addr(&sB[stage][(wave + 4 * i) * 2048]), dB[i], ks * 128);
      dma16(ra, lds_addr(&sB[stage][(wave + 4 * i) * 2048 + 1024]), dB[i], ks * 128 + 64);
    }
  };
  auto issue_scales = [&](int chunk) {   // E8M0 dwords of steps 4*chunk .. 4*chunk+3
#pragma unroll
    for (int d = 0; d < 4; ++d)
      dma4(rws, lds_addr(&sSa[chunk & 1][d][wave * 64]), dS, min(4 * chunk + d, KS - 1) * 4);
  };

  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // LDS A fragments this wave multiplies
  int fA[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) fA[i] = W13 ? (i < 4 ? 4 * wn + i : 8 + 4 * wn + (i - 4)) : 8 * wn + i;

  auto compute = [&](int stage, int ks) {
    const int cb = (ks >> 2) & 1, d = ks & 3;
    v8i bop[4];
    int sbv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int fb = 4 * wm + j;
      const v4i lo = *reinterpret_cast<const v4i*>(&sB[stage][fb * 2048 + lane * 16]);
      const v4i hi = *reinterpret_cast<const v4i*>(&sB[stage][fb * 2048 + 1024 + lane * 16]);
      bop[j][0] = lo[0]; bop[j][1] = lo[1]; bop[j][2] = lo[2]; bop[j][3] = lo[3];
      bop[j][4] = hi[0]; bop[j][5] = hi[1]; bop[j][6] = hi[2]; bop[j][7] = hi[3];
      sbv[j] = sSb[fb * 16 + c][ks];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const v4i w4 = *reinterpret_cast<const v4i*>(&sA[stage][fA[i] * 1024 + lane * 16]);
      v8i aop;
      aop[0] = w4[0]; aop[1] = w4[1]; aop[2] = w4[2]; aop[3] = w4[3];
      aop[4] = 0; aop[5] = 0; aop[6] = 0; aop[7] = 0;
      const int sav = (int)(sSa[cb][d][fA[i] * 16 + c] >> (8 * q));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = mfma_scale_16x16x128<kFmtE2M1, kFmtE4M3>(aop, bop[j], acc[i][j], sav, sbv[j]);
    }
  };

  // prologue: scales of chunk 0, codes of steps 0 .. kStages-1
  issue_scales(0);
#pragma unroll
  for (int s = 0; s < kStages; ++s)
    if (s < KS) issue_codes(s, s);

  // Step ks waits for its codes; the only later loads are the codes of the (up to
  // two) following steps and possibly a scale chunk, which makes the wait stricter.
  for (int ks0 = 0; ks0 < KS; ks0 += kStages) {
#pragma unroll
    for (int st = 0; st < kStages; ++st) {
      const int ks = ks0 + st;
      if (ks < KS) {
        if (ks + 2 < KS) wait_vmcnt<2 * kCodeDma>();
        else if (ks + 1 < KS) wait_vmcnt<kCodeDma>();
        else wait_vmcnt<0>();
        __syncthreads();
        compute(st, ks);
        __syncthreads();
        if ((ks & 3) == 0) issue_scales((ks >> 2) + 1);
        if (ks + kStages < KS) issue_codes(st, ks + kStages);
      }
    }
  }
  wait_vmcnt<0>();

  if (W13) {
    // SwiGLU + FP8 requantization. Lane (c, q) of token fragment j holds h columns
    // 16i + 4q .. 16i + 4q + 3 (i = 0..3, gate acc[i], up acc[4+i]) of this wave's 64
    // h columns, for tile row 64*wm + 16j + c.
    float amax[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float h = silu_mul(acc[i][j][r], acc[4 + i][j][r]);
          acc[i][j][r] = h;
          m = fmaxf(m, fabsf(h));
        }
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      amax[j] = m;
    }
    if (q == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sRed[wn][64 * wm + 16 * j + c] = amax[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 64 * wm + 16 * j + c;
      const float m = fmaxf(sRed[0][row], sRed[1][row]);
      const int ex = e8m0_exponent(m);
      const float inv = exp2_neg(ex);
      if (row < nrows) {
        uint8_t* dst = a.h_q + (int64_t)(row0 + row) * a.I + nb * 128 + 64 * wn + q * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t packed = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) packed |= e4m3_encode(acc[i][j][r] * inv) << (8 * r);
          *reinterpret_cast<uint32_t*>(dst + 16 * i) = packed;
        }
        if (wn == 0 && q == 0) a.h_s[(int64_t)(row0 + row) * (a.I / 128) + nb] = (uint8_t)(ex + 127);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 64 * wm + 16 * j + c;
      if (row < nrows) {
        const int64_t slot = a.sorted_pairs[row0 + row];
        float* dst = a.o + slot * a.H + nb * 256 + 128 * wn + q * 4;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<float4*>(dst + 16 * i) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    }
  }
}

}  // namespace

// The large-M kernels need whole 256-column W2 tiles and the tile's activation
// scales in LDS (at most kMaxKS K steps for both GEMMs).
bool large_path_supported(const moe_dims& d) {
  return d.H % 256 == 0 && d.H / 128 <= kMaxKS && d.I / 128 <= kMaxKS;
}

hipError_t launch_w13_large(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                            const int32_t* offsets, const int32_t* sorted_pairs, const uint8_t* x_q,
                            const uint8_t* x_s, const uint8_t* w13, const uint8_t* w13_s, uint8_t* h_q,
                            uint8_t* h_s, hipStream_t s) {
  if (max_items <= 0) return hipSuccess;
  LargeArgs a{items, n_items, offsets, sorted_pairs, x_q, x_s, w13, w13_s, h_q, h_s, nullptr, d.H, d.I, d.K};
  hipLaunchKernelGGL(k_gemm_large<true>, dim3(d.I / 128, (unsigned)max_items), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_w2_large(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                           const int32_t* offsets, const int32_t* sorted_pairs, const uint8_t* h_q,
                           const uint8_t* h_s, const uint8_t* w2, const uint8_t* w2_s, float* o, hipStream_t s) {
  if (max_items <= 0) return hipSuccess;
  LargeArgs a{items, n_items, offsets, sorted_pairs, h_q, h_s, w2, w2_s, nullptr, nullptr, o, d.H, d.I, d.K};
  hipLaunchKernelGGL(k_gemm_large<false>, dim3(d.H / 256, (unsigned)max_items), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
