// Dense FP8 x FP8 GEMMs of the shared expert ("Pushing the Limits of Serving
// DeepSeek-V4-Pro", section 3.3: a dense SwiGLU FFN whose output is added to the
// routed sum with weight 1), on the gfx950 block-scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E4M3.
//
// The weights carry one E8M0 scale per 128 x 128 block; a 16-row MFMA fragment
// lies inside one 128-row block, so its scale operand is the block's byte for
// the K step, the same in every lane. The activations (x codes, or the SwiGLU
// codes of W13s for W2s) carry one scale per token and 128 columns.
//
// Tile: 128 token rows x 256 weight rows, full K, ascending K steps. Four waves in
// a 2 x 2 grid, each 128 weight rows (8 fragments) x 64 tokens (4 fragments).
//   W13s: weight rows = gate rows [n0, n0+128) and up rows [Is+n0, Is+n0+128);
//         the epilogue applies SwiGLU and requantizes each token's 128 h columns
//         to E4M3 with one E8M0 scale (same blog, section 4.3).
//   W2s:  256 output columns, rows [T, H] for the combine (fp16 codes with one
//         power-of-two scale per 32 columns, as the routed per-pair rows); when H is an odd
//         multiple of 128 the last tile's second half reads zeros and is not stored.
//
// Data movement: three one-step LDS stages (32 KB of weight codes + 16 KB of
// activation codes each), filled by direct-to-LDS copies of 8 rows x 128 B per
// instruction, rows XOR-swizzled by (row / 2) % 8 in 16-byte chunks. The copy of
// step k+3 is issued while step k is multiplied, so two steps of copies are in
// flight. The K-step count is padded to even with a step of zeros (exact: the
// MFMA adds zero products).
//
// W13s in bf16 (the form moe_ffn runs). The block-scaled MFMA sums the products of
// a 32-element block after truncating each to 13 fraction bits below the block's
// largest exponent sum; with FP8 x FP8 operands (up to 8 significant bits per
// product, wide dynamic range inside a block) that moves gate/up values by about
// 1e-5 of their size and changed 0.1-0.2% of the SwiGLU codes. Every dequantized
// E4M3 value (code x power-of-two scale) is exact in bf16, and the bf16 MFMA keeps
// 24 fraction bits (about 1e-7 relative on the same dots), so the gate/up GEMM
// runs on v_mfma_f32_16x16x32_bf16 over operands expanded to bf16 once per call:
// the weights with their block scale folded in, the activations written by the
// quantizer. A 128-byte LDS row of a stage then holds 64 K; lane (c, q) reads the
// chunks q and 4 + q of its row, which are exactly the bf16 instruction's K
// 8q .. 8q+7 of the stage's first and second 32 K. Costs twice the MFMA time of
// the FP8 form (0.36 TFLOP at 32K tokens, Is 384).
#include "device_common.h"
#include "host_internal.h"
#include "lds_copy.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokRows = 128;             // token rows per tile
constexpr int kWRows = 256;               // weight rows per tile
constexpr int kBufs = 3;                  // one-step LDS stages
constexpr int kStageA = kWRows * 128;     // weight codes per step
constexpr int kStageB = kTokRows * 128;   // activation codes per step
constexpr int kCopies = 12;               // direct-to-LDS copies per wave per step (8 weight + 4 activation)
constexpr int kMaxSteps = 64;             // K steps whose scales fit the tile's LDS tables
constexpr int kSbRow = kMaxSteps + 4;     // activation-scale row stride (17 dwords: distinct banks)

struct DenseArgs {
  const uint8_t* act;      // W13s: x_q [T, H] (bf16 form: x_hat [T, H] bf16); W2s: sh_q [T, Is]
  const uint8_t* act_s;    // [T, Kd/128] (unused in the bf16 form)
  const uint8_t* w;        // [N, Kd] E4M3 (bf16 form: [N, Kd] bf16, scales folded in)
  const uint8_t* w_s;      // [N/128, Kd/128] E8M0 (unused in the bf16 form)
  uint8_t* h_q;            // W13s out [T, Is]
  uint8_t* h_s;            // [T, Is/128]
  uint16_t* o;             // W2s out [T, N]: fp16 codes
  uint8_t* os;             // and their 32-column scales [T, N/32]
  uint32_t act_bytes, w_bytes;
  int T, Kd, N, Is;
};

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4f mfma_bf16_16x16x32(const v4i a, const v4i b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

template <bool W13, bool BF16 = false>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_dense(DenseArgs a) {
  static_assert(W13 || !BF16, "the bf16 form is the gate/up GEMM");
  __shared__ __attribute__((aligned(1024))) uint8_t sA[kBufs][kStageA];   // [buf][row][128 B]
  __shared__ __attribute__((aligned(1024))) uint8_t sB[kBufs][kStageB];
  __shared__ __attribute__((aligned(16))) uint8_t sSb[kTokRows][kSbRow];  // [row][step]
  __shared__ __attribute__((aligned(16))) uint8_t sSw[2][kMaxSteps];      // [128-row block][step]
  __shared__ float sRed[2][kTokRows];

  const int nb = blockIdx.x;
  const int t0 = blockIdx.y * kTokRows;
  const int nrows = min(kTokRows, a.T - t0);
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int row_bytes = BF16 ? 2 * a.Kd : a.Kd;      // one operand row in global memory
  const int KS = row_bytes / 128;                     // 128-byte LDS steps (bf16: 64 K each)
  const int KSp = (KS + 1) & ~1;                      // padded to even with a zero step

  // first weight row of each 128-row half of the tile
  const int wbase0 = W13 ? nb * 128 : nb * 256;
  const int wbase1 = W13 ? a.Is + nb * 128 : nb * 256 + 128;

  // scale tables: activation scales of the tile's tokens (padding rows repeat the
  // last valid token; steps past the last read as 2^-127), weight block scales of
  // the two 128-row halves (a half past N reads 2^-127)
  if constexpr (!BF16) {
    const int r = tid >> 1, s0 = (tid & 1) * (kMaxSteps / 2);
    const uint8_t* src = a.act_s + (int64_t)(t0 + min(r, nrows - 1)) * KS;
    uint32_t v[kMaxSteps / 8];
#pragma unroll
    for (int i = 0; i < kMaxSteps / 8; ++i) {
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int st = s0 + 4 * i + b;
        const uint32_t byte = src[min(st, KS - 1)];
        w |= (st < KS ? byte : 0u) << (8 * b);
      }
      v[i] = w;
    }
#pragma unroll
    for (int i = 0; i < kMaxSteps / 8; ++i) *reinterpret_cast<uint32_t*>(&sSb[r][s0 + 4 * i]) = v[i];
    if (tid < 2 * kMaxSteps) {
      const int h = tid / kMaxSteps, st = tid % kMaxSteps;
      const int blk = (h ? wbase1 : wbase0) / 128;
      const bool ok = st < KS && blk < a.N / 128;
      sSw[h][st] = ok ? a.w_s[(int64_t)blk * KS + st] : 0;
    }
  }

  const v4i_s rw = rsrc4(a.w, a.w_bytes);
  const v4i_s ra = rsrc4(a.act, a.act_bytes);
  // Copy plan (per wave, per step): weight LDS rows 64*wave + 8i + l/8 (i < 8),
  // token LDS rows 32*wave + 8i + l/8 (i < 4); lane l's physical chunk l%8 holds
  // logical chunk (l%8) ^ s(row), s(row) = (row / 2) % 8 = 4 (i % 2) + l / 16.
  // A wave's 64 weight rows are consecutive rows of one half (gate/up or W2s
  // columns), so instruction i adds 8i rows to one lane offset.
  const int sw0 = ((lane & 7) ^ (lane >> 4)) << 4;
  const int sw1 = ((lane & 7) ^ (4 | (lane >> 4))) << 4;
  const int wrow_lane = (wave < 2 ? wbase0 : wbase1) + 64 * (wave & 1) + (lane >> 3);
  const int dA = wrow_lane * row_bytes;
  int dB[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    dB[i] = (t0 + min(32 * wave + 8 * i + (lane >> 3), nrows - 1)) * row_bytes + ((i & 1) ? sw1 : sw0);

  // copy instructions of step st into buffer buf, 3 per part (parts 0..3: weight
  // 2p, 2p+1 and activation p), so they spread over the MFMA groups
  auto issue_part = [&](int buf, int st, int p) {
    const bool valid = st < KS;
#pragma unroll
    for (int i = 2 * p; i < 2 * p + 2; ++i)
      dma16(rsrc_sized(rw, valid), lds_addr(&sA[buf][(64 * wave + 8 * i) * 128]),
            dA + 8 * i * row_bytes + ((i & 1) ? sw1 : sw0) + st * 128, 0);
    dma16(rsrc_sized(ra, valid), lds_addr(&sB[buf][(32 * wave + 8 * p) * 128]), dB[p] + st * 128, 0);
  };

  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // operand reads: a fragment row (16f + c) has swizzle (c / 2) % 8; the lane's two
  // 16-byte chunks (K 16q.. and 64+16q..) sit at fixed per-lane offsets
  const int off0 = c * 128 + ((q ^ (c >> 1)) << 4);
  const int off1 = c * 128 + (((4 + q) ^ (c >> 1)) << 4);
  // this wave's weight fragments: W13s gate 4wn..4wn+3 (half 0), up 8+4wn.. (half 1);
  // W2s 8wn..8wn+7 (half wn)
  auto a_frag = [&](int i) { return W13 ? (i < 4 ? 4 * wn + i : 8 + 4 * wn + (i - 4)) : 8 * wn + i; };
  const uint8_t* pA0 = &sA[0][0] + off0;
  const uint8_t* pA1 = &sA[0][0] + off1;
  const uint8_t* pB0 = &sB[0][0] + wm * 4 * 2048 + off0;
  const uint8_t* pB1 = &sB[0][0] + wm * 4 * 2048 + off1;
  const uint8_t* pSb = &sSb[0][0] + (wm * 4 * 16 + c) * kSbRow;

  struct Ops {
    v8i w[8];
    v8i b[4];
    int sw[2];
    int sb[4];
  };
  // 8 parts: p < 4 token fragment p; p >= 4 weight fragments 2(p-4), 2(p-4)+1
  auto load_part = [&](Ops& o, int buf, int st, int p) {
    if (p < 4) {
      const int ob = buf * kStageB + p * 2048;
      const v4i lo = *reinterpret_cast<const v4i*>(pB0 + ob);
      const v4i hi = *reinterpret_cast<const v4i*>(pB1 + ob);
      o.b[p][0] = lo[0]; o.b[p][1] = lo[1]; o.b[p][2] = lo[2]; o.b[p][3] = lo[3];
      o.b[p][4] = hi[0]; o.b[p][5] = hi[1]; o.b[p][6] = hi[2]; o.b[p][7] = hi[3];
      if constexpr (!BF16) {
        o.sb[p] = pSb[st + p * 16 * kSbRow];
        if (p == 0) {
          o.sw[0] = sSw[W13 ? 0 : wn][st];
          o.sw[1] = sSw[W13 ? 1 : wn][st];
        }
      }
    } else {
#pragma unroll
      for (int i = 2 * (p - 4); i < 2 * (p - 4) + 2; ++i) {
        const int oa = buf * kStageA + a_frag(i) * 2048;
        const v4i lo = *reinterpret_cast<const v4i*>(pA0 + oa);
        const v4i hi = *reinterpret_cast<const v4i*>(pA1 + oa);
        o.w[i][0] = lo[0]; o.w[i][1] = lo[1]; o.w[i][2] = lo[2]; o.w[i][3] = lo[3];
        o.w[i][4] = hi[0]; o.w[i][5] = hi[1]; o.w[i][6] = hi[2]; o.w[i][7] = hi[3];
      }
    }
  };
  auto mma_row = [&](const Ops& o, int i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (BF16) {
        // K 0..31 of the stage (ints 0..3 of each operand), then K 32..63
        acc[i][j] = mfma_bf16_16x16x32(v4i{o.w[i][0], o.w[i][1], o.w[i][2], o.w[i][3]},
                                       v4i{o.b[j][0], o.b[j][1], o.b[j][2], o.b[j][3]}, acc[i][j]);
        acc[i][j] = mfma_bf16_16x16x32(v4i{o.w[i][4], o.w[i][5], o.w[i][6], o.w[i][7]},
                                       v4i{o.b[j][4], o.b[j][5], o.b[j][6], o.b[j][7]}, acc[i][j]);
      } else {
        acc[i][j] = mfma_scale_16x16x128<kFmtE4M3, kFmtE4M3>(o.w[i], o.b[j], acc[i][j], o.sw[i < 4 ? 0 : 1], o.sb[j]);
      }
    }
  };

  // Prologue: copies of steps 0..2, operands of step 0.
  __syncthreads();
#pragma unroll
  for (int b = 0; b < kBufs; ++b)
#pragma unroll
    for (int p = 0; p < 4; ++p) issue_part(b, b, p);
  wait_vmcnt<2 * kCopies>();
  __syncthreads();
  Ops opsA, opsB;
#pragma unroll
  for (int p = 0; p < 8; ++p) load_part(opsA, 0, 0, p);

  // Step k (buffer k % 3), operands in `cur`: wait for this wave's copies of step
  // k+1 (the newest 12 loads are step k+2's) and barrier: step k+1 is in LDS and
  // every wave has read step k's buffer. Then 8 groups of (4 MFMAs of step k, one
  // operand part of step k+1, copies of step k+3 into step k's buffer in parts
  // 0..3), separated by scheduling barriers. The loop body has no branches.
  auto step = [&](Ops& cur, Ops& nxt, int k) {
    const int buf = k % kBufs, nbuf = (k + 1) % kBufs;
    wait_vmcnt<kCopies>();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      mma_row(cur, p);
      load_part(nxt, nbuf, min(k + 1, KSp - 1), p);
      if (p < 4) issue_part(buf, k + 3, p);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int k = 0; k < KSp; k += 2) {
    step(opsA, opsB, k);
    step(opsB, opsA, k + 1);
  }
  wait_vmcnt<0>();

  if (W13) {
    // SwiGLU + FP8 requantization: lane (c, q) of token fragment j holds h columns
    // 16i + 4q .. +3 (gate acc[i], up acc[4+i], i < 4) of this wave's 64 columns.
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
        uint8_t* dst = a.h_q + (int64_t)(t0 + row) * a.Is + nb * 128 + 64 * wn + q * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *reinterpret_cast<uint32_t*>(dst + 16 * i) =
              e4m3_pack4(acc[i][j][0] * inv, acc[i][j][1] * inv, acc[i][j][2] * inv, acc[i][j][3] * inv);
        }
        if (wn == 0 && q == 0) a.h_s[(int64_t)(t0 + row) * (a.Is / 128) + nb] = (uint8_t)(ex + 127);
      }
    }
  } else {
    const int col0 = nb * 256 + 128 * wn;
    if (col0 < a.N) {   // wave-uniform
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 64 * wm + 16 * j + c;
        const int64_t t = t0 + (row < nrows ? row : 0);
        v4f r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = acc[i][j];
        store_o_row128(r, row < nrows, a.o + t * a.N + col0 + q * 4, a.os + t * (a.N / 32) + col0 / 32, q);
      }
    }
  }
}

// FP8 E4M3 codes with one E8M0 scale per 128 x 128 block -> bf16 values with the
// scale folded in: w[n][k] = E4M3(code) * 2^(scale - 127). Exact while the value
// stays inside bf16's range (block scales 2^-124 .. 2^119). One thread per 8
// consecutive codes.
__global__ __launch_bounds__(256) void k_fp8_block_to_bf16(const uint8_t* __restrict__ w,
                                                            const uint8_t* __restrict__ w_s,
                                                            uint16_t* __restrict__ out, int64_t n8, int Kd) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= n8) return;
  const int64_t e0 = g * 8;
  const int64_t n = e0 / Kd;
  const int k = (int)(e0 - n * Kd);
  const int ex = (int)w_s[(n / 128) * (Kd / 128) + k / 128] - 127;
  const uint2 c = *reinterpret_cast<const uint2*>(w + e0);
  const uint2 lo = e4m3x4_to_bf16(c.x, ex), hi = e4m3x4_to_bf16(c.y, ex);
  const uint32_t r[4] = {lo.x, lo.y, hi.x, hi.y};
  *reinterpret_cast<uint4*>(out + e0) = make_uint4(r[0], r[1], r[2], r[3]);
}

}  // namespace

bool dense_path_supported(const moe_dims& d) { return d.H / 128 <= kMaxSteps && d.Is / 128 <= kMaxSteps; }

hipError_t launch_shared13_bf16(const moe_dims& d, const uint16_t* x_hat, const uint8_t* w13s, const uint8_t* w13s_s,
                                uint16_t* w13s_bf16, uint8_t* sh_q, uint8_t* sh_s, hipStream_t s) {
  const int64_t n8 = (int64_t)2 * d.Is * d.H / 8;
  hipLaunchKernelGGL(k_fp8_block_to_bf16, dim3((unsigned)ceil_div(n8, 256)), dim3(256), 0, s, w13s, w13s_s, w13s_bf16,
                     n8, d.H);
  DenseArgs a{reinterpret_cast<const uint8_t*>(x_hat), nullptr, reinterpret_cast<const uint8_t*>(w13s_bf16), nullptr,
              sh_q, sh_s, nullptr, nullptr,
              (uint32_t)((int64_t)d.T * d.H * 2), (uint32_t)((int64_t)2 * d.Is * d.H * 2), d.T, d.H, 2 * d.Is, d.Is};
  hipLaunchKernelGGL((k_gemm_dense<true, true>), dim3(d.Is / 128, (unsigned)ceil_div(d.T, kTokRows)), dim3(kThreads),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_shared2(const moe_dims& d, const uint8_t* sh_q, const uint8_t* sh_s, const uint8_t* w2s,
                          const uint8_t* w2s_s, uint16_t* so, uint8_t* sos, hipStream_t s) {
  DenseArgs a{sh_q, sh_s, w2s, w2s_s, nullptr, nullptr, so, sos,
              (uint32_t)((int64_t)d.T * d.Is), (uint32_t)((int64_t)d.H * d.Is), d.T, d.Is, d.H, d.Is};
  hipLaunchKernelGGL(k_gemm_dense<false>, dim3((unsigned)ceil_div(d.H, kWRows), (unsigned)ceil_div(d.T, kTokRows)),
                     dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
