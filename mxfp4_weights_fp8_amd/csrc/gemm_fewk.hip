// W2 grouped GEMM for a short reduction: I <= 384, at most three 128-K steps, as
// in one MoE-TP8 rank's share of the expert intermediate ("Pushing the Limits of
// Serving DeepSeek-V4-Pro", section 3.1: MoE-TP splits the 3072 intermediate
// columns of every expert 8 ways, 384 per rank).
//
// With so few K steps, a 128-row x 256-column workgroup of the large-M kernel
// spends most of its time on its own prologue (routed-row tile, scales, first
// copies) and epilogue, and with one such workgroup per CU the MFMAs and the
// epilogue of all four waves run one after the other. Here a workgroup owns 128
// routed rows and walks a run of 128-column blocks of W2: each wave keeps its 4
// routed-row fragments of every K step in registers (read once from memory), the
// E2M1 codes and E8M0 scales of block b+1 are copied into the other half of a
// double buffer while block b is multiplied and written, and the footprint (about
// 69 KB of LDS, 226 VGPRs at three K steps) lets two workgroups share a CU.
//
// Waves: a 2 x 2 grid, wave (wm, wn) = routed rows [64 wm, +64) (4 fragments, MFMA
// B side, E4M3) x output columns [64 wn, +64) of the block (4 weight fragments,
// MFMA A side), 16 accumulator tiles of v_mfma_scale_f32_16x16x128_f8f6f4.
// LDS: weights [buffer][step][fragment][1 KB in the MFMA's lane order] (the
// kernel-native layout, copied block by block); weight scales [buffer][row][4 KS B]
// in their global order; the routed rows' output slots; 4 KB per wave for staging
// output rows.
#include "device_common.h"
#include "host_internal.h"
#include "lds_copy.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = kLargeRows;   // routed rows per workgroup
constexpr int kCols = 128;          // output columns per block (8 weight fragments)
constexpr int kMaxKS = 3;

// Output rows of a wave's 64 x 64 tile, stored through LDS. A row of the tile: its
// first fp16 column (o), its first scale byte (os), and whether it is stored (ok;
// padding rows are not).
struct ORow {
  uint16_t* o;
  uint8_t* os;
  bool ok;
};
constexpr int kStageBytes = 32 * 128;   // per wave: 32 rows x 64 fp16 columns

// A wave's 64 x 64 output tile in acc[i][j] (lane (c, q): columns 16 i + 4 q .. +3 of
// tile row 16 j + c), written as fp16 codes with one power-of-two scale per 32
// columns (the codes and scale bytes of store_o_rows<4>). Written straight from the
// MFMA layout, one store instruction covers 32-byte pieces of 16 rows; these rows
// go through the wave's own LDS area instead, 32 rows at a time (16-byte chunk c of
// row r at chunk c ^ (r % 8)), and are read back 8 lanes per row, so that each store
// instruction writes whole 128-byte lines of 8 rows. (The few-K W2 at a MoE-TP8
// rank's shape writes 4 GB of rows per call and is bound by these stores.) A
// wave's LDS operations complete in order, so the area needs no barrier.
// row_at(r), r = 0 .. 63: the tile row's ORow.
template <typename RowFn>
__device__ __forceinline__ void store_o_tile64(const v4f (&acc)[4][4], uint8_t* stage, const RowFn& row_at,
                                               int lane) {
  const int q = lane >> 4, c = lane & 15;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * half + jj;
      int ex[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float m = 0.f;
#pragma unroll
        for (int i = 2 * b; i < 2 * b + 2; ++i)
#pragma unroll
          for (int k = 0; k < 4; ++k) m = fmaxf(m, fabsf(acc[i][j][k]));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        ex[b] = o_exponent(m);
      }
      if (q == 0) {
        const ORow w = row_at(16 * j + c);
        if (w.ok) *reinterpret_cast<uint16_t*>(w.os) = (uint16_t)((ex[0] + 127) | ((ex[1] + 127) << 8));
      }
      const int r = 16 * jj + c;   // row of the staged half
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float inv = exp2_neg(ex[i >> 1]);
        const int chunk = (2 * i + (q >> 1)) ^ (r & 7);
        *reinterpret_cast<uint2*>(stage + r * 128 + chunk * 16 + 8 * (q & 1)) =
            f16_pack4(acc[i][j][0] * inv, acc[i][j][1] * inv, acc[i][j][2] * inv, acc[i][j][3] * inv);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 8 * k + (lane >> 3), chunk = lane & 7;
      const v4i v = *reinterpret_cast<const v4i*>(stage + r * 128 + ((chunk ^ (r & 7)) << 4));
      const ORow w = row_at(32 * half + r);
      if (w.ok) *reinterpret_cast<v4i*>(w.o + 8 * chunk) = v;
    }
  }
}

struct FewKArgs {
  const int2* items;
  const int32_t* n_items;  // items [first[0], n_items[0]) of the list are this launch's
  const int32_t* offsets;
  const int32_t* sorted_pairs;
  const uint8_t* h_q;      // [P, I] E4M3, rows in plan order
  const uint8_t* h_s;      // [P, I/128] E8M0
  const uint8_t* w2;       // [E, H, I/2], kernel-native layout
  const uint8_t* w2_s;     // [E, H, I/32]
  uint16_t* o;             // per-pair rows: fp16 codes
  uint8_t* os;             // and their 32-column scales
  uint32_t h_bytes;        // size of h_q
  int item_shift;          // 1: items hold 256 rows, workgroup y covers half y % 2 of item y / 2
  int H, I;
  int blocks_per_wg;       // 128-column blocks per workgroup (the last run may be shorter)
  const int32_t* first = nullptr;   // null: from item 0
};

template <int KS>
__global__ __launch_bounds__(kThreads, 2) void k_w2_fewk(FewKArgs a) {
  // weight scales of a block: 128 rows x 4 KS bytes, copied as 256-byte dword
  // copies, kScaleCopies per wave (the ones past the block's bytes fetch nothing
  // and land in the padding)
  constexpr int kScaleCopies = (2 * KS + 3) / 4;
  __shared__ __attribute__((aligned(1024))) uint8_t sA[2][KS][8 * 1024];       // [buf][step][fragment][1 KB]
  __shared__ __attribute__((aligned(16))) uint8_t sSa[2][4 * kScaleCopies * 256];  // [buf][row][4 KS B] + padding
  __shared__ int sSlot[kRows];
  __shared__ __attribute__((aligned(16))) uint8_t sStage[kThreads / 64][kStageBytes];

  const int item = (a.first ? a.first[0] : 0) + (int)(blockIdx.y >> a.item_shift);
  if (item >= a.n_items[0]) return;
  const int2 it = a.items[item];
  const int e = it.x;
  const int e_begin = a.offsets[e], e_end = a.offsets[e + 1];
  const int row0 = e_begin + it.y + (blockIdx.y & a.item_shift) * kRows;   // first sorted row of the tile
  const int nrows = min(kRows, e_end - row0);
  if (nrows <= 0) return;                               // empty second half of a 256-row item
  const int n_blocks = a.H / kCols;
  const int b_first = blockIdx.x * a.blocks_per_wg;
  const int b_count = min(n_blocks, b_first + a.blocks_per_wg) - b_first;
  if (b_count <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int I = a.I, srow = I / 32;                     // srow = 4 KS scale bytes per weight row

  if (tid < kRows) sSlot[tid] = a.sorted_pairs[row0 + (tid < nrows ? tid : 0)];

  // routed-row fragments j (rows 64 wm + 16 j + c; padding repeats the first row):
  // lane (c, q) holds K 16q .. +15 and 64 + 16q .. +15 of every K step
  const rsrc_t rh = make_rsrc(a.h_q, a.h_bytes);
  v8i bq[4][KS];
  int sb[4][KS];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 64 * wm + 16 * j + c;
    const int hr = row0 + (r < nrows ? r : 0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const v4i lo = buf_load16(rh, hr * I + s * 128 + 16 * q, 0);
      const v4i hi = buf_load16(rh, hr * I + s * 128 + 64 + 16 * q, 0);
      bq[j][s][0] = lo[0]; bq[j][s][1] = lo[1]; bq[j][s][2] = lo[2]; bq[j][s][3] = lo[3];
      bq[j][s][4] = hi[0]; bq[j][s][5] = hi[1]; bq[j][s][6] = hi[2]; bq[j][s][7] = hi[3];
      sb[j][s] = a.h_s[(int64_t)hr * KS + s];
    }
  }
  wait_vmcnt<0>();

  const int64_t w_bytes = (int64_t)a.H * (I / 2);
  const v4i_s rw = rsrc4(a.w2 + (int64_t)e * w_bytes, (uint32_t)w_bytes);
  const v4i_s rws = rsrc4(a.w2_s + (int64_t)e * a.H * srow, (uint32_t)(a.H * srow));
  // Weight block b into buffer buf: wave w copies fragments 2w, 2w+1 (expert rows
  // 128 b + 16 f ..) of every K step, then its share of the block's 128 contiguous
  // scale rows (256-byte chunk 4k + w for copy k).
  auto copy_block = [&](int b, int buf) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int frag = 2 * wave + f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        dma16(rw, lds_addr(&sA[buf][s][frag * 1024]), (8 * b + frag) * 16 * (I / 2) + s * 1024 + lane * 16, 0);
    }
#pragma unroll
    for (int k = 0; k < kScaleCopies; ++k) {
      const int chunk = 4 * k + wave;
      dma4(rsrc_sized(rws, chunk < 2 * KS), lds_addr(&sSa[buf][chunk * 256]),
           b * kCols * srow + chunk * 256 + lane * 4, 0);
    }
  };
  constexpr int kCopiesPerBlock = 2 * KS + kScaleCopies;   // per wave
  copy_block(b_first, 0);
  __syncthreads();                                      // sSlot

  for (int bi = 0; bi < b_count; ++bi) {
    const int buf = bi & 1;
    if (bi + 1 < b_count) {
      copy_block(b_first + bi + 1, buf ^ 1);
      wait_vmcnt<kCopiesPerBlock>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int frag = 4 * wn + i;
        const v4i w = *reinterpret_cast<const v4i*>(&sA[buf][s][frag * 1024 + lane * 16]);
        const int sa = sSa[buf][(frag * 16 + c) * srow + 4 * s + q];
        v8i aop;
        aop[0] = w[0]; aop[1] = w[1]; aop[2] = w[2]; aop[3] = w[3];
        aop[4] = 0; aop[5] = 0; aop[6] = 0; aop[7] = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = mfma_scale_16x16x128<kFmtE2M1, kFmtE4M3>(aop, bq[j][s], acc[i][j], sa, sb[j][s]);
      }
    }

    // per-pair rows of this block: tile row r is routed row 64 wm + r, at its slot
    const int col0 = (b_first + bi) * kCols + 64 * wn;
    store_o_tile64(acc, sStage[wave], [&](int r) {
      const int row = 64 * wm + r;
      const int64_t slot = sSlot[row < nrows ? row : 0];
      return ORow{a.o + slot * a.H + col0, a.os + slot * (a.H / 32) + col0 / 32, row < nrows};
    }, lane);
    __syncthreads();   // every wave has read buffer buf before block bi+2 is copied into it
  }
}

// Dense shared expert, W2s with a short reduction (Is <= 384, as for one MoE-TP8
// rank: the pages split the shared expert's intermediate like the routed experts'):
// out[t, n] = sum_k sh[t, k] W2s[n, k], FP8 E4M3 x E4M3 with the token's E8M0 scale
// per 128 columns of sh and one E8M0 scale per 128 x 128 block of W2s. A workgroup
// owns 128 tokens; each wave keeps its 4 token fragments for every K step in
// registers (read once from memory), and the workgroup walks a run of 128-column
// blocks of W2s, double-buffering each block's codes in LDS (rows of 128 bytes per K
// step, 16-byte chunk index XORed by (row / 2) % 8) behind the previous block's
// MFMAs and stores. Waves: 2 x 2, wave (wm, wn) = tokens [64 wm, +64) x columns
// [64 wn, +64) of the block; rows are written like the routed per-pair rows.
constexpr int kSCols = 128;   // output columns per block

struct SharedFewKArgs {
  const uint8_t* sh_q;     // [T, Is] E4M3
  const uint8_t* sh_s;     // [T, Is/128] E8M0
  const uint8_t* w;        // W2s [H, Is] E4M3
  const uint8_t* w_s;      // [H/128, Is/128] E8M0
  uint16_t* o;             // [T, H] fp16 codes
  uint8_t* os;             // [T, H/32] their scales
  int T, H, Is;
  int blocks_per_wg;
};

template <int KS>
__global__ __launch_bounds__(kThreads, 1) void k_shared2_fewk(SharedFewKArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sW[2][KS][kSCols * 128];   // [buf][step][row][128 B]
  __shared__ __attribute__((aligned(16))) uint8_t sStage[kThreads / 64][kStageBytes];

  const int t0 = blockIdx.y * kRows;
  const int n_blocks = a.H / kSCols;
  const int b_first = blockIdx.x * a.blocks_per_wg;
  const int b_count = min(n_blocks, b_first + a.blocks_per_wg) - b_first;
  if (b_count <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int Is = a.Is;

  // token fragments j (rows 64 wm + 16 j + c) of every K step: lane (c, q) holds K
  // 16q .. +15 and 64 + 16q .. +15 of the step; tokens past T read zeros
  const rsrc_t rs = make_rsrc(a.sh_q, (uint32_t)((int64_t)a.T * Is));
  v8i bq[4][KS];
  int sb[4][KS];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + 64 * wm + 16 * j + c;
    const int tc = min(t, a.T);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const v4i lo = buf_load16(rs, tc * Is + s * 128 + 16 * q, 0);
      const v4i hi = buf_load16(rs, tc * Is + s * 128 + 64 + 16 * q, 0);
      bq[j][s][0] = lo[0]; bq[j][s][1] = lo[1]; bq[j][s][2] = lo[2]; bq[j][s][3] = lo[3];
      bq[j][s][4] = hi[0]; bq[j][s][5] = hi[1]; bq[j][s][6] = hi[2]; bq[j][s][7] = hi[3];
      sb[j][s] = t < a.T ? (int)a.sh_s[(int64_t)t * KS + s] : 127;
    }
  }
  wait_vmcnt<0>();

  // Block b into buffer buf: instruction (i, s) of wave w copies rows 32w + 8i .. +7
  // of K step s, lane l -> row + l/8, physical chunk l%8 holding logical chunk
  // (l%8) ^ (row / 2) % 8.
  const v4i_s rw = rsrc4(a.w, (uint32_t)((int64_t)a.H * Is));
  auto copy_block = [&](int b, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 32 * wave + 8 * i + (lane >> 3);
      const int off = (b * kSCols + row) * Is + (((lane & 7) ^ ((row >> 1) & 7)) << 4);
#pragma unroll
      for (int s = 0; s < KS; ++s) dma16(rw, lds_addr(&sW[buf][s][(32 * wave + 8 * i) * 128]), off + s * 128, 0);
    }
  };
  constexpr int kCopiesPerBlock = 4 * KS;               // per wave
  copy_block(b_first, 0);

  // weight fragment i = block rows 64 wn + 16 i + c, swizzle (c / 2) % 8
  const int offA0 = (64 * wn + c) * 128 + ((q ^ (c >> 1)) << 4);
  const int offA1 = (64 * wn + c) * 128 + (((4 + q) ^ (c >> 1)) << 4);

  for (int bi = 0; bi < b_count; ++bi) {
    const int buf = bi & 1;
    const int b = b_first + bi;
    if (bi + 1 < b_count) {
      copy_block(b + 1, buf ^ 1);
      wait_vmcnt<kCopiesPerBlock>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int sw = a.w_s[b * KS + s];                  // the block's 128 x 128 scale of step s
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4i lo = *reinterpret_cast<const v4i*>(&sW[buf][s][offA0 + i * 16 * 128]);
        const v4i hi = *reinterpret_cast<const v4i*>(&sW[buf][s][offA1 + i * 16 * 128]);
        v8i aop;
        aop[0] = lo[0]; aop[1] = lo[1]; aop[2] = lo[2]; aop[3] = lo[3];
        aop[4] = hi[0]; aop[5] = hi[1]; aop[6] = hi[2]; aop[7] = hi[3];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = mfma_scale_16x16x128<kFmtE4M3, kFmtE4M3>(aop, bq[j][s], acc[i][j], sw, sb[j][s]);
      }
    }

    // tile row r is token t0 + 64 wm + r
    const int col0 = b * kSCols + 64 * wn;
    store_o_tile64(acc, sStage[wave], [&](int r) {
      const int t = t0 + 64 * wm + r;
      const int64_t tt = t < a.T ? t : t0;
      return ORow{a.o + tt * a.H + col0, a.os + tt * (a.H / 32) + col0 / 32, t < a.T};
    }, lane);
    __syncthreads();   // every wave has read buffer buf before block bi+2 is copied into it
  }
}

}  // namespace

bool fewk2_supported(const moe_dims& d) {
  const int64_t P = (int64_t)d.T * d.K;
  return d.I / 128 <= kMaxKS && d.H % kCols == 0 && P * d.I < ((int64_t)1 << 31) &&
         (int64_t)d.H * (d.I / 2) < ((int64_t)1 << 31);
}

hipError_t launch_w2_fewk(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                          int item_rows, const int32_t* offsets, const int32_t* sorted_pairs, const uint8_t* h_q,
                          const uint8_t* h_s, const uint8_t* w2, const uint8_t* w2_s, uint16_t* o, uint8_t* os,
                          hipStream_t s, const int32_t* first) {
  if (max_items <= 0) return hipSuccess;
  const int shift = item_rows == 2 * kRows ? 1 : 0;
  const int n_blocks = d.H / kCols;
  // four runs of column blocks per routed-row tile: more, shorter workgroups (a
  // shorter tail at the end of the grid) for three more reads of the routed rows
  const int per_wg = (n_blocks + 3) / 4;
  const int64_t P = (int64_t)d.T * d.K;
  FewKArgs a{items, n_items, offsets, sorted_pairs, h_q, h_s, w2, w2_s, o, os, (uint32_t)(P * d.I), shift,
             d.H, d.I, per_wg};
  a.first = first;
  dim3 grid((unsigned)ceil_div(n_blocks, per_wg), (unsigned)(max_items << shift));
  switch (d.I / 128) {
    case 1: hipLaunchKernelGGL(k_w2_fewk<1>, grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_w2_fewk<2>, grid, dim3(kThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL(k_w2_fewk<3>, grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool shared2_fewk_supported(const moe_dims& d) {
  return d.Is > 0 && d.Is / 128 <= kMaxKS && d.H % kSCols == 0 && (int64_t)d.H * d.Is < ((int64_t)1 << 31);
}

hipError_t launch_shared2_fewk(const moe_dims& d, const uint8_t* sh_q, const uint8_t* sh_s, const uint8_t* w2s,
                               const uint8_t* w2s_s, uint16_t* so, uint8_t* sos, hipStream_t s) {
  const int n_blocks = d.H / kSCols;
  const int per_wg = (n_blocks + 3) / 4;
  SharedFewKArgs a{sh_q, sh_s, w2s, w2s_s, so, sos, d.T, d.H, d.Is, per_wg};
  dim3 grid((unsigned)ceil_div(n_blocks, per_wg), (unsigned)ceil_div(d.T, kRows));
  switch (d.Is / 128) {
    case 1: hipLaunchKernelGGL(k_shared2_fewk<1>, grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_shared2_fewk<2>, grid, dim3(kThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL(k_shared2_fewk<3>, grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
