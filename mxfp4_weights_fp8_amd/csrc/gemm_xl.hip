// Large-M grouped GEMMs on 256-row work items: 256 routed rows x 256 weight rows
// per workgroup, on the gfx950 block-scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4.
//
// Prefill routing puts most routed rows in a few heavy experts ("Pushing the Limits
// of Serving DeepSeek-V4-Pro", section 3.3), whose rows fill whole 256-row items;
// the planner sends the remainder of each expert (1..128 rows) to the 128-row tile.
// Per MFMA, a 256 x 256 tile moves 25% fewer bytes from L2 into LDS than a 256 x 128
// tile (0.5 B per weight element and 1 B per routed-row element, each loaded once
// per workgroup and K step) and reads 25% fewer operand bytes from LDS (each wave
// owns 128 x 128 outputs).
//
// Waves: a 2 x 2 grid; wave (wm, wn) owns routed rows [128 wm, +128) (8 fragments
// of 16, MFMA B side, E4M3) and 128 weight rows (8 fragments, MFMA A side, E2M1):
//   W13: gate fragments 4wn..4wn+3 and up fragments 8+4wn.. of the tile's 128 gate
//        rows [n0, n0+128) and 128 up rows [I+n0, I+n0+128), so one lane holds gate
//        and up of the same h columns and the workgroup sees whole 128-column
//        blocks for the fused FP8 requantization (same blog, section 4.3);
//   W2:  output columns [128 wn, +128) of the tile's 256.
// The 64 accumulator tiles of a wave (256 registers) live in the AGPR file; the
// MFMAs are issued from inline asm with "+a" operands so that the compiler keeps
// each tile in fixed AGPRs (its own register choice copied accumulators between
// the register files inside the K loop).
//
// LDS (161792 bytes for W13, 162816 for W2):
//   weights: four one-step buffers (buffer s % 4 holds K step s), [fragment][1 KB
//     in lane order] (the kernel-native weight layout, copied block by block), 64 KB;
//   routed rows: two buffers of one K step (128 B of E4M3 per row), 64 KB;
//   weight E8M0 scales: three chunks of four K steps (16 B per row), 12 KB;
//   activation scales of the whole tile: 68 B per routed row, 17 KB.
// Routed rows are stored as 128-byte lines with the 16-byte chunk index XORed by
// (row / 2) % 8, so that a fragment read hits every bank once per 16 lanes; a
// weight fragment is read by lane l at 16*l.
//
// Schedule of one K step s (per wave): 8 columns; column j issues the 8 MFMAs of
// routed-row fragment j against the 8 weight fragments of step s, reads routed-row
// fragment j+1 of step s (four rotating register buffers) and weight fragment j of
// step s+1 (two register sets). After column 6 every wave has read all routed-row
// fragments of step s, so a barrier there (M_s) frees that buffer. The window of
// copies between M_{s-1} and M_s (column 7 of step s-1, columns 0-3 of step s) holds,
// in this order:
//   routed rows of step s+1 (into the buffer step s-1 used): four copies in column
//     7, two in each of columns 0 and 1;
//   one quarter of weight-scale chunk (s+5)/4 in column 0 (needed from the reads of
//     step 4*chunk, made while step 4*chunk-1 runs; its buffer held chunk-3);
//   the weights of step s+3, two blocks in each of columns 2 and 3, into the buffer
//     of step s-1 (last read while step s-2 ran).
// Copies complete in issue order, so M_s waits until at most this wave's 4 weight
// copies are in flight: everything needed after M_s has landed, and the weights,
// which come from HBM more often than the routed rows, have until M_{s+1} (eleven
// columns of MFMAs) instead of a few columns. Measured on the 32K prefill: spreading
// the copies over five columns instead of issuing them together after the barrier
// took 2.5% off the W13 launch; the one-step buffers with the longer weight lead
// (against two-step stages copied in one window and waited at the next barrier)
// another 2.5–4% off W13 and 3.5% off W2.
// Copies past the last step use a buffer resource of size 0 (they write zeros and
// touch no memory), so the loop body has no branches.
#include "device_common.h"
#include "host_internal.h"
#include "lds_copy.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTok = kXlRows;            // routed rows per tile
constexpr int kARows = 256;              // weight rows per tile
constexpr int kStepA = kARows * 64;     // E2M1 codes of one K step
constexpr int kStepB = kTok * 128;       // E4M3 codes of one K step
constexpr int kChunkRow = 16;            // weight-scale bytes per row and chunk (four K steps)
constexpr int kChunk = kARows * kChunkRow;
constexpr int kMaxKS = 64;               // K steps whose activation scales fit in LDS
constexpr int kSbRow = kMaxKS + 4;       // activation-scale bytes per routed row (17 dwords)
constexpr int kSbBytes = kTok * kSbRow;  // a whole number of 256-byte copy blocks

struct XlArgs {
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
  uint16_t* o;             // W2 out: fp16 codes per pair slot
  uint8_t* os;             // and their 32-column scales
  uint32_t act_bytes;      // size of act
  uint32_t act_s_bytes;    // size of act_s
  int act_s_dma;           // act_s rows are 4-byte aligned: copy them with dword copies
  int H, I, K;
  int gi, gn;              // XCD group: gi work items x gn column blocks
  int ngn;                 // column groups (column blocks / gn)
  int P;                   // pairs (entries of sorted_pairs)
};

// acc += A (E2M1, 32 K values per lane) x B (E4M3) with E8M0 scales: byte 0 of sa,
// byte OB of sb (op_sel); acc stays in AGPRs. The compiler does not know that the
// statement is an MFMA, so it inserts no wait states after VALU writes of the
// operands: s_nop 4 provides them (the MFMA pipe is busy with the previous MFMA).
template <int OB>
__device__ __forceinline__ void mma_agpr(v4f& acc, const v4i& a, const v8i& b, int sa, int sb) {
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (OB == 0)
    asm volatile("s_nop 4\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4"
                 : "+a"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
  else if constexpr (OB == 1)
    asm volatile("s_nop 4\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[0,1,0] op_sel_hi:[0,0,0] cbsz:4"
                 : "+a"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
  else if constexpr (OB == 2)
    asm volatile("s_nop 4\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,1,0] cbsz:4"
                 : "+a"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
  else
    asm volatile("s_nop 4\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[0,1,0] op_sel_hi:[0,1,0] cbsz:4"
                 : "+a"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
#endif
}

struct AOps {     // one K step of this wave's 8 weight fragments
  v4i w[8];
  int sa[8];
};

template <bool W13>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_xl(XlArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA[4][kStepA];    // [step % 4][fragment][1 KB]
  __shared__ __attribute__((aligned(1024))) uint8_t sB[2][kStepB];    // [step][row][128 B]
  __shared__ __attribute__((aligned(16))) uint8_t sSa[3][kChunk];     // [chunk][row][16 B]
  __shared__ __attribute__((aligned(16))) uint8_t sSb[kSbBytes];      // [row][kSbRow B]
  __shared__ int sTok[kTok];
  __shared__ int sSlot[W13 ? 1 : kTok];

  // Workgroup -> (work item, column block). The hardware hands out workgroups to
  // the 8 XCDs round-robin by linear id, and each XCD has its own L2, so the
  // workgroups an XCD runs together form one group of gi work items x gn column
  // blocks: the group's routed-row tiles are fetched once per XCD and shared by gn
  // workgroups, its weight slices shared by gi. Groups run heavy items first.
  const int L = blockIdx.x, xcd = L & 7, idx = L >> 3, gsz = a.gi * a.gn;
  const int sl = idx / gsz, pos = idx - sl * gsz;
  const int grp = sl * 8 + xcd, ig = grp / a.ngn, ng = grp - ig * a.ngn;
  const int item = ig * a.gi + pos / a.gn;
  if (item >= a.n_items[0]) return;
  const int2 it = a.items[item];
  const int e = it.x;
  const int e_begin = a.offsets[e], e_end = a.offsets[e + 1];
  const int row0 = e_begin + it.y;                      // first sorted row of the tile
  const int nrows = min(kTok, e_end - row0);
  const int nb = ng * a.gn + pos % a.gn;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  const int Kdim = W13 ? a.H : a.I;                     // reduction length
  const int N = W13 ? 2 * a.I : a.H;                    // weight rows per expert
  const int KS = Kdim / 128;                            // K steps (a multiple of 4)
  const int wrow = Kdim / 2, srow = Kdim / 32, arow = Kdim;

  const v4i_s rw = rsrc4(a.w + (int64_t)e * N * wrow, (uint32_t)(N * wrow));
  const v4i_s rws = rsrc4(a.w_s + (int64_t)e * N * srow, (uint32_t)(N * srow));
  const v4i_s ra = rsrc4(a.act, a.act_bytes);
  const v4i_s ras = rsrc4(a.act_s, a.act_s_bytes);

  // expert weight row of LDS row r (0..255): fragments of 16 rows
  auto w_row = [&](int r) -> int {
    const int f = r >> 4;
    if (W13) return (f < 8 ? 0 : a.I) + nb * 128 + (f & 7) * 16 + (r & 15);
    return nb * 256 + r;
  };
  // Copy plans (per wave). Weights (kernel-native layout: a fragment's codes of one
  // K step are 1 KB in lane order): instruction i of a K step copies the block of LDS
  // fragment 4*wave + i to LDS [fragment][1 KB] of the step's buffer; a wave's 64
  // weight rows are consecutive expert rows. Routed rows: instruction i
  // moves LDS rows 64*wave + 8i .. +7, lane l -> row +l/8, physical chunk l%8 holding
  // logical chunk (l%8) ^ s(row), s(row) = (row / 2) % 8 = 4 (i % 2) + l / 16. Weight
  // scales: instruction i moves rows 64*wave + 16i .. +15, lane l -> row +l/4, dword
  // l%4 of the chunk. Lane offsets are loop-invariant registers; the K position goes
  // in the scalar offset (the hardware range check covers the lane offset only, and
  // a copy past the last step takes a size-0 resource, which masks every lane).
  const int sw0 = ((lane & 7) ^ (lane >> 4)) << 4;
  const int sw1 = ((lane & 7) ^ (4 | (lane >> 4))) << 4;
  const int dA = w_row(64 * wave) * wrow + lane * 16;   // 64 consecutive expert rows per wave
  const int dS = w_row(64 * wave + (lane >> 2)) * srow + (lane & 3) * 4;
  int dW[4], dB[8], dSc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dW[i] = dA + 16 * i * wrow;
#pragma unroll
  for (int i = 0; i < 4; ++i) dSc[i] = dS + 16 * i * srow;

  auto copy_w = [&](int step, int i) {    // weight fragment 4 wave + i of K step `step`
    dma16(rsrc_sized(rw, step < KS), lds_addr(&sA[step & 3][(4 * wave + i) * 1024]), dW[i], step * 1024);
  };
  auto copy_t = [&](int step, int i) {    // routed rows of K step `step`, instruction i
    dma16(rsrc_sized(ra, step < KS), lds_addr(&sB[step & 1][(64 * wave + 8 * i) * 128]), dB[i], step * 128);
  };
  auto copy_s = [&](int chunk, int i) {   // weight scales of K steps 4 chunk .. +3, instruction i
    dma4(rsrc_sized(rws, 4 * chunk < KS), lds_addr(&sSa[chunk % 3][(64 * wave + 16 * i) * kChunkRow]), dSc[i],
         chunk * kChunkRow);
  };

  // Prologue. The tile's sorted pairs come first, one dword copy per wave into
  // routed-row buffer 1 (written by no copy before window 0); then scale chunk 0 and
  // quarter 0 of chunk 1 and the weights of steps 0-2, which need only the expert
  // and mostly come from HBM. Copies complete in issue order, so waiting until this
  // wave's 17 later copies are the only ones in flight finds the pairs in LDS while
  // the weights are still on their way.
  int32_t* sPairs = reinterpret_cast<int32_t*>(&sB[1][0]);   // [kTok]
  {
    const int np = min(a.P - row0, kTok);   // entries past the list read as zeros
    dma4(rsrc4(a.sorted_pairs + row0, (uint32_t)np * 4u), lds_addr(sPairs + 64 * wave), (64 * wave + lane) * 4, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) copy_s(0, i);
  copy_s(1, 0);
#pragma unroll
  for (int st = 0; st < 3; ++st)
#pragma unroll
    for (int i = 0; i < 4; ++i) copy_w(st, i);
  wait_vmcnt<17>();
  __syncthreads();
  // routed rows of the tile -> activation row (padding repeats the first row); W2
  // also keeps each row's output slot
  {
    const int pair = sPairs[tid < nrows ? tid : 0];
    sTok[tid] = W13 ? pair / a.K : row0 + (tid < nrows ? tid : 0);
    if (!W13) sSlot[W13 ? 0 : tid] = pair;
  }
  __syncthreads();

  // Activation scales: aligned rows by dword copies (instruction i of wave w covers
  // LDS dwords 64(4i + w) .. +63 of the table, row = dword / 17; the 17th dword of a
  // row and dwords past KS fetch bytes that are never read, offsets past the tensor
  // read zeros); otherwise one thread per row loads bytes.
  constexpr int kSbDw = kSbRow / 4;
  constexpr int kSbDma = kSbBytes / 1024;               // dword copies per wave
  if (a.act_s_dma) {
#pragma unroll
    for (int i = 0; i < kSbDma; ++i) {
      const int dw = 64 * (4 * i + wave) + lane;
      const int row = dw / kSbDw;
      dma4(ras, lds_addr(sSb + 256 * (4 * i + wave)), sTok[row] * KS + 4 * (dw - row * kSbDw), 0);
    }
  } else {
    const uint8_t* src = a.act_s + (int64_t)sTok[tid] * KS;
    uint32_t v[kMaxKS / 4];
#pragma unroll
    for (int i = 0; i < kMaxKS / 4; ++i) {
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int st = 4 * i + b;
        const uint32_t byte = src[min(st, KS - 1)];    // unconditional load, masked below
        w |= (st < KS ? byte : 0u) << (8 * b);
      }
      v[i] = w;
    }
#pragma unroll
    for (int i = 0; i < kMaxKS / 4; ++i) *reinterpret_cast<uint32_t*>(&sSb[tid * kSbRow + 4 * i]) = v[i];
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    dB[i] = sTok[64 * wave + 8 * i + (lane >> 3)] * arow + ((i & 1) ? sw1 : sw0);
  }
  // then the routed rows of step 0; (after M_{-1}) the column-7 part of window 0
#pragma unroll
  for (int i = 0; i < 8; ++i) copy_t(0, i);
  wait_vmcnt<0>();
  __syncthreads();

  // Operand reads. A lane reads 16-byte chunk q (and 4 + q) of its fragment row;
  // fragment rows are multiples of 16, so row c has swizzle (c / 2) % 8. Buffer,
  // fragment and step-in-chunk offsets are compile-time constants added to a few
  // per-lane base addresses (LDS reads take them as immediate offsets).
  const int off0 = c * 128 + ((q ^ (c >> 1)) << 4);
  const int off1 = c * 128 + (((4 + q) ^ (c >> 1)) << 4);
  auto a_row = [&](int i) {   // first LDS row of this wave's weight fragment i
    return W13 ? (i < 4 ? 64 * wn + 16 * i : 128 + 64 * wn + 16 * (i - 4)) : 128 * wn + 16 * i;
  };
  const uint8_t* pA = &sA[0][0] + lane * 16;   // + step buffer, fragment (a_row * 64)
  const uint8_t* pB0 = &sB[0][0] + 128 * wm * 128 + off0;
  const uint8_t* pB1 = &sB[0][0] + 128 * wm * 128 + off1;
  const uint8_t* pSa = &sSa[0][0] + c * kChunkRow + q;   // + chunk buffer, a_row(i) * 16, (step % 4) * 4
  const uint8_t* pSb = sSb + (128 * wm + c) * kSbRow;     // + 16 j kSbRow + 4 (step / 4)

  // weight fragment i of a K step: step buffer sbuf (step % 4), scale chunk base sa
  // (buffer of the step's chunk), step % 4 = u
  auto read_a = [&](AOps& o, int sbuf, const uint8_t* sa, int u, int i) {
    o.w[i] = *reinterpret_cast<const v4i*>(pA + sbuf * kStepA + a_row(i) * 64);
    o.sa[i] = sa[a_row(i) * kChunkRow + u * 4];
  };
  v8i bf[4];
  auto read_b = [&](int buf, int j, int slot) {  // routed-row fragment j from buffer buf
    const v4i lo = *reinterpret_cast<const v4i*>(pB0 + buf * kStepB + j * 2048);
    const v4i hi = *reinterpret_cast<const v4i*>(pB1 + buf * kStepB + j * 2048);
    bf[slot][0] = lo[0]; bf[slot][1] = lo[1]; bf[slot][2] = lo[2]; bf[slot][3] = lo[3];
    bf[slot][4] = hi[0]; bf[slot][5] = hi[1]; bf[slot][6] = hi[2]; bf[slot][7] = hi[3];
  };
  // activation-scale bytes of four K steps of routed-row fragment j (one dword; the
  // MFMA's op_sel picks the step's byte)
  auto read_bs = [&](int t, int j) { return *reinterpret_cast<const int*>(pSb + 16 * j * kSbRow + 4 * t); };

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  AOps ops[2];
  int bsc[8], bsn[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) read_a(ops[0], 0, pSa, 0, i);
#pragma unroll
  for (int j = 0; j < 8; ++j) bsc[j] = read_bs(0, j);
  read_b(0, 0, 0);
  // column-7 part of window 0 (normally issued in column 7 of the previous step)
#pragma unroll
  for (int i = 0; i < 4; ++i) copy_t(1, i);

  // K steps 4t .. 4t+3; step u uses register set u % 2 and reads step 4t+u+1 into
  // the other one.
  for (int t = 0; t < KS / 4; ++t) {
    const uint8_t* saC = pSa + (t % 3) * kChunk;          // chunk t
    const uint8_t* saN = pSa + ((t + 1) % 3) * kChunk;    // chunk t + 1
    auto step = [&](auto U) {
      constexpr int u = decltype(U)::value;
      const int s = 4 * t + u;
      AOps& cur = ops[u & 1];
      AOps& nxt = ops[(u + 1) & 1];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < 7) read_b(u & 1, j + 1, (j + 1) & 3);
        else read_b((u + 1) & 1, 0, 0);      // after M_s: routed rows of step s+1 are in LDS
        // weight fragment j of step s+1 (buffer (s+1)%4, chunk (s+1)/4)
        read_a(nxt, (u + 1) & 3, u < 3 ? saC : saN, (u + 1) & 3, j);
        if (u == 3) bsn[j] = read_bs(t + 1, j);
#pragma unroll
        for (int i = 0; i < 8; ++i) mma_agpr<u>(acc[i][j], cur.w[i], bf[j & 3], cur.sa[i], bsc[j]);
        // window s (before M_s), columns 0-3: the rest of the routed rows of step s+1,
        // one weight-scale quarter, then the weights of step s+3
        if (j < 2) {
          copy_t(s + 1, 4 + 2 * j);
          copy_t(s + 1, 5 + 2 * j);
        }
        if (j == 2 || j == 3) {          // weights of step s+3, last in the window
          copy_w(s + 3, 2 * (j - 2));
          copy_w(s + 3, 2 * (j - 2) + 1);
        }
        if (j == 0) copy_s((s + 5) >> 2, (s + 5) & 3);
        // window s+1, column 7 (after M_s): half of the routed rows of step s+2
        if (j == 7) {
#pragma unroll
          for (int i = 0; i < 4; ++i) copy_t(s + 2, i);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (j == 6) {                    // M_s: all but the 4 weight copies of step s+3
          wait_vmcnt<4>();
          __syncthreads();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
#pragma unroll
    for (int j = 0; j < 8; ++j) bsc[j] = bsn[j];
  }
  wait_vmcnt<0>();
  // The compiler does not see the MFMAs in the asm statements, so it inserts no wait
  // states before the accumulators are read: 64 of them here, with scheduling
  // barriers so that no read moves above.
  __builtin_amdgcn_sched_barrier(0);
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#endif
  __builtin_amdgcn_sched_barrier(0);

  if (W13) {
    // SwiGLU + FP8 requantization. Lane (c, q) of routed-row fragment j holds h
    // columns 64wn + 16i + 4q .. +3 (i = 0..3: gate acc[i], up acc[4+i]) of tile row
    // 128wm + 16j + c. The two waves sharing a row exchange their amax in LDS (the
    // routed-row buffers are free once every copy has landed). The codes are staged
    // as the tile's 128-byte rows of h (16-byte chunk k of row r at chunk k ^ (r % 8))
    // and stored as whole cache lines, eight rows per instruction.
    __syncthreads();
    float* sRed = reinterpret_cast<float*>(&sB[0][0]);          // [2 halves][2 waves][kTok]
    uint8_t* sH = &sB[1][0];                                      // [kTok][128 B]
#pragma unroll
    for (int half = 0; half < 2; ++half) {    // routed-row fragments 4 half .. +3
      float hv[4][4][4];
      float amax[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * half + jj;
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float h = silu_mul(acc[i][j][r], acc[4 + i][j][r]);
            hv[jj][i][r] = h;
            m = fmaxf(m, fabsf(h));
          }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        amax[jj] = m;
      }
      float* red = sRed + half * 2 * kTok;
      if (q == 0) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) red[wn * kTok + 128 * wm + 16 * (4 * half + jj) + c] = amax[jj];
      }
      __syncthreads();
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = 128 * wm + 16 * (4 * half + jj) + c;
        const float m = fmaxf(red[row], red[kTok + row]);
        const int ex = e8m0_exponent(m);
        const float inv = exp2_neg(ex);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<uint32_t*>(sH + row * 128 + (((4 * wn + i) ^ (row & 7)) << 4) + 4 * q) =
              e4m3_pack4(hv[jj][i][0] * inv, hv[jj][i][1] * inv, hv[jj][i][2] * inv, hv[jj][i][3] * inv);
        if (row < nrows && wn == 0 && q == 0) a.h_s[(int64_t)(row0 + row) * (a.I / 128) + nb] = (uint8_t)(ex + 127);
      }
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 8; ++st) {       // wave w: rows 64 w .. +63
      const int r = 64 * wave + 8 * st + (lane >> 3), chunk = lane & 7;
      const v4i v = *reinterpret_cast<const v4i*>(sH + r * 128 + ((chunk ^ (r & 7)) << 4));
      if (r < nrows) *reinterpret_cast<v4i*>(a.h_q + (int64_t)(row0 + r) * a.I + nb * 128 + chunk * 16) = v;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 128 * wm + 16 * j + c;
      const int64_t slot = sSlot[W13 ? 0 : (row < nrows ? row : 0)];
      const int col0 = nb * 256 + 128 * wn;
      v4f r[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = acc[i][j];
      store_o_row128(r, row < nrows, a.o + slot * a.H + col0 + q * 4, a.os + slot * (a.H / 32) + col0 / 32, q);
    }
  }
}

}  // namespace

// XCD group shape: gn divides the column-block count, gi = 32 / gn (one workgroup
// per CU, 32 CUs per XCD); the shape with the fewest fetched bytes per workgroup
// (routed-row tile act_b over gn workgroups, weight slice w_b over gi) wins. The
// grid is a whole number of groups per XCD.
struct XcdGroups {
  int gi, gn, ngn;
  int64_t grid;
};
static XcdGroups xcd_groups(int n_blocks, int64_t max_items, double act_b, double w_b) {
  constexpr int kCusPerXcd = 32;
  XcdGroups g{1, 1, n_blocks, 0};
  double best = 1e300;
  for (int gn = 1; gn <= n_blocks && gn <= kCusPerXcd; ++gn) {
    if (n_blocks % gn) continue;
    const int gi = kCusPerXcd / gn;
    const double cost = (gi * act_b + gn * w_b) / (gi * gn);
    if (cost < best) { best = cost; g.gi = gi; g.gn = gn; }
  }
  g.ngn = n_blocks / g.gn;
  const int64_t groups = (max_items + g.gi - 1) / g.gi * g.ngn;
  g.grid = (groups + 7) / 8 * 8 * g.gi * g.gn;
  return g;
}

bool xl13_supported(const moe_dims& d) { return large_path_supported(d) && (d.H / 128) % 4 == 0; }
bool xl2_supported(const moe_dims& d) { return large_path_supported(d) && (d.I / 128) % 4 == 0; }

hipError_t launch_w13_xl(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                         const int32_t* offsets, const int32_t* sorted_pairs, const uint8_t* x_q,
                         const uint8_t* x_s, const uint8_t* w13, const uint8_t* w13_s, uint8_t* h_q,
                         uint8_t* h_s, hipStream_t s) {
  if (max_items <= 0) return hipSuccess;
  const int KS = d.H / 128;
  const XcdGroups g = xcd_groups(d.I / 128, max_items, (double)kTok * d.H, 256.0 * (d.H / 2 + d.H / 32));
  XlArgs a{items, n_items, offsets, sorted_pairs, x_q, x_s, w13, w13_s, h_q, h_s, nullptr, nullptr,
           (uint32_t)((int64_t)d.T * d.H), (uint32_t)((int64_t)d.T * KS),
           KS % 4 == 0 && (uintptr_t)x_s % 4 == 0, d.H, d.I, d.K, g.gi, g.gn, g.ngn, d.T * d.K};
  hipLaunchKernelGGL(k_gemm_xl<true>, dim3((unsigned)g.grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_w2_xl(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                        const int32_t* offsets, const int32_t* sorted_pairs, const uint8_t* h_q,
                        const uint8_t* h_s, const uint8_t* w2, const uint8_t* w2_s, uint16_t* o, uint8_t* os, hipStream_t s) {
  if (max_items <= 0) return hipSuccess;
  const int KS = d.I / 128;
  const int64_t P = (int64_t)d.T * d.K;
  const XcdGroups g = xcd_groups(d.H / 256, max_items, (double)kTok * d.I, 256.0 * (d.I / 2 + d.I / 32));
  XlArgs a{items, n_items, offsets, sorted_pairs, h_q, h_s, w2, w2_s, nullptr, nullptr, o, os,
           (uint32_t)(P * d.I), (uint32_t)(P * KS), KS % 4 == 0 && (uintptr_t)h_s % 4 == 0, d.H, d.I, d.K,
           g.gi, g.gn, g.ngn, (int)P};
  hipLaunchKernelGGL(k_gemm_xl<false>, dim3((unsigned)g.grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
