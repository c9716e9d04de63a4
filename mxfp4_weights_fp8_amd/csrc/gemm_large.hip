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
//   W2:  256 output columns; the epilogue writes each pair's row to its token-major
//        slot (fp16 codes with one power-of-two scale per 32 columns).
//
// Data movement: HBM/L2 -> LDS with direct-to-LDS buffer loads (buffer_load_dwordx4
// ... lds; lane l's 16 bytes land at M0 + 16*l), issued from inline asm with explicit
// vmcnt waits and barriers. Every copy instruction moves whole 128-byte lines: one
// weight fragment of one K step (the weights are in the kernel-native layout, 1 KB
// of consecutive bytes in the MFMA's lane order, read back by each lane at 16*l:
// no bank conflicts) or 8 routed rows x 128 B (one step of E4M3 codes). The vector
// L1 handles a limited number of line requests per cycle, and copying 16 rows x
// 64 B per instruction ran at a third of the rate of 8 rows x 128 B. Routed rows sit
// in LDS row-major with the 16-byte chunk index XORed by (row / 2) % 8: an MFMA
// fragment read (16 rows, one chunk per lane group) then covers all 64 banks once
// per 16 lanes (even rows in one 128-byte half of a bank row, odd rows in the
// other, each with 8 distinct chunks).
// A stage holds two K steps (32 KB of weights + 32 KB of activations); two stages.
// The weight E8M0 scales of eight K steps (32 B per row) come by dword copies of 8
// rows each; the activation scales of the whole tile are copied once, before the
// first stage.
#include "device_common.h"
#include "host_internal.h"
#include "lds_copy.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokTile = kLargeRows;      // 128 routed rows per tile
constexpr int kARows = 256;               // weight rows per tile
constexpr int kStageK = 2;                // 128-K steps per LDS stage
constexpr int kStageA = kARows * 128;     // bytes of E2M1 codes per stage (128 B per row)
constexpr int kStageB = kTokTile * 128;   // bytes of E4M3 codes per K step
constexpr int kCodeDma = 16;              // direct-to-LDS code copies per wave per stage
constexpr int kScaleSteps = 8;            // K steps per weight-scale chunk (32 B per row)
constexpr int kMaxKS = 64;                // K steps whose activation scales fit the tile's LDS
// LDS strides of the scale tables, padded so that the 16 rows of an MFMA fragment
// fall on 16 distinct banks: weight scales in groups of 8 rows x 32 B with 32 B of
// padding per group (the fragment's second 8 rows shift by 8 banks), activation
// scales 68 B per routed row (17 dwords).
constexpr int kSaGroup = 8 * kScaleSteps * 4 + 32;   // bytes per 8-row group
constexpr int kSbRow = kMaxKS + 4;
// whole rounds of the 4 waves' 256-byte dword copies (the last round runs past the
// tile's 128 * 68 bytes: without this padding it wrote into the next LDS array)
constexpr int kSbBytes = (kTokTile * kSbRow + 1023) / 1024 * 1024;

struct LargeArgs {
  const int2* items;
  const int32_t* n_items;  // items [first[0], n_items[0]) of the list are this launch's
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
  int item_shift;          // 1: items hold 256 rows, workgroup y covers half y % 2 of item y / 2
  int H, I, K;
  const int32_t* first = nullptr;   // null: from item 0
};

template <bool W13>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_large(LargeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA[2][kStageA];                 // [stage][row][128 B]
  __shared__ __attribute__((aligned(1024))) uint8_t sB[2][kStageK][kStageB];        // [stage][step][row][128 B]
  __shared__ __attribute__((aligned(16))) uint8_t sSa[2][kARows / 8][kSaGroup];     // [chunk buf][8-row group][row][step][4]
  __shared__ __attribute__((aligned(16))) uint8_t sSb[kSbBytes];                    // [row][step], kSbRow B per row
  __shared__ int sTok[kTokTile];
  __shared__ int sSlot[W13 ? 1 : kTokTile];
  __shared__ float sRed[2][kTokTile];

  const int item = (a.first ? a.first[0] : 0) + (int)(blockIdx.y >> a.item_shift);
  if (item >= a.n_items[0]) return;
  const int2 it = a.items[item];
  const int e = it.x;
  const int e_begin = a.offsets[e], e_end = a.offsets[e + 1];
  const int row0 = e_begin + it.y + (blockIdx.y & a.item_shift) * kTokTile;   // first sorted row of the tile
  const int nrows = min(kTokTile, e_end - row0);
  if (nrows <= 0) return;                               // empty second half of a 256-row item
  const int nb = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, c = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  const int Kdim = W13 ? a.H : a.I;                     // reduction length
  const int N = W13 ? 2 * a.I : a.H;                    // weight rows per expert
  const int KS = Kdim / 128;                            // 128-K steps
  const int NS = (KS + kStageK - 1) / kStageK;          // stages
  const int wrow = Kdim / 2, srow = Kdim / 32, arow = Kdim;

  // routed rows of the tile -> activation row index (padding repeats the first row);
  // W2 also keeps each row's output slot for the epilogue
  if (tid < kTokTile) {
    const int r = row0 + (tid < nrows ? tid : 0);
    const int pair = a.sorted_pairs[r];
    sTok[tid] = W13 ? pair / a.K : r;
    if (!W13) sSlot[W13 ? 0 : tid] = pair;
  }
  __syncthreads();
  // Activation scales of the whole tile (KS bytes per routed row) into rows of
  // kSbRow bytes. Aligned rows: dword copies straight into LDS, issued with the
  // prologue copies (instruction i of wave w covers LDS dwords 64(4i + w) .. +63, row
  // = dword / 17; the 17th dword of a row and dwords past KS fetch bytes that are
  // never read, and offsets past the tensor read zeros). Otherwise two threads per
  // row load bytes, all loads issued before the first LDS store.
  const v4i_s ras = rsrc4(a.act_s, a.act_s_bytes);
  constexpr int kSbDw = kSbRow / 4;                       // 17 dwords per row
  constexpr int kSbDma = (kTokTile * kSbDw + 255) / 256;  // rounds of copies (one per wave and round)
  static_assert(kSbDma * 4 * 256 <= kSbBytes, "the activation-scale copies stay inside sSb");
  auto issue_act_scales = [&]() {
#pragma unroll
    for (int i = 0; i < kSbDma; ++i) {
      const int dw = 64 * (4 * i + wave) + lane;
      const int row = min(dw / kSbDw, kTokTile - 1);
      dma4(ras, lds_addr(sSb + 256 * (4 * i + wave)), sTok[row] * KS + 4 * (dw - (dw / kSbDw) * kSbDw), 0);
    }
  };
  if (!a.act_s_dma) {
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
    for (int i = 0; i < kMaxKS / 8; ++i) *reinterpret_cast<uint32_t*>(&sSb[r * kSbRow + s0 + 4 * i]) = v[i];
  }

  // Buffer resources of this expert's weights and scales and of the activations.
  // The hardware range check applies to the lane offset, so every offset that can
  // run past a row end (the last stage of an odd K-step count, scale chunks past
  // the last step) is in the lane offset, and copies that would only fetch unused
  // bytes take a resource of size 0: they write zeros to LDS and touch no memory.
  const v4i_s rw = rsrc4(a.w + (int64_t)e * N * wrow, (uint32_t)(N * wrow));
  const v4i_s rws = rsrc4(a.w_s + (int64_t)e * N * srow, (uint32_t)(N * srow));
  const v4i_s ra = rsrc4(a.act, a.act_bytes);

  // expert weight row of LDS row r (0..255): fragments of 16 rows
  auto w_row = [&](int r) -> int {
    const int f = r >> 4;
    if (W13) return (f < 8 ? 0 : a.I) + nb * 128 + (f & 7) * 16 + (r & 15);
    return nb * 256 + r;
  };
  // Copy plan (per wave, per stage): 8 weight instructions, instruction i copies the
  // 1 KB block of LDS fragment 4*wave + i/2 and K step 2*stage + i%2 (the weights are
  // in the kernel-native layout: a fragment's codes of one K step are 1 KB in lane
  // order) to LDS [fragment][step][1 KB]; the 64 weight rows a wave copies are
  // consecutive expert rows (fragments of the gate or the up half, or of the W2
  // column block), so instruction i adds i/2 fragments to one lane offset.
  // 8 activation instructions, step wave/2 of the stage, routed rows
  // 64*(wave%2) + 8i .. +7, lane l -> row +l/8, physical chunk l%8 holding logical
  // chunk (l%8) ^ s(row), s(row) = (row / 2) % 8 = 4 (i % 2) + l / 16; routed rows
  // are arbitrary and take one lane offset each.
  const int r_lane = 64 * wave + (lane >> 3);           // LDS row of scale copy 0
  const int sw0 = ((lane & 7) ^ (lane >> 4)) << 4;      // swizzled chunk, even i
  const int sw1 = ((lane & 7) ^ (4 | (lane >> 4))) << 4; // odd i
  const int dA = w_row(64 * wave) * wrow + lane * 16;
  const int dS = w_row(r_lane) * srow + (lane & 7) * 4;
  int dB[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) dB[i] = sTok[64 * (wave & 1) + 8 * i + (lane >> 3)] * arow + ((i & 1) ? sw1 : sw0);
  const int b_step = wave >> 1;                         // step of the stage this wave copies

  // Copy instructions i (weight rows 64*wave + 8i .., routed rows 64*(wave%2) + 8i ..)
  // of stage stg (K steps 2stg, 2stg+1) into LDS buffer buf; valid == false (a
  // stage past the last) writes zeros.
  auto issue_part = [&](int buf, int stg, bool valid, int i) {
    dma16(rsrc_sized(rw, valid), lds_addr(&sA[buf][(4 * wave + (i >> 1)) * 2048 + (i & 1) * 1024]),
          dA + 16 * (i >> 1) * wrow + (i & 1) * 1024 + stg * 2048, 0);
    dma16(rsrc_sized(ra, valid), lds_addr(&sB[buf][b_step][(64 * (wave & 1) + 8 * i) * 128]),
          dB[i] + (stg * kStageK + b_step) * 128, 0);
  };
  auto issue_stage = [&](int buf, int stg, bool valid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_part(buf, stg, valid, i);
  };
  // Weight scales: chunk c (K steps 8c .. 8c+7, 32 B per row) goes to buffer c % 2,
  // in four parts of two 8-row copy instructions per wave. Part m of chunk c is
  // issued by stage 4c - 5 + m: the part that reuses chunk c-2's buffer follows the
  // last read of chunk c-2 (stage 4c-5's first step), and the last part is waited
  // for before step 8c is read (at stage 4c-1). Chunks past the last step write zeros.
  auto issue_scales = [&](int chunk, int part) {
    const v4i_s r_s = rsrc_sized(rws, chunk * kScaleSteps < KS);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 2 * part + h;
      dma4(r_s, lds_addr(&sSa[chunk & 1][8 * wave + i][0]), dS + chunk * kScaleSteps * 4 + 8 * i * srow, 0);
    }
  };

  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // LDS byte offsets of the operand reads. Fragment rows are multiples of 16, so a
  // row's swizzle (row / 2) % 8 is (c / 2) % 8 and the two 16-byte chunks a lane reads for
  // a K step (E2M1: chunk q of step 0 / 4+q of step 1 of the stage; E4M3: chunks
  // q and 4+q of its step) sit at two fixed per-lane offsets; stage, step and
  // fragment add compile-time constants.
  const int off0 = c * 128 + ((q ^ (c >> 1)) << 4);
  const int off1 = c * 128 + (((4 + q) ^ (c >> 1)) << 4);
  // this wave's 8 weight fragments: W13 gate 4wn..4wn+3 and up 8+4wn..; W2 8wn..8wn+7
  const int a_wave = W13 ? wn * 4 * 2048 : wn * 8 * 2048;
  auto a_frag = [](int i) { return W13 ? (i < 4 ? i : 8 + (i - 4)) * 2048 : i * 2048; };
  const uint8_t* pA = &sA[0][0] + a_wave + lane * 16;   // + stage, fragment, step * 1 KB
  const uint8_t* pB0 = &sB[0][0][0] + wm * 4 * 2048 + off0;
  const uint8_t* pB1 = &sB[0][0][0] + wm * 4 * 2048 + off1;
  // weight scales: lane group q reads its K block's byte of the (row, step) dword
  // (fragment f, row c) -> group 2f + c/8, row c%8 of the group
  const uint8_t* pSa = &sSa[0][0][0] + (a_wave / 2048) * 2 * kSaGroup + (c >> 3) * kSaGroup + (c & 7) * 32 + q;
  const uint8_t* pSb = sSb + (wm * 4 * 16 + c) * kSbRow;

  // Operands of one K step in registers: this wave's 4 routed-row fragments (E4M3)
  // and 8 weight fragments (E2M1) with their E8M0 scales. They are read in 8
  // parts (p < 4: routed-row fragment p; p >= 4: weight fragments 2(p-4), 2(p-4)+1)
  // so that LDS reads interleave with the MFMAs of the other register set.
  struct Ops {
    v8i b[4];
    v4i w[8];
    int sb[4];
    int sa[8];
  };
  auto load_part = [&](Ops& o, const int buf, const int h, int ks, const int p) {   // h: step within the stage
    if (p < 4) {
      const int ob = buf * kStageK * kStageB + h * kStageB + p * 2048;
      const v4i lo = *reinterpret_cast<const v4i*>(pB0 + ob);
      const v4i hi = *reinterpret_cast<const v4i*>(pB1 + ob);
      o.b[p][0] = lo[0]; o.b[p][1] = lo[1]; o.b[p][2] = lo[2]; o.b[p][3] = lo[3];
      o.b[p][4] = hi[0]; o.b[p][5] = hi[1]; o.b[p][6] = hi[2]; o.b[p][7] = hi[3];
      o.sb[p] = pSb[ks + p * 16 * kSbRow];
    } else {
      const uint8_t* sa = pSa + ((ks / kScaleSteps) & 1) * (kARows / 8 * kSaGroup) + (ks % kScaleSteps) * 4;
#pragma unroll
      for (int i = 2 * (p - 4); i < 2 * (p - 4) + 2; ++i) {
        o.w[i] = *reinterpret_cast<const v4i*>(pA + buf * kStageA + a_frag(i) + h * 1024);
        o.sa[i] = sa[a_frag(i) / 2048 * 2 * kSaGroup];
      }
    }
  };
  // the 4 MFMAs of weight fragment i
  auto mma_row = [&](const Ops& o, const int i) {
    v8i aop;
    aop[0] = o.w[i][0]; aop[1] = o.w[i][1]; aop[2] = o.w[i][2]; aop[3] = o.w[i][3];
    aop[4] = 0; aop[5] = 0; aop[6] = 0; aop[7] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = mfma_scale_16x16x128<kFmtE2M1, kFmtE4M3>(aop, o.b[j], acc[i][j], o.sa[i], o.sb[j]);
  };

  // Prologue: activation scales (aligned rows), weight scales of chunk 0 and part 0
  // of chunk 1, codes of stages 0 and 1, operands of step 0. A wave whose copies
  // are all in LDS has no copies of its own left but those of stage 1, so after
  // the barrier every copy but stage 1's has landed.
  if (a.act_s_dma) issue_act_scales();
#pragma unroll
  for (int m = 0; m < 4; ++m) issue_scales(0, m);
  issue_scales(1, 0);
  issue_stage(0, 0, true);
  issue_stage(1, 1, NS > 1);
  wait_vmcnt<kCodeDma>();
  __syncthreads();
  Ops opsA, opsB;
#pragma unroll
  for (int p = 0; p < 8; ++p) load_part(opsA, 0, 0, 0, p);

  // Stage k (both K steps valid, buffer k % 2); on entry opsA holds step 2k.
  //   Multiply step 2k while reading step 2k+1 into opsB.
  //   Wait for this wave's copies of stage k+1 (issued one stage earlier) and
  //   barrier: stage k+1 is in LDS, and every wave has read stage k.
  //   Multiply step 2k+1 while reading step 2k+2 into opsA (after the last full
  //   stage with an even K-step count this reads a stale buffer, never used) and
  //   issuing the copies of stage k+2 into stage k's buffer and one scale part.
  // The body has no branches. Each half is 8 groups of 4 MFMAs, one operand part
  // and (second half) two copy instructions, separated by scheduling barriers, so
  // LDS reads and copies issue between MFMAs instead of in bursts that would stall
  // the wave with the MFMA pipe idle.
  const int NF = KS / kStageK;   // stages with both K steps
  for (int k = 0; k < NF; ++k) {
    const int buf = k & 1;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      mma_row(opsA, p);
      load_part(opsB, buf, 1, 2 * k + 1, p);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    const bool more = k + 2 < NS;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      mma_row(opsB, p);
      load_part(opsA, buf ^ 1, 0, min(2 * k + 2, KS - 1), p);
      if (p == 0) issue_scales((k + 1) / 4 + 1, (k + 1) % 4);
      issue_part(buf, k + 2, more, p);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (KS & 1) {                  // the last K step, alone in its stage
#pragma unroll
    for (int p = 0; p < 8; ++p) mma_row(opsA, p);
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
          *reinterpret_cast<uint32_t*>(dst + 16 * i) =
              e4m3_pack4(acc[i][j][0] * inv, acc[i][j][1] * inv, acc[i][j][2] * inv, acc[i][j][3] * inv);
        }
        if (wn == 0 && q == 0) a.h_s[(int64_t)(row0 + row) * (a.I / 128) + nb] = (uint8_t)(ex + 127);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 64 * wm + 16 * j + c;
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

// The large-M kernels need whole 256-column W2 tiles and the tile's activation
// scales in LDS (at most kMaxKS K steps for both GEMMs).
bool large_path_supported(const moe_dims& d) {
  return d.H % 256 == 0 && d.H / 128 <= kMaxKS && d.I / 128 <= kMaxKS;
}

hipError_t launch_w13_large(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                            int item_rows, const int32_t* offsets, const int32_t* sorted_pairs,
                            const uint8_t* x_q, const uint8_t* x_s, const uint8_t* w13, const uint8_t* w13_s,
                            uint8_t* h_q, uint8_t* h_s, hipStream_t s, const int32_t* first) {
  if (max_items <= 0) return hipSuccess;
  const int shift = item_rows == 2 * kTokTile ? 1 : 0;
  const int KS = d.H / 128;
  LargeArgs a{items, n_items, offsets, sorted_pairs, x_q, x_s, w13, w13_s, h_q, h_s, nullptr, nullptr,
              (uint32_t)((int64_t)d.T * d.H), (uint32_t)((int64_t)d.T * KS),
              KS % 4 == 0 && (uintptr_t)x_s % 4 == 0, shift, d.H, d.I, d.K};
  a.first = first;
  hipLaunchKernelGGL(k_gemm_large<true>, dim3(d.I / 128, (unsigned)(max_items << shift)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_w2_large(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                           int item_rows, const int32_t* offsets, const int32_t* sorted_pairs,
                           const uint8_t* h_q, const uint8_t* h_s, const uint8_t* w2, const uint8_t* w2_s,
                           uint16_t* o, uint8_t* os, hipStream_t s, const int32_t* first) {
  if (max_items <= 0) return hipSuccess;
  const int shift = item_rows == 2 * kTokTile ? 1 : 0;
  const int KS = d.I / 128;
  const int64_t P = (int64_t)d.T * d.K;
  LargeArgs a{items, n_items, offsets, sorted_pairs, h_q, h_s, w2, w2_s, nullptr, nullptr, o, os,
              (uint32_t)(P * d.I), (uint32_t)(P * KS), KS % 4 == 0 && (uintptr_t)h_s % 4 == 0,
              shift, d.H, d.I, d.K};
  a.first = first;
  hipLaunchKernelGGL(k_gemm_large<false>, dim3(d.H / 256, (unsigned)(max_items << shift)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
