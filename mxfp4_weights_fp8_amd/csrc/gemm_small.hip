// Small-M grouped GEMMs (decode shapes, at most 16 routed rows per tile), on the
// gfx950 block-scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4.
//
// A 7-token verify leaves each expert a handful of rows, so generic tiles of 16+
// token rows mostly compute padding ("Optimization progress report",
// Optimization 06). Here the weights take the MFMA's 16-row A side (E2M1, one
// E8M0 scale per 32 K) and the routed tokens its 16-column B side (E4M3, the
// per-128 activation scale replicated over the four 32-blocks). The work is a
// stream of the expert's weights, in the kernel-native layout (a fragment's codes of
// one K step are 1 KB of consecutive bytes in lane order): each lane loads its 16
// bytes per fragment and K step straight from HBM into registers (no reuse across
// waves, so no LDS staging), four K steps of a wave's fragments in flight.
// (Measured on decode7: W13 0.1725 -> 0.155 ms and W2 0.096 -> 0.082 ms against
// loading the same bytes from row-major codes, 16 rows x 64 B per instruction.)
//
// W13 (gate/up, "Pushing the Limits of Serving DeepSeek-V4-Pro", section 3.3):
// a workgroup owns 128 columns of h = silu(gate) * up, i.e. gate rows
// [n0, n0+128) and up rows [I+n0, I+n0+128) of the expert, so the fused SwiGLU +
// FP8 requantization epilogue (same blog, section 4.3) sees a whole 128-column
// scale block per routed row and writes W2's E4M3 operand and E8M0 scales
// directly.
// W2 (down): a workgroup owns 64 * kW2Frags output columns; the epilogue writes
// each routed pair's row to its token-major slot p = t*K + j for the top-k combine
// (fp16 codes with one power-of-two scale per 32 columns).
#include "small_unit.h"

namespace moe {
namespace {

using namespace small;

constexpr int kThreads = 256;
// Work split: W13 workgroups of 4 waves, each streaming two gate and two up
// fragments; W2 waves of 2 fragments, 4 waves per workgroup (decode7, 39 experts:
// 0.111 -> 0.097 ms against 4 fragments, more and shorter streams keep more of HBM
// busy). W13 was 8 waves of one gate and one up fragment (0.1875 -> 0.1745 ms
// against 4 waves of two pairs, measured on an earlier loop); with the current loop
// (packed layout, four-step ring of scales) 4 waves of two pairs measured the same
// on decode7 (0.2188 vs 0.2185 ms per step) and 1.1% faster on the 256-token step
// (1.905 vs 1.926 ms), bitwise equal.
constexpr int kW13Waves = 4;
constexpr int kW2Frags = 2;
// Rows of list slots a small-M launch covers at once; more slots are walked by a
// grid-stride loop (decode lists stay below it: one slot per workgroup row).
constexpr int64_t kMaxSlotRows = 1024;

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_w13_small(
    const SmallLists lists,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
    const uint8_t* __restrict__ x_q, const uint8_t* __restrict__ x_s, const uint8_t* __restrict__ w13,
    const uint8_t* __restrict__ w13_s, uint8_t* __restrict__ h_q, uint8_t* __restrict__ h_s, int H, int I,
    int K) {
  __shared__ float red[WAVES * 16];
  extern __shared__ __attribute__((aligned(16))) uint8_t sS[];   // [256 weight rows][H/32] E8M0
  // grid-stride over the list slots (the grid is capped; slots past a list's
  // device-side count are empty); every thread walks the same slots
  for (int y = blockIdx.y; y < lists.cap0 + lists.cap1; y += gridDim.y) {
    const int l = y >= lists.cap0;
    const int item = y - (l ? lists.cap0 : 0);
    if (item >= lists.n_items[l][0]) continue;
    w13_small_unit<WAVES>(lists.items[l][item], lists.rows[l], blockIdx.x, offsets, sorted_pairs, x_q, x_s, w13,
                          w13_s, h_q, h_s, H, I, K, sS, red);
  }
}

template <int NF>
__global__ __launch_bounds__(kThreads) void k_w2_small(
    const SmallLists lists,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
    const uint8_t* __restrict__ h_q, const uint8_t* __restrict__ h_s, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ w2_s, uint16_t* __restrict__ o, uint8_t* __restrict__ os, int H, int I) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sS[];   // [256 weight rows][I/32] E8M0
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_wave = blockIdx.x * 64 * NF + wave * 16 * NF;
  for (int y = blockIdx.y; y < lists.cap0 + lists.cap1; y += gridDim.y) {   // as in k_w13_small
    const int l = y >= lists.cap0;
    const int item = y - (l ? lists.cap0 : 0);
    if (item >= lists.n_items[l][0]) continue;
    w2_small_wave<NF>(lists.items[l][item], lists.rows[l], n_wave, offsets, sorted_pairs, h_q, h_s, w2, w2_s, o, os,
                      H, I, sS + wave * staged_bytes(16 * NF * (I / 32)));
  }
}

}  // namespace

hipError_t launch_w13_small(const moe_dims& d, const SmallLists& lists, const int32_t* offsets,
                            const int32_t* sorted_pairs,
                            const uint8_t* x_q, const uint8_t* x_s, const uint8_t* w13, const uint8_t* w13_s,
                            uint8_t* h_q, uint8_t* h_s, hipStream_t s) {
  const int64_t max_items = (int64_t)lists.cap0 + lists.cap1;
  if (max_items <= 0) return hipSuccess;
  constexpr int WAVES = kW13Waves;
  dim3 grid(d.I / 128, (unsigned)(max_items < kMaxSlotRows ? max_items : kMaxSlotRows));
  // weight scales in LDS: per wave two runs of 128/WAVES rows x H/32 bytes
  const size_t lds = (size_t)WAVES * 2 * staged_bytes(128 / WAVES * (d.H / 32));
  hipLaunchKernelGGL(k_w13_small<WAVES>, grid, dim3(WAVES * 64), lds, s, lists,
                     offsets, sorted_pairs,
                     x_q, x_s, w13, w13_s, h_q, h_s, d.H, d.I, d.K);
  return hipGetLastError();
}

hipError_t launch_w2_small(const moe_dims& d, const SmallLists& lists, const int32_t* offsets,
                           const int32_t* sorted_pairs,
                           const uint8_t* h_q, const uint8_t* h_s, const uint8_t* w2, const uint8_t* w2_s,
                           uint16_t* o, uint8_t* os, hipStream_t s) {
  const int64_t max_items = (int64_t)lists.cap0 + lists.cap1;
  if (max_items <= 0) return hipSuccess;
  constexpr int NF = kW2Frags;
  dim3 grid((unsigned)ceil_div(d.H, 64 * NF), (unsigned)(max_items < kMaxSlotRows ? max_items : kMaxSlotRows));
  // weight scales in LDS: per wave one run of 16*NF rows x I/32 bytes
  const size_t lds = (size_t)(kThreads / 64) * staged_bytes(16 * NF * (d.I / 32));
  hipLaunchKernelGGL(k_w2_small<NF>, grid, dim3(kThreads), lds, s, lists,
                     offsets, sorted_pairs,
                     h_q, h_s, w2, w2_s, o, os, d.H, d.I);
  return hipGetLastError();
}

}  // namespace moe
