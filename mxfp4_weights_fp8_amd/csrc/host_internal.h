// Host-side internals shared by the C-ABI layer and the kernel launchers:
// tiling constants, workspace layouts and launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_mxfp4.h"

namespace moe {

// ---------------------------------------------------------------- constants
constexpr int kSmallRows = 16;       // rows per small-M tile (MFMA N side)
constexpr int kDefaultSmallMax = 16; // experts with <= this many pairs take the small-M path
constexpr int kLargeRows = 128;      // rows per large-M tile
constexpr int kXlRows = 256;         // rows per extra-large (256 x 256) large-M tile
constexpr int kPlanChunk = 2048;     // pairs per route-planner block
constexpr int kMaxExperts = 4096;
constexpr int kMaxTopK = 64;
constexpr int kFoldPairs = 512;      // up to this many pairs the small-M launch also takes the 128-row items
constexpr int kMaxSmallDim = 16384;  // H and I: the small-M kernels keep 8*H (W13) or 4*I (W2) bytes of scales in LDS

inline int small_max_of(const moe_dims& d) { return d.small_max > 0 ? d.small_max : kDefaultSmallMax; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Upper bounds on the tile work lists the planner builds (host-side, from dims
// only, so grids can be sized without reading device data).
inline int64_t small_items_bound(const moe_dims& d) {
  int64_t P = (int64_t)d.T * d.K;
  int64_t sm = small_max_of(d);
  int64_t experts = P < d.E ? P : d.E;
  // each small expert (1 <= M <= sm) yields ceil(M / kSmallRows) tiles
  return sm <= kSmallRows ? experts : experts + P / kSmallRows;
}
// Experts with more than small_max pairs split into 256-row items (the last one
// when more than 128 rows remain) and at most one 128-row item (a remainder of
// 1..128 rows).
inline int64_t big_experts_bound(const moe_dims& d) {
  int64_t P = (int64_t)d.T * d.K;
  int64_t big = P / (small_max_of(d) + 1);   // experts with more than small_max pairs
  return big > d.E ? d.E : big;
}
inline int64_t large_items_bound(const moe_dims& d) { return big_experts_bound(d); }
// Every 256-row item holds more than 128 rows (the full ones 256, an expert's last
// one 129..256), so there are at most P / 129 of them; and at most P / 256 full ones
// plus one last one per expert above small_max. The smaller bound sizes the list and
// the grids (a launch whose workgroups all find no item still costs microseconds).
inline int64_t xl_items_bound(const moe_dims& d) {
  const int64_t P = (int64_t)d.T * d.K;
  const int64_t by_rows = P / (kXlRows / 2 + 1), by_experts = P / kXlRows + big_experts_bound(d);
  return by_rows < by_experts ? by_rows : by_experts;
}

// ---------------------------------------------------------------- plan workspace
// int32 header, then the two tile lists (int2 = {expert, first row}), then the
// planner's per-block scratch.
struct PlanWs {
  int32_t* hdr;           // [0] small, [1] 128-row, [2] 256-row item counts; [3] / [4] the 128-row
                          // items (rows ascending) that W13 / W2 walk as 16-row tiles
  int2* small_items;
  int2* large_items;      // 128-row items
  int2* xl_items;         // 256-row items
  int32_t* local_rank;    // [P]
  int32_t* block_counts;  // [E][NB]
  int32_t* block_base;    // [E][NB]
  int64_t small_cap, large_cap, xl_cap, nb;
};
size_t plan_ws_layout(const moe_dims& d, void* base, PlanWs* out);

// Exact-shape tiling per GEMM: the 128-row items (1..128 rows each) of at most this
// many rows run W13 (w13) or W2 as 16-row small-M tiles; the planner orders those
// items by rows and counts them into hdr[3] / hdr[4]. 128 = all of them (batches of
// at most kFoldPairs pairs, or shapes without large-M tiles); else moe_dims.tile_w13
// / tile_w2, or the tuned table for (H, I).
int tile_small_rows(const moe_dims& d, bool w13);

// ---------------------------------------------------------------- ffn workspace
// Activations and SwiGLU rows stay bf16 (no FP8 quantization): MOE_FLAG_A16 and
// MOE_FLAG_NVFP4.
inline bool bf16_rows(const moe_dims& d) { return (d.flags & (MOE_FLAG_A16 | MOE_FLAG_NVFP4)) != 0; }

struct FfnWs {
  uint8_t* x_q;   // [T, H]
  uint8_t* x_s;   // [T, H/128]
  uint8_t* h_q;   // [P, I]
  uint8_t* h_s;   // [P, I/128]
  uint16_t* o;    // [P, H] per-pair W2 outputs (fp16 codes of o * 2^-e), slot p = t*K + j
  uint8_t* os;    // [P, H/32] their scales (byte e + 127 per 32 columns)
  uint8_t* sh_q;  // [T, Is]
  uint8_t* sh_s;  // [T, Is/128]
  uint16_t* so;   // [T, H] shared-expert output (fp16 codes)
  uint8_t* sos;   // [T, H/32] their scales
  uint16_t* x_hat;      // [T, H] bf16 quantized activations (shared expert only)
  uint16_t* w13s_bf16;  // [2Is, H] bf16 shared gate/up weights, block scales folded in
  int32_t* sync;        // [chain_sync_words] counters of the decode chain, zeroed by the quantizer
};
size_t ffn_ws_layout(const moe_dims& d, void* base, FfnWs* out);

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.
hipError_t launch_plan(const moe_dims& d, const int32_t* ids, int32_t* offsets, int32_t* sorted_pairs,
                       int32_t* pair_rows, int32_t* status, const PlanWs& ws, hipStream_t s);
// Row-major E2M1 codes [rows, K/2] -> the kernel-native blocked layout (rows % 16
// == 0, K % 128 == 0).
hipError_t launch_pack_weights(const uint8_t* w, uint8_t* out, int64_t rows, int K, hipStream_t s);
// x_hat (optional): the quantized values E4M3(code) * scale as bf16 [T, H].
// zero / n_zero (optional): int32 words set to zero by the launch (counters that a
// later kernel of the same call needs at zero).
hipError_t launch_quant_act(const uint16_t* x, uint8_t* x_q, uint8_t* x_s, int T, int H, hipStream_t s,
                            uint16_t* x_hat = nullptr, int32_t* zero = nullptr, int n_zero = 0);
// Small-M kernels walk up to two work lists in one launch: workgroup row y <
// cap0 takes item y of list 0, the rest item y - cap0 of list 1; an item covers
// rows[l] routed rows in 16-row tiles (counts live on the device).
struct SmallLists {
  const int2* items[2];
  const int32_t* n_items[2];
  int cap0, cap1;
  int rows[2];
};
inline SmallLists small_lists(const int2* items, const int32_t* n_items, int64_t cap, int rows) {
  return SmallLists{{items, items}, {n_items, n_items}, (int)cap, 0, {rows, rows}};
}
// A list of items of more than 16 rows (one workgroup walks their tiles one after
// another) as list 0, ahead of the single list of `rest`: those long workgroups take
// the lowest rows y, which start first, instead of trailing the launch.
inline SmallLists long_items_first(const int2* items, const int32_t* n_items, int64_t cap, int rows,
                                   const SmallLists& rest) {
  return SmallLists{{items, rest.items[0]}, {n_items, rest.n_items[0]}, (int)cap, rest.cap0, {rows, rest.rows[0]}};
}
hipError_t launch_w13_small(const moe_dims& d, const SmallLists& lists, const int32_t* offsets,
                            const int32_t* sorted_pairs, const uint8_t* x_q, const uint8_t* x_s,
                            const uint8_t* w13, const uint8_t* w13_s, uint8_t* h_q, uint8_t* h_s, hipStream_t s);
hipError_t launch_w2_small(const moe_dims& d, const SmallLists& lists, const int32_t* offsets,
                           const int32_t* sorted_pairs, const uint8_t* h_q, const uint8_t* h_s,
                           const uint8_t* w2, const uint8_t* w2_s, uint16_t* o, uint8_t* os, hipStream_t s);
// 128-row large-M tiles; item_rows 128 or 256 (a 256-row item runs as two
// 128-row workgroups). first: the launch takes items [first[0], n_items[0]) of the
// list (null: from 0).
bool large_path_supported(const moe_dims& d);
hipError_t launch_w13_large(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                            int item_rows, const int32_t* offsets, const int32_t* sorted_pairs,
                            const uint8_t* x_q, const uint8_t* x_s, const uint8_t* w13, const uint8_t* w13_s,
                            uint8_t* h_q, uint8_t* h_s, hipStream_t s,
                            const int32_t* first = nullptr);
hipError_t launch_w2_large(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                           int item_rows, const int32_t* offsets, const int32_t* sorted_pairs,
                           const uint8_t* h_q, const uint8_t* h_s, const uint8_t* w2, const uint8_t* w2_s,
                           uint16_t* o, uint8_t* os, hipStream_t s,
                            const int32_t* first = nullptr);
// 256 x 256 large-M tiles on 256-row items (a K-step count that is a multiple of 4 and the
// large-M shape limits).
// W2 with at most 3 K steps (I <= 384): a workgroup keeps its 128 routed rows in LDS
// and walks a run of 256-column blocks.
bool fewk2_supported(const moe_dims& d);
// The shared expert's W2s with at most 3 K steps (Is <= 384): token fragments in
// registers, runs of 128-column blocks.
bool shared2_fewk_supported(const moe_dims& d);
hipError_t launch_shared2_fewk(const moe_dims& d, const uint8_t* sh_q, const uint8_t* sh_s, const uint8_t* w2s,
                               const uint8_t* w2s_s, uint16_t* so, uint8_t* sos, hipStream_t s);
hipError_t launch_w2_fewk(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                          int item_rows, const int32_t* offsets, const int32_t* sorted_pairs, const uint8_t* h_q,
                          const uint8_t* h_s, const uint8_t* w2, const uint8_t* w2_s, uint16_t* o, uint8_t* os,
                          hipStream_t s,
                            const int32_t* first = nullptr);
bool xl13_supported(const moe_dims& d);
bool xl2_supported(const moe_dims& d);
hipError_t launch_w13_xl(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                         const int32_t* offsets, const int32_t* sorted_pairs, const uint8_t* x_q,
                         const uint8_t* x_s, const uint8_t* w13, const uint8_t* w13_s, uint8_t* h_q,
                         uint8_t* h_s, hipStream_t s);
hipError_t launch_w2_xl(const moe_dims& d, const int2* items, const int32_t* n_items, int64_t max_items,
                        const int32_t* offsets, const int32_t* sorted_pairs, const uint8_t* h_q,
                        const uint8_t* h_s, const uint8_t* w2, const uint8_t* w2_s, uint16_t* o, uint8_t* os, hipStream_t s);
// Dense FP8 shared expert: W13s + SwiGLU/requant into sh_q/sh_s, then W2s into
// fp32 rows so [T, H]. Needs H/128 and Is/128 at most 64.
bool dense_path_supported(const moe_dims& d);
// The gate/up GEMM in bf16: expands w13s (FP8, 128 x 128 block scales) into
// w13s_bf16 (workspace, [2Is, H]) and multiplies by x_hat (bf16 quantized
// activations). Needs T * H < 2^30.
hipError_t launch_shared13_bf16(const moe_dims& d, const uint16_t* x_hat, const uint8_t* w13s, const uint8_t* w13s_s,
                                uint16_t* w13s_bf16, uint8_t* sh_q, uint8_t* sh_s, hipStream_t s);
hipError_t launch_shared2(const moe_dims& d, const uint8_t* sh_q, const uint8_t* sh_s, const uint8_t* w2s,
                          const uint8_t* w2s_s, uint16_t* so, uint8_t* sos, hipStream_t s);
// 4-bit weights x bf16 activations (MOE_FLAG_A16, MOE_FLAG_NVFP4): x [T, H] bf16 ->
// h [P, I] bf16 (SwiGLU output, rows in plan order) -> per-pair rows; every item
// walked in 16-row tiles. *_gs null: MXFP4 (E8M0 per 32); else NVFP4 (E4M3 per 16
// and these per-expert fp32 tensor scales).
hipError_t launch_w13_a16(const moe_dims& d, const SmallLists& lists, const int32_t* offsets,
                          const int32_t* sorted_pairs, const uint16_t* x, const uint8_t* w13, const uint8_t* w13_s,
                          const float* w13_gs, uint16_t* h, hipStream_t s);
hipError_t launch_w2_a16(const moe_dims& d, const SmallLists& lists, const int32_t* offsets,
                         const int32_t* sorted_pairs, const uint16_t* h, const uint8_t* w2, const uint8_t* w2_s,
                         const float* w2_gs, uint16_t* o, uint8_t* os, hipStream_t s);
// The persistent decode chain (W13 + SwiGLU/requant, W2 and the combine in one
// launch, per-expert and per-column-block counters in `sync`, which must be zero):
// used when every item can be walked in 16-row tiles, T*K <= kFoldPairs.
size_t chain_sync_words(const moe_dims& d);
hipError_t launch_decode_chain(const moe_dims& d, const PlanWs& pw, const int32_t* offsets,
                               const int32_t* sorted_pairs, const int32_t* pair_rows, const uint8_t* x_q,
                               const uint8_t* x_s, const uint8_t* w13, const uint8_t* w13_s, uint8_t* h_q,
                               uint8_t* h_s, const uint8_t* w2, const uint8_t* w2_s, uint16_t* o, uint8_t* os,
                               const float* topk_weights, const uint16_t* so, const uint8_t* sos, uint16_t* y,
                               int32_t* sync, hipStream_t s);
hipError_t launch_combine(const uint16_t* o, const uint8_t* os, const float* topk_weights, const int32_t* pair_rows,
                          const uint16_t* so, const uint8_t* sos,
                          uint16_t* y, int T, int H, int K, hipStream_t s);

}  // namespace moe
