// C ABI of the routed MoE FFN (declared in include/moe_mxfp4.h): argument checks,
// workspace carving and the launch sequence. Nothing here allocates, synchronizes
// or reads device memory, so every call is an enqueue on the caller's stream.
#include <mutex>

#include "host_internal.h"

namespace moe {

size_t ffn_ws_layout(const moe_dims& d, void* base, FfnWs* out) {
  const int64_t T = d.T, H = d.H, I = d.I, P = (int64_t)d.T * d.K, Is = d.Is;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + (bytes ? bytes : 1), 256);
    return o;
  };
  const size_t o_xq = take((size_t)(T * H));
  const size_t o_xs = take((size_t)(T * H / 128));
  const size_t o_hq = take((size_t)(P * I) * (bf16_rows(d) ? 2 : 1));   // bf16 activations: bf16 rows
  const size_t o_hs = take((size_t)(P * I / 128));
  const size_t o_o = take(sizeof(uint16_t) * (size_t)(P * H));
  const size_t o_os = take((size_t)(P * H / 32));
  const size_t o_shq = take((size_t)(T * Is));
  const size_t o_shs = take((size_t)(T * Is / 128));
  const size_t o_so = take(Is ? sizeof(uint16_t) * (size_t)(T * H) : 0);
  const size_t o_sos = take(Is ? (size_t)(T * H / 32) : 0);
  const size_t o_xhat = take(Is ? sizeof(uint16_t) * (size_t)(T * H) : 0);
  const size_t o_w13s = take(Is ? sizeof(uint16_t) * (size_t)(2 * Is * H) : 0);
  const size_t o_sync = take(sizeof(int32_t) * chain_sync_words(d));
  if (out) {
    char* b = static_cast<char*>(base);
    out->x_q = reinterpret_cast<uint8_t*>(b + o_xq);
    out->x_s = reinterpret_cast<uint8_t*>(b + o_xs);
    out->h_q = reinterpret_cast<uint8_t*>(b + o_hq);
    out->h_s = reinterpret_cast<uint8_t*>(b + o_hs);
    out->o = reinterpret_cast<uint16_t*>(b + o_o);
    out->os = reinterpret_cast<uint8_t*>(b + o_os);
    out->sh_q = reinterpret_cast<uint8_t*>(b + o_shq);
    out->sh_s = reinterpret_cast<uint8_t*>(b + o_shs);
    out->so = reinterpret_cast<uint16_t*>(b + o_so);
    out->sos = reinterpret_cast<uint8_t*>(b + o_sos);
    out->x_hat = reinterpret_cast<uint16_t*>(b + o_xhat);
    out->w13s_bf16 = reinterpret_cast<uint16_t*>(b + o_w13s);
    out->sync = reinterpret_cast<int32_t*>(b + o_sync);
  }
  return off;
}

namespace {

int validate(const moe_dims* d) {
  if (!d) return MOE_EINVAL;
  if (d->T < 0 || d->H <= 0 || d->I <= 0 || d->E < 1 || d->E > kMaxExperts || d->K < 1 || d->K > kMaxTopK ||
      d->Is < 0 || d->small_max < 0 || (d->flags & ~(MOE_FLAG_DECODE_CHAIN | MOE_FLAG_A16 | MOE_FLAG_NVFP4)) != 0 ||
      d->tile_w13 < -1 || d->tile_w13 > kLargeRows || d->tile_w2 < -1 || d->tile_w2 > kLargeRows)
    return MOE_EINVAL;
  if (d->H % 128 || d->I % 128 || d->Is % 128) return MOE_EUNSUPPORTED;
  if ((int64_t)d->T * d->K > (int64_t)1 << 30) return MOE_EUNSUPPORTED;
  if (d->H > (1 << 20) || d->I > (1 << 20) || d->Is > (1 << 20)) return MOE_EUNSUPPORTED;
  // the small-M kernels stage a workgroup's weight scales in LDS (8 H or 8 I bytes)
  if (d->H > kMaxSmallDim || d->I > kMaxSmallDim) return MOE_EUNSUPPORTED;
  // kernels address activations, SwiGLU outputs and one expert's weights with
  // 32-bit byte offsets
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)d->T * d->H >= lim || (int64_t)d->T * d->K * d->I >= lim || (int64_t)d->I * d->H >= lim ||
      (int64_t)d->T * d->Is >= lim)
    return MOE_EUNSUPPORTED;
  // bf16 activations: no shared expert; 2-byte activation and SwiGLU rows
  if (bf16_rows(*d) && (d->Is > 0 || 2 * (int64_t)d->T * d->H >= lim || 2 * (int64_t)d->T * d->K * d->I >= lim))
    return MOE_EUNSUPPORTED;
  return MOE_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

inline void record(const moe_debug* dbg, int which, hipStream_t s) {
  if (dbg && dbg->events && dbg->events[which]) hipEventRecord((hipEvent_t)dbg->events[which], s);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int moe_validate(const moe_dims* dims) { return validate(dims); }

size_t moe_plan_workspace_bytes(const moe_dims* dims) {
  if (validate(dims) != MOE_OK) return 0;
  return plan_ws_layout(*dims, nullptr, nullptr);
}

size_t moe_ffn_workspace_bytes(const moe_dims* dims) {
  if (validate(dims) != MOE_OK) return 0;
  return ffn_ws_layout(*dims, nullptr, nullptr);
}

int moe_plan(const moe_dims* dims, const int32_t* topk_ids, int32_t* expert_offsets, int32_t* sorted_pairs,
             int32_t* pair_rows, int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate(dims);
  if (rc != MOE_OK) return rc;
  const bool any = dims->T > 0;
  if (!expert_offsets || !status || !ws || (any && (!topk_ids || !sorted_pairs || !pair_rows))) return MOE_EINVAL;
  PlanWs pw;
  if (ws_bytes < plan_ws_layout(*dims, ws, &pw)) return MOE_EWORKSPACE;
  return hip_status(launch_plan(*dims, topk_ids, expert_offsets, sorted_pairs, pair_rows, status, pw,
                                (hipStream_t)stream));
}

int moe_quant_act(const moe_dims* dims, const uint16_t* x, uint8_t* x_q, uint8_t* x_s, void* stream) {
  int rc = validate(dims);
  if (rc != MOE_OK) return rc;
  if (dims->T == 0) return MOE_OK;
  if (!x || !x_q || !x_s) return MOE_EINVAL;
  return hip_status(launch_quant_act(x, x_q, x_s, dims->T, dims->H, (hipStream_t)stream));
}

int moe_pack_weights(const moe_dims* dims, const uint8_t* w13, uint8_t* w13_packed, const uint8_t* w2,
                     uint8_t* w2_packed, void* stream) {
  int rc = validate(dims);
  if (rc != MOE_OK) return rc;
  if (!w13 != !w13_packed || !w2 != !w2_packed) return MOE_EINVAL;
  if ((w13 && w13 == w13_packed) || (w2 && w2 == w2_packed)) return MOE_EINVAL;   // not in place
  const moe_dims& d = *dims;
  hipStream_t s = (hipStream_t)stream;
  if (w13 && launch_pack_weights(w13, w13_packed, (int64_t)d.E * 2 * d.I, d.H, s) != hipSuccess) return MOE_EHIP;
  if (w2 && launch_pack_weights(w2, w2_packed, (int64_t)d.E * d.H, d.I, s) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

}  // extern "C"

namespace moe {
namespace {

// Argument checks of moe_ffn / moe_ffn_static / moe_ffn_nvfp4 that need no workspace.
int ffn_args(const moe_dims* dims, const uint16_t* x, const float* topk_weights, const int32_t* expert_offsets,
             const int32_t* sorted_pairs, const int32_t* pair_rows, const void* plan_ws, const uint8_t* w13,
             const uint8_t* w13_s, const uint8_t* w2, const uint8_t* w2_s, const moe_shared* shared,
             const uint16_t* y) {
  int rc = validate(dims);
  if (rc != MOE_OK) return rc;
  const moe_dims& d = *dims;
  if (d.T == 0) return MOE_OK;
  if (!x || !topk_weights || !expert_offsets || !sorted_pairs || !pair_rows || !plan_ws || !w13 || !w13_s || !w2 ||
      !w2_s || !y)
    return MOE_EINVAL;
  const bool use_shared = shared != nullptr && d.Is > 0;
  if (use_shared && (!shared->w13s || !shared->w13s_s || !shared->w2s || !shared->w2s_s)) return MOE_EINVAL;
  if (use_shared && (!dense_path_supported(d) || (int64_t)d.T * d.H >= ((int64_t)1 << 30)))
    return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// The launch sequence of the FFN on a checked argument set and a workspace of at
// least ffn_ws_layout(d) bytes.
// w13_gs / w2_gs: NVFP4's per-expert tensor scales (null for MXFP4 weights).
int ffn_enqueue(const moe_dims& d, const uint16_t* x, const float* topk_weights, const int32_t* expert_offsets,
                const int32_t* sorted_pairs, const int32_t* pair_rows, const void* plan_ws, const uint8_t* w13,
                const uint8_t* w13_s, const uint8_t* w2, const uint8_t* w2_s, const moe_shared* shared, uint16_t* y,
                const moe_debug* dbg, void* ws, hipStream_t s, const float* w13_gs = nullptr,
                const float* w2_gs = nullptr) {
  const bool use_shared = shared != nullptr && d.Is > 0;
  FfnWs fw;
  ffn_ws_layout(d, ws, &fw);
  PlanWs pw;
  plan_ws_layout(d, const_cast<void*>(plan_ws), &pw);
  uint8_t* x_q = dbg && dbg->x_q ? dbg->x_q : fw.x_q;
  uint8_t* x_s = dbg && dbg->x_s ? dbg->x_s : fw.x_s;
  uint8_t* h_q = dbg && dbg->h_q ? dbg->h_q : fw.h_q;
  uint8_t* h_s = dbg && dbg->h_s ? dbg->h_s : fw.h_s;

  const int64_t P = (int64_t)d.T * d.K;
  if (bf16_rows(d)) {
    // bf16 activations: no quantization; every item list walked in 16-row tiles
    uint16_t* h = dbg && dbg->h_q ? reinterpret_cast<uint16_t*>(dbg->h_q) : reinterpret_cast<uint16_t*>(fw.h_q);
    const SmallLists sl = long_items_first(pw.large_items, pw.hdr + 1, pw.large_cap, kLargeRows,
                                           small_lists(pw.small_items, pw.hdr + 0, pw.small_cap, kSmallRows));
    const SmallLists sxl = small_lists(pw.xl_items, pw.hdr + 2, pw.xl_cap, kXlRows);
    record(dbg, MOE_EV_START, s);
    record(dbg, MOE_EV_QUANT_DONE, s);
    hipError_t err = launch_w13_a16(d, sl, expert_offsets, sorted_pairs, x, w13, w13_s, w13_gs, h, s);
    if (err == hipSuccess && P > kXlRows / 2)
      err = launch_w13_a16(d, sxl, expert_offsets, sorted_pairs, x, w13, w13_s, w13_gs, h, s);
    if (err != hipSuccess) return MOE_EHIP;
    record(dbg, MOE_EV_W13_DONE, s);
    err = launch_w2_a16(d, sl, expert_offsets, sorted_pairs, h, w2, w2_s, w2_gs, fw.o, fw.os, s);
    if (err == hipSuccess && P > kXlRows / 2)
      err = launch_w2_a16(d, sxl, expert_offsets, sorted_pairs, h, w2, w2_s, w2_gs, fw.o, fw.os, s);
    if (err != hipSuccess) return MOE_EHIP;
    record(dbg, MOE_EV_W2_DONE, s);
    record(dbg, MOE_EV_SHARED_DONE, s);
    err = launch_combine(fw.o, fw.os, topk_weights, pair_rows, nullptr, nullptr, y, d.T, d.H, d.K, s);
    if (err != hipSuccess) return MOE_EHIP;
    record(dbg, MOE_EV_END, s);
    return MOE_OK;
  }
  // Decode shapes on request (every item walkable in 16-row tiles): one persistent
  // launch runs W13, W2 and the combine, with the shared expert ahead of it
  const bool chain = (d.flags & MOE_FLAG_DECODE_CHAIN) && P <= kFoldPairs;
  record(dbg, MOE_EV_START, s);
  hipError_t err = launch_quant_act(x, x_q, x_s, d.T, d.H, s, use_shared ? fw.x_hat : nullptr,
                                    chain ? fw.sync : nullptr, chain ? (int)chain_sync_words(d) : 0);
  if (err != hipSuccess) return MOE_EHIP;
  record(dbg, MOE_EV_QUANT_DONE, s);
  if (chain) {
    if (use_shared) {
      uint8_t* sh_q = dbg && dbg->sh_q ? dbg->sh_q : fw.sh_q;
      uint8_t* sh_s = dbg && dbg->sh_s ? dbg->sh_s : fw.sh_s;
      err = launch_shared13_bf16(d, fw.x_hat, shared->w13s, shared->w13s_s, fw.w13s_bf16, sh_q, sh_s, s);
      if (err != hipSuccess) return MOE_EHIP;
      err = shared2_fewk_supported(d)
                ? launch_shared2_fewk(d, sh_q, sh_s, shared->w2s, shared->w2s_s, fw.so, fw.sos, s)
                : launch_shared2(d, sh_q, sh_s, shared->w2s, shared->w2s_s, fw.so, fw.sos, s);
      if (err != hipSuccess) return MOE_EHIP;
    }
    record(dbg, MOE_EV_SHARED_DONE, s);
    err = launch_decode_chain(d, pw, expert_offsets, sorted_pairs, pair_rows, x_q, x_s, w13, w13_s, h_q, h_s, w2,
                              w2_s, fw.o, fw.os, topk_weights, use_shared ? fw.so : nullptr,
                              use_shared ? fw.sos : nullptr, y, fw.sync, s);
    if (err != hipSuccess) return MOE_EHIP;
    record(dbg, MOE_EV_W13_DONE, s);
    record(dbg, MOE_EV_W2_DONE, s);
    record(dbg, MOE_EV_END, s);
    return MOE_OK;
  }

  // Work lists: 16-row items (small experts), 256-row items and 128-row items
  // (remainders of 1..128 rows, by rows). A 256-row item needs an expert with more
  // than 128 pairs and a 128-row item one with more than small_max, so launches that
  // could only find empty lists are skipped. Exact-shape tiling per GEMM: the
  // 128-row items of at most tile_small_rows(d, GEMM) rows (a prefix, hdr[3] for
  // W13 and hdr[4] for W2) ride in that GEMM's small-M launch as 16-row tiles, the
  // rest run as 128-row tiles from the cut on; up to kFoldPairs pairs (or without
  // large-M tiles) all of them are small.
  const bool large = large_path_supported(d);
  const bool any_xl = P > kXlRows / 2, any_l = P > small_max_of(d);
  const int t13 = tile_small_rows(d, true), t2 = tile_small_rows(d, false);
  auto lists_for = [&](int t, const int32_t* cut) {
    const SmallLists sl = small_lists(pw.small_items, pw.hdr + 0, pw.small_cap, kSmallRows);
    return any_l && t > 0 ? long_items_first(pw.large_items, cut, pw.large_cap, kLargeRows, sl) : sl;
  };
  const SmallLists sl13 = lists_for(t13, pw.hdr + 3), sl2 = lists_for(t2, pw.hdr + 4);
  const SmallLists sxl = small_lists(pw.xl_items, pw.hdr + 2, pw.xl_cap, kXlRows);

  err = launch_w13_small(d, sl13, expert_offsets, sorted_pairs, x_q, x_s, w13, w13_s, h_q, h_s, s);
  if (err != hipSuccess) return MOE_EHIP;
  if (any_xl) {
    if (large && xl13_supported(d))
      err = launch_w13_xl(d, pw.xl_items, pw.hdr + 2, pw.xl_cap, expert_offsets, sorted_pairs, x_q, x_s, w13,
                          w13_s, h_q, h_s, s);
    else if (large)
      err = launch_w13_large(d, pw.xl_items, pw.hdr + 2, pw.xl_cap, kXlRows, expert_offsets, sorted_pairs, x_q,
                             x_s, w13, w13_s, h_q, h_s, s);
    else   // shapes the large-M tiles do not cover: the small-M kernel walks the items
      err = launch_w13_small(d, sxl, expert_offsets, sorted_pairs, x_q, x_s, w13, w13_s, h_q, h_s, s);
    if (err != hipSuccess) return MOE_EHIP;
  }
  if (any_l && t13 < kLargeRows) {
    err = launch_w13_large(d, pw.large_items, pw.hdr + 1, pw.large_cap, kLargeRows, expert_offsets, sorted_pairs,
                           x_q, x_s, w13, w13_s, h_q, h_s, s, pw.hdr + 3);
    if (err != hipSuccess) return MOE_EHIP;
  }
  record(dbg, MOE_EV_W13_DONE, s);

  err = launch_w2_small(d, sl2, expert_offsets, sorted_pairs, h_q, h_s, w2, w2_s, fw.o, fw.os, s);
  if (err != hipSuccess) return MOE_EHIP;
  const bool fewk = large && fewk2_supported(d);
  if (any_xl) {
    if (fewk)
      err = launch_w2_fewk(d, pw.xl_items, pw.hdr + 2, pw.xl_cap, kXlRows, expert_offsets, sorted_pairs, h_q, h_s,
                           w2, w2_s, fw.o, fw.os, s);
    else if (large && xl2_supported(d))
      err = launch_w2_xl(d, pw.xl_items, pw.hdr + 2, pw.xl_cap, expert_offsets, sorted_pairs, h_q, h_s, w2, w2_s,
                         fw.o, fw.os, s);
    else if (large)
      err = launch_w2_large(d, pw.xl_items, pw.hdr + 2, pw.xl_cap, kXlRows, expert_offsets, sorted_pairs, h_q, h_s,
                            w2, w2_s, fw.o, fw.os, s);
    else
      err = launch_w2_small(d, sxl, expert_offsets, sorted_pairs, h_q, h_s, w2, w2_s, fw.o, fw.os, s);
    if (err != hipSuccess) return MOE_EHIP;
  }
  if (any_l && t2 < kLargeRows) {
    if (fewk)
      err = launch_w2_fewk(d, pw.large_items, pw.hdr + 1, pw.large_cap, kLargeRows, expert_offsets, sorted_pairs,
                           h_q, h_s, w2, w2_s, fw.o, fw.os, s, pw.hdr + 4);
    else
      err = launch_w2_large(d, pw.large_items, pw.hdr + 1, pw.large_cap, kLargeRows, expert_offsets, sorted_pairs,
                            h_q, h_s, w2, w2_s, fw.o, fw.os, s, pw.hdr + 4);
    if (err != hipSuccess) return MOE_EHIP;
  }
  record(dbg, MOE_EV_W2_DONE, s);

  if (use_shared) {
    uint8_t* sh_q = dbg && dbg->sh_q ? dbg->sh_q : fw.sh_q;
    uint8_t* sh_s = dbg && dbg->sh_s ? dbg->sh_s : fw.sh_s;
    err = launch_shared13_bf16(d, fw.x_hat, shared->w13s, shared->w13s_s, fw.w13s_bf16, sh_q, sh_s, s);
    if (err != hipSuccess) return MOE_EHIP;
    err = shared2_fewk_supported(d)
              ? launch_shared2_fewk(d, sh_q, sh_s, shared->w2s, shared->w2s_s, fw.so, fw.sos, s)
              : launch_shared2(d, sh_q, sh_s, shared->w2s, shared->w2s_s, fw.so, fw.sos, s);
    if (err != hipSuccess) return MOE_EHIP;
  }
  record(dbg, MOE_EV_SHARED_DONE, s);

  err = launch_combine(fw.o, fw.os, topk_weights, pair_rows, use_shared ? fw.so : nullptr, use_shared ? fw.sos : nullptr,
                       y, d.T, d.H, d.K, s);
  if (err != hipSuccess) return MOE_EHIP;
  record(dbg, MOE_EV_END, s);
  return MOE_OK;
}

// ---------------------------------------------------------------- static scratch
// The workspace of moe_ffn_static: one array per GPU, loaded with the library's
// code object and held until the process ends. Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the device symbol); it
// uses the address hipGetSymbolAddress returns for the current device, looked up
// once per device on that device's first call.
constexpr size_t kStaticScratchBytes = MOE_FFN_STATIC_MAX_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch` (nullptr and the HIP error on failure).
void* scratch_ptr(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_ffn(const moe_dims* dims, const uint16_t* x, const float* topk_weights, const int32_t* expert_offsets,
            const int32_t* sorted_pairs, const int32_t* pair_rows, const void* plan_ws, const uint8_t* w13,
            const uint8_t* w13_s, const uint8_t* w2, const uint8_t* w2_s, const moe_shared* shared, uint16_t* y,
            const moe_debug* dbg, void* ws, size_t ws_bytes, void* stream) {
  int rc = ffn_args(dims, x, topk_weights, expert_offsets, sorted_pairs, pair_rows, plan_ws, w13, w13_s, w2, w2_s,
                    shared, y);
  if (rc == MOE_OK && (dims->flags & MOE_FLAG_NVFP4)) return MOE_EINVAL;   // needs moe_ffn_nvfp4's tensor scales
  if (rc != MOE_OK || dims->T == 0) return rc;
  if (!ws) return MOE_EINVAL;
  if (ws_bytes < ffn_ws_layout(*dims, nullptr, nullptr)) return MOE_EWORKSPACE;
  return ffn_enqueue(*dims, x, topk_weights, expert_offsets, sorted_pairs, pair_rows, plan_ws, w13, w13_s, w2, w2_s,
                     shared, y, dbg, ws, (hipStream_t)stream);
}

int moe_ffn_static(const moe_dims* dims, const uint16_t* x, const float* topk_weights,
                   const int32_t* expert_offsets, const int32_t* sorted_pairs, const int32_t* pair_rows,
                   const void* plan_ws, const uint8_t* w13, const uint8_t* w13_s, const uint8_t* w2,
                   const uint8_t* w2_s, const moe_shared* shared, uint16_t* y, const moe_debug* dbg, void* stream) {
  int rc = ffn_args(dims, x, topk_weights, expert_offsets, sorted_pairs, pair_rows, plan_ws, w13, w13_s, w2, w2_s,
                    shared, y);
  if (rc == MOE_OK && (dims->flags & MOE_FLAG_NVFP4)) return MOE_EINVAL;
  if (rc != MOE_OK || dims->T == 0) return rc;
  if (ffn_ws_layout(*dims, nullptr, nullptr) > kStaticScratchBytes) return MOE_ESCRATCH;
  hipError_t err;
  void* ws = scratch_ptr(&err);
  if (!ws) return MOE_EHIP;
  // every workspace byte the kernels read is written earlier in the same call, so
  // nothing is cleared
  return ffn_enqueue(*dims, x, topk_weights, expert_offsets, sorted_pairs, pair_rows, plan_ws, w13, w13_s, w2, w2_s,
                     shared, y, dbg, ws, (hipStream_t)stream);
}

int moe_ffn_nvfp4(const moe_dims* dims, const uint16_t* x, const float* topk_weights, const int32_t* expert_offsets,
                  const int32_t* sorted_pairs, const int32_t* pair_rows, const void* plan_ws, const uint8_t* w13,
                  const uint8_t* w13_s, const float* w13_gs, const uint8_t* w2, const uint8_t* w2_s,
                  const float* w2_gs, uint16_t* y, const moe_debug* dbg, void* ws, size_t ws_bytes, void* stream) {
  int rc = ffn_args(dims, x, topk_weights, expert_offsets, sorted_pairs, pair_rows, plan_ws, w13, w13_s, w2, w2_s,
                    nullptr, y);
  if (rc == MOE_OK && !(dims->flags & MOE_FLAG_NVFP4)) return MOE_EINVAL;
  if (rc != MOE_OK || dims->T == 0) return rc;
  if (!w13_gs || !w2_gs || !ws) return MOE_EINVAL;
  if (ws_bytes < ffn_ws_layout(*dims, nullptr, nullptr)) return MOE_EWORKSPACE;
  return ffn_enqueue(*dims, x, topk_weights, expert_offsets, sorted_pairs, pair_rows, plan_ws, w13, w13_s, w2, w2_s,
                     nullptr, y, dbg, ws, (hipStream_t)stream, w13_gs, w2_gs);
}

const char* moe_status_string(int code) {
  switch (code) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: null pointer or dimension out of range";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: shape outside what the kernels support";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: a HIP launch failed";
    case MOE_ESCRATCH: return "MOE_ESCRATCH: the call needs more workspace than moe_ffn_static's static scratch holds";
    default: return "unknown moe status code";
  }
}

}  // extern "C"
