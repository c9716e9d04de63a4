/*
 * moe_mxfp4.h -- C ABI of the routed Mixture-of-Experts FFN with MXFP4 expert
 * weights and online-quantized FP8 activations, for AMD Instinct MI355X (gfx950).
 *
 * The method: "Pushing the Limits of Serving DeepSeek-V4-Pro" (LMSYS blog on
 * serving DeepSeek-V4-Pro on H20; the news summary and the numbered translation
 * carry the same text). Its MoE runner keeps expert weights in MXFP4 and
 * quantizes activations to FP8 on the fly (section 2.2, capacity); runs the W13
 * (gate/up) and W2 (down) expert GEMMs, tuned separately on routed shapes
 * (section 3.3); fuses SwiGLU with the quantization that hands W2 its FP8 data
 * and scales (section 4.3); and ends in a top-k reduction plus a shared-expert add
 * (section 3.2). "Optimization progress report" (DeepSeek-V4-Flash on GB10) packs
 * the tokens by expert ahead of the MoE launch without changing the
 * token-to-expert mapping (Optimization 14) and uses a dedicated small-M tiling
 * for the 7-token verify (Optimization 06).
 *
 * Formats (OCP MX v1.0 / OCP FP8, which the pages name only as "MXFP4" and "FP8"):
 *   E2M1 weight codes, two per byte, low nibble = even K index;
 *   E8M0 scales, value 2^(code-127), one per 32 weights along K;
 *   E4M3FN activation codes (max 448), one E8M0 scale per token per 128 columns,
 *   chosen as the smallest power of two with amax <= 448 * scale, elements rounded
 *   to nearest-even;
 *   bf16 passed as uint16_t bit patterns.
 *
 * Conventions for every entry point below:
 *   - All tensor pointers are DEVICE pointers, 16-byte aligned, row-major unless
 *     stated otherwise (moe_ffn's expert weight codes are in the layout of
 *     moe_pack_weights); the caller allocates and owns every buffer. The library
 *     never allocates or frees memory and keeps no pointer past the call
 *     (moe_ffn_static alone uses a static device array of the library's own in
 *     place of a workspace; see there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on it: no host synchronization, no host
 *     read of device data, so calls can be captured into a HIP graph.
 *   - Return value: MOE_OK (0) or a negative MOE_E* code; argument checks run on
 *     the host before anything is enqueued, so an error leaves the outputs
 *     untouched. moe_status_string() names a code. Faults in device data (ids
 *     outside [0, E)) are not errors: such pairs are dropped and counted in
 *     status[0] (see moe_plan).
 *   - Results are deterministic: identical inputs give bitwise identical outputs.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* null pointer or dimension out of range */
  MOE_EUNSUPPORTED = -2,  /* shape outside what the kernels support (e.g. H % 128) */
  MOE_EWORKSPACE = -3,    /* workspace too small */
  MOE_EHIP = -4,          /* a HIP launch failed (hipGetLastError after enqueue) */
  MOE_ESCRATCH = -5       /* moe_ffn_static: the call needs more than MOE_FFN_STATIC_MAX_BYTES */
};

/* Problem dimensions.
 *   T  tokens (>= 0; T == 0 is a valid no-op)
 *   H  hidden size, multiple of 128, at most 16384 (K of W13, N of W2)
 *   I  intermediate size per expert, multiple of 128, at most 16384 (per rank for
 *      an MoE-TP slice)
 *   E  routed experts, 1..4096
 *   K  picks per token (top-k), 1..64
 *   Is shared-expert intermediate size, multiple of 128, 0 = no shared expert
 *   small_max  experts with at most this many routed pairs use the small-M
 *      (decode) tiling, larger ones the large-M (prefill) tiling; 0 selects the
 *      library default (16). moe_plan and moe_ffn must see the same value.
 *   flags  0, or MOE_FLAG_DECODE_CHAIN, MOE_FLAG_A16, MOE_FLAG_NVFP4 (below).
 *   tile_w13, tile_w2  exact-shape tiling per GEMM ("Pushing the Limits of Serving
 *      DeepSeek-V4-Pro", section 3.3: separate W13 and W2 configurations tuned on the
 *      expert sizes the routing produces). An expert above small_max pairs is split
 *      into 256-row items and at most one item of 1..128 rows (its remainder, or the
 *      whole expert when it has at most 128 pairs). Such an item of at most tile_w13
 *      (tile_w2) rows runs W13 (W2) as 16-row small-M tiles, a larger one as one
 *      128-row large-M tile. 0 selects the library's table, tuned on MI355X per
 *      (H, I); -1 sends none to the small-M tiles; 1..128 is the row limit itself.
 *      Results are bitwise identical for every choice (each dot product is summed in
 *      the same order by every tiling). moe_plan and moe_ffn must see the same values. */
typedef struct moe_dims {
  int32_t T, H, I, E, K, Is;
  int32_t small_max;
  int32_t flags;
  int32_t tile_w13, tile_w2;
} moe_dims;

/* moe_ffn at decode shapes (T*K <= 512): run W13 + SwiGLU/requant, W2 and the
 * top-k combine as ONE persistent launch in which each expert's W2 work starts
 * when its W13 work has signalled and each 128-column block of y is combined by
 * the W2 unit that finishes it ("Pushing the Limits of Serving DeepSeek-V4-Pro",
 * section 4.3), instead of separate launches. Results are bitwise identical
 * either way. Measured on MI355X at the 7-token verify: 0.230 ms per step against
 * 0.219 ms with separate launches, so it is off by default. Ignored above 512
 * pairs. */
#define MOE_FLAG_DECODE_CHAIN 1

/* MXFP4 weights x bf16 activations ("MXFP4A16", the variant beside MXFP4AFP8 in
 * "Pushing the Limits of Serving DeepSeek-V4-Pro", Appendix D.2): moe_ffn does not
 * quantize x; gate/up = W13 . x with the MXFP4 weights dequantized exactly to bf16,
 * h = bf16(silu(gate) * up) (round to nearest even) is W2's operand, y as usual.
 * The same plan, weight layout and combine; no shared expert (MOE_EUNSUPPORTED);
 * T*H and T*K*I below 2^30. Every item is walked in 16-row tiles (the decode
 * tiling): HBM-bound and efficient at decode shapes, correct but slow for prefill.
 * The workspace holds bf16 SwiGLU rows; moe_debug.h_q then receives them as bf16
 * [P, I] (2 bytes per element) and x_q, x_s, h_s are not written.
 * MOE_FLAG_DECODE_CHAIN is ignored with it. */
#define MOE_FLAG_A16 2

/* NVFP4 expert weights with bf16 activations, run through moe_ffn_nvfp4 (moe_ffn
 * and moe_ffn_static return MOE_EINVAL for it). Same activation path, limits and
 * workspace as MOE_FLAG_A16 (bf16 SwiGLU rows, no shared expert). */
#define MOE_FLAG_NVFP4 4

/* Dense shared expert ("Pushing the Limits of Serving DeepSeek-V4-Pro", section
 * 3.2: its output is added to the top-k reduction with weight 1). FP8 E4M3 weights
 * with one E8M0 scale per 128x128 block:
 *   w13s   [2*Is, H]   rows [0, Is) gate, [Is, 2*Is) up
 *   w13s_s [2*Is/128, H/128]
 *   w2s    [H, Is]
 *   w2s_s  [H/128, Is/128] */
typedef struct moe_shared {
  const uint8_t* w13s;
  const uint8_t* w13s_s;
  const uint8_t* w2s;
  const uint8_t* w2s_s;
} moe_shared;

/* Optional inspection / timing outputs of moe_ffn (any member may be NULL).
 *   x_q [T, H], x_s [T, H/128]      activation codes and scales
 *   h_q [P, I], h_s [P, I/128]      SwiGLU-output codes and scales, rows in plan
 *                                   order (row r belongs to pair sorted_pairs[r]);
 *                                   P = T*K; rows past expert_offsets[E] unwritten
 *   sh_q [T, Is], sh_s [T, Is/128]  the shared expert's SwiGLU-output codes/scales
 *   When given, the kernels write these buffers instead of the workspace copies.
 *   events: if non-NULL, an array of MOE_FFN_NUM_EVENTS hipEvent_t (as void*)
 *   recorded on `stream` at the stage boundaries listed below. */
enum {
  MOE_EV_START = 0,       /* before activation quantization */
  MOE_EV_QUANT_DONE,      /* after activation quantization */
  MOE_EV_W13_DONE,        /* after the W13 GEMM + SwiGLU + requant kernels */
  MOE_EV_W2_DONE,         /* after the W2 GEMM kernels */
  MOE_EV_SHARED_DONE,     /* after the shared expert (same as W2_DONE without one) */
  MOE_EV_END,             /* after the top-k combine */
  MOE_FFN_NUM_EVENTS
};
typedef struct moe_debug {
  uint8_t* x_q;
  uint8_t* x_s;
  uint8_t* h_q;
  uint8_t* h_s;
  uint8_t* sh_q;
  uint8_t* sh_s;
  void* const* events;
} moe_debug;

/* Host-only argument check of a dims struct: MOE_OK, MOE_EINVAL or MOE_EUNSUPPORTED. */
int moe_validate(const moe_dims* dims);

/* Bytes of device workspace moe_plan needs (and moe_ffn reads back as plan_ws). */
size_t moe_plan_workspace_bytes(const moe_dims* dims);

/* Route plan ("Optimization progress report", Optimization 14: pack tokens by
 * expert ahead of the MoE launch, token-to-expert mapping unchanged).
 *   topk_ids       [T, K] int32   expert of pick j of token t; pair p = t*K + j
 *   expert_offsets [E+1]  int32   out: exclusive scan of per-expert pair counts
 *   sorted_pairs   [P]    int32   out: pair ids ordered by expert, then by p
 *                                 (stable); entries past expert_offsets[E] are -1
 *   pair_rows      [P]    int32   out: position of pair p in sorted_pairs, -1 if dropped
 *   status         [1]    int32   out: number of pairs dropped for an id outside [0, E)
 *   ws, ws_bytes                  plan workspace (>= moe_plan_workspace_bytes);
 *                                 holds the tile work lists and must be passed,
 *                                 unchanged, to moe_ffn as plan_ws.
 * Errors: MOE_EINVAL (null pointer, bad dims), MOE_EWORKSPACE, MOE_EHIP. */
int moe_plan(const moe_dims* dims, const int32_t* topk_ids, int32_t* expert_offsets,
             int32_t* sorted_pairs, int32_t* pair_rows, int32_t* status, void* ws,
             size_t ws_bytes, void* stream);

/* Online FP8 activation quantization ("Pushing the Limits of Serving
 * DeepSeek-V4-Pro", section 2.2): x bf16 [T, H] -> x_q E4M3 [T, H] and x_s E8M0
 * [T, H/128] (one scale per token per 128 columns). moe_ffn runs the same kernel;
 * this entry point exposes it alone. Errors: MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP. */
int moe_quant_act(const moe_dims* dims, const uint16_t* x, uint8_t* x_q, uint8_t* x_s,
                  void* stream);

/* Kernel-native layout of the MXFP4 expert weights, converted once when the
 * weights are loaded (the scales keep their row-major layout). A row-major code
 * tensor w[R][K/2] (R rows of K weights) becomes blocks of 16 rows x 128 K: block
 * (g, s), rows 16g .. 16g+15 and code bytes 64s .. 64s+63 of each row, is 1 KB at
 * byte offset g*16*(K/2) + s*1024, and inside it byte 16*(16q + c) + b holds
 * w[16g + c][64s + 16q + b] (q = 0..3, c = 0..15, b = 0..15): the order in which a
 * 64-lane wave holds a 16-row fragment of one 128-K step of the MFMA, so each
 * fragment streams as one contiguous kilobyte. Same size as the input.
 *   w13 [E, 2I, H/2] -> w13_packed (R = E*2I, K = H)
 *   w2  [E, H, I/2]  -> w2_packed  (R = E*H,  K = I)
 * Either pair may be NULL (that tensor is skipped); outputs must not alias inputs.
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP. */
int moe_pack_weights(const moe_dims* dims, const uint8_t* w13, uint8_t* w13_packed, const uint8_t* w2,
                     uint8_t* w2_packed, void* stream);

/* Bytes of device workspace moe_ffn needs for these dims. */
size_t moe_ffn_workspace_bytes(const moe_dims* dims);

/* The routed MoE FFN, y = sum_j w[t,j] * W2[e] . Q(silu(W1[e] . Q(x_t)) * (W3[e] . Q(x_t)))
 * (+ shared expert), e = topk_ids[t, j]; Q = FP8 E4M3 quantization with one
 * power-of-two scale per 128 elements; W1/W3 = W13 rows [0, I) / [I, 2I).
 * "Pushing the Limits of Serving DeepSeek-V4-Pro": MXFP4 expert weights with FP8
 * activations quantized online (section 2.2), separate W13 and W2 grouped GEMMs
 * (section 3.3), SwiGLU fused with the quantization that writes W2's FP8 operand
 * and scales (section 4.3), top-k reduction plus the shared-expert add (section
 * 3.2); the route comes from moe_plan ("Optimization progress report",
 * Optimization 14).
 *   x              [T, H] bf16
 *   topk_weights   [T, K] float32  routing weight of each pick, applied after W2
 *   expert_offsets, sorted_pairs, pair_rows, plan_ws   from moe_plan (same dims)
 *   w13   [E, 2I, H/2]  MXFP4 codes in the layout of moe_pack_weights
 *   w13_s [E, 2I, H/32] E8M0 scales, row-major
 *   w2    [E, H, I/2]   MXFP4 codes in the layout of moe_pack_weights
 *   w2_s  [E, H, I/32]  E8M0 scales, row-major
 *   shared          optional dense FP8 shared expert (NULL or dims->Is == 0: none);
 *                   with one, T * H must be below 2^30
 *   y     [T, H] bf16 out
 *   dbg             optional inspection outputs / stage events (NULL: none)
 *   ws, ws_bytes    workspace (>= moe_ffn_workspace_bytes), owned by the caller;
 *                   nothing in it needs to be initialized
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP. */
int moe_ffn(const moe_dims* dims, const uint16_t* x, const float* topk_weights,
            const int32_t* expert_offsets, const int32_t* sorted_pairs, const int32_t* pair_rows,
            const void* plan_ws, const uint8_t* w13, const uint8_t* w13_s, const uint8_t* w2,
            const uint8_t* w2_s, const moe_shared* shared, uint16_t* y, const moe_debug* dbg,
            void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. moe_ffn with the same
 * arguments and results, minus the workspace: the library uses a static device
 * array of MOE_FFN_STATIC_MAX_BYTES instead, one per GPU, set up on the first
 * call on each device and held until the process ends. The call itself allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 *   Limit: moe_ffn_workspace_bytes(dims) must be at most MOE_FFN_STATIC_MAX_BYTES
 *   (64 MiB: decode steps of up to about 256 tokens x top-8 at hidden 7168);
 *   larger calls return MOE_ESCRATCH and enqueue nothing.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 *   (two streams, or two host threads) race and must be serialized by the caller.
 *   The array keeps the last call's contents; nothing in it needs to start at
 *   zero (every byte a call reads was written earlier in the same call).
 * Errors: as moe_ffn, plus MOE_ESCRATCH; MOE_EHIP also if the array's device
 * address cannot be looked up. */
#define MOE_FFN_STATIC_MAX_BYTES ((size_t)64 << 20)
int moe_ffn_static(const moe_dims* dims, const uint16_t* x, const float* topk_weights,
                   const int32_t* expert_offsets, const int32_t* sorted_pairs, const int32_t* pair_rows,
                   const void* plan_ws, const uint8_t* w13, const uint8_t* w13_s, const uint8_t* w2,
                   const uint8_t* w2_s, const moe_shared* shared, uint16_t* y, const moe_debug* dbg,
                   void* stream);

/* The routed MoE FFN with NVFP4 expert weights consumed as stored ("Optimization
 * progress report", Optimization 05: native NVFP4 MoE, no re-quantization of the
 * weights). The page names the format only; the layout is NVIDIA's published
 * NVFP4: E2M1 codes, one E4M3 scale per 16 consecutive K elements and one fp32
 * scale per tensor, w = E2M1 * E4M3 * tensor scale. Activations are bf16 and the
 * SwiGLU output is rounded once to bf16 (as MOE_FLAG_A16); no shared expert.
 *   dims->flags   must include MOE_FLAG_NVFP4 (plan, workspace size and this call)
 *   w13    [E, 2I, H/2] E2M1 codes, low nibble = even K, in the layout of
 *                       moe_pack_weights (the same packing as MXFP4 codes)
 *   w13_s  [E, 2I, H/16] E4M3 block scales (non-negative, finite), row-major
 *   w13_gs [E] float32   tensor scale of each expert's W13
 *   w2     [E, H, I/2]   codes, packed as w13
 *   w2_s   [E, H, I/16]  E4M3 block scales, row-major
 *   w2_gs  [E] float32   tensor scale of each expert's W2
 *   everything else as moe_ffn; dbg->h_q receives bf16 [P, I] SwiGLU rows.
 * Errors: MOE_EINVAL (also without MOE_FLAG_NVFP4 or a tensor-scale pointer),
 * MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP. */
int moe_ffn_nvfp4(const moe_dims* dims, const uint16_t* x, const float* topk_weights,
                  const int32_t* expert_offsets, const int32_t* sorted_pairs, const int32_t* pair_rows,
                  const void* plan_ws, const uint8_t* w13, const uint8_t* w13_s, const float* w13_gs,
                  const uint8_t* w2, const uint8_t* w2_s, const float* w2_gs, uint16_t* y,
                  const moe_debug* dbg, void* ws, size_t ws_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* moe_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
