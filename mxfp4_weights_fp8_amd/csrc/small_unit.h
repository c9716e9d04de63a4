// Device code of the small-M grouped GEMMs (decode shapes, at most 16 routed rows
// per tile) on the gfx950 block-scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4,
// shared by the per-GEMM kernels (gemm_small.hip) and the persistent decode chain
// (gemm_chain.hip).
//
// The weights take the MFMA's 16-row A side (E2M1, one E8M0 scale per 32 K) and the
// routed tokens its 16-column B side (E4M3, the per-128 activation scale replicated
// over the four 32-blocks). The work is a stream of the expert's weights, in the
// kernel-native layout (a fragment's codes of one K step are 1 KB of consecutive
// bytes in lane order): each lane loads its 16 bytes per fragment and K step
// straight from HBM into registers (no reuse across waves, so no LDS staging), four
// K steps of a wave's fragments in flight.
#pragma once

#include "device_common.h"
#include "host_internal.h"
#include "lds_copy.h"

namespace moe {
namespace small {

// Cache policy of the activation-side scale loads (x scales in W13, SwiGLU scales in
// W2). COH = true selects device-scope coherent accesses (sc1), for data another
// workgroup of the same launch wrote (the decode chain): they bypass the
// non-coherent L1 and per-XCD L2 copies, so no cache maintenance is needed. Scale
// bytes of several items share a cache line, so a line read for one item could be
// a stale copy for another. The code rows themselves keep the default policy even
// then: a row belongs to one item, occupies whole cache lines, and nothing in the
// launch reads it before its item is complete (and the launch starts with
// invalidated caches), so no cache can hold a stale copy; the eight waves of a W2
// unit, which all read the same rows, then share them through L2 (sc1 loads of the
// rows cost 420 MB of extra memory traffic per decode7 step).
template <bool COH>
constexpr int kActPolicy = COH ? 16 : 0;

// Stores of rows a later unit of the same launch reads: device-scope coherent (sc1)
// when COH, plain otherwise.
template <bool COH, typename V>
__device__ __forceinline__ void store_row(V* p, V v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

__device__ __forceinline__ v8i fp4_operand(const v4i w) {
  v8i a;
  a[0] = w[0]; a[1] = w[1]; a[2] = w[2]; a[3] = w[3];
  a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
  return a;
}

// Operands of one K step for NF weight fragments: per fragment 16 bytes of E2M1
// codes and the dword holding the four E8M0 scales of this step's 32-blocks
// (lane group q uses byte q); the token rows' E4M3 codes and their scale.
template <int NF>
struct Step {
  v4i w[NF];
  int ws[NF];
  v8i x;
  int xs;
};

// Where a wave's operands live: buffer resources (wave-uniform) and per-lane
// byte offsets; step s adds s*1024 (codes), s*128 (activation codes), s (activation
// scales) as wave-uniform offsets. The weight scales are in LDS: sl[f] is the
// lane's row of fragment f there (KS dwords, dword s = the four 32-block scales
// of step s).
template <int NF>
struct Stream {
  rsrc_t w, x, xs;
  int wo[NF];
  const uint8_t* sl[NF];
  int xo, xso;
};

template <int NF, bool COH>
__device__ __forceinline__ void load_step(Step<NF>& r, const Stream<NF>& p, int s) {
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    r.w[f] = buf_load16_nt(p.w, p.wo[f], s * 1024);
    r.ws[f] = *reinterpret_cast<const int*>(p.sl[f] + s * 4);
  }
  const v4i lo = buf_load16(p.x, p.xo, s * 128), hi = buf_load16(p.x, p.xo, s * 128 + 64);
  r.x[0] = lo[0]; r.x[1] = lo[1]; r.x[2] = lo[2]; r.x[3] = lo[3];
  r.x[4] = hi[0]; r.x[5] = hi[1]; r.x[6] = hi[2]; r.x[7] = hi[3];
  r.xs = buf_load1<kActPolicy<COH>>(p.xs, p.xso, s);
}

template <int NF>
__device__ __forceinline__ void mma_step(const Step<NF>& r, int qshift, v4f* acc) {
#pragma unroll
  for (int f = 0; f < NF; ++f)
    acc[f] = mfma_scale_16x16x128<kFmtE2M1, kFmtE4M3>(fp4_operand(r.w[f]), r.x, acc[f], r.ws[f] >> qshift, r.xs);
}

// LDS bytes of one staged run of `bytes`: whole 1 KB copy instructions.
__host__ __device__ constexpr int staged_bytes(int bytes) { return (bytes + 1023) / 1024 * 1024; }

// Copy one or two contiguous byte runs (src0, then src1 when non-null, `bytes`
// each; wave-uniform arguments) into LDS at dst, run h at dst + h*staged_bytes,
// with direct-to-LDS 16-byte-per-lane copies (1 KB per instruction; lanes past
// the run read zeros into the run's padding). The wave alone reads what it copied;
// stream_k waits for the copies (vmcnt 0) before its first LDS read, so no
// barrier is needed.
__device__ __forceinline__ void stage_scales(const uint8_t* src0, const uint8_t* src1, int bytes, uint8_t* dst,
                                             int lane) {
  for (int h = 0; h < (src1 ? 2 : 1); ++h) {
    const v4i_s r = rsrc4(h ? src1 : src0, (uint32_t)bytes);
    for (int off = 0; off < bytes; off += 1024)
      dma16(r, lds_addr(dst + h * staged_bytes(bytes) + off), lane * 16 + off, 0);
  }
}

// Codes of one K step (the scales travel separately, four steps at a time).
template <int NF>
struct Codes {
  v4i w[NF];
  v8i x;
};

template <int NF, bool COH>
__device__ __forceinline__ void load_codes(Codes<NF>& r, const Stream<NF>& p, int s) {
#pragma unroll
  for (int f = 0; f < NF; ++f) r.w[f] = buf_load16_nt(p.w, p.wo[f], s * 1024);   // read once per step
  const v4i lo = buf_load16(p.x, p.xo, s * 128), hi = buf_load16(p.x, p.xo, s * 128 + 64);
  r.x[0] = lo[0]; r.x[1] = lo[1]; r.x[2] = lo[2]; r.x[3] = lo[3];
  r.x[4] = hi[0]; r.x[5] = hi[1]; r.x[6] = hi[2]; r.x[7] = hi[3];
}

// acc[f] += sum over KS steps of 128 K.
// Main path (KS a multiple of 4): the codes of kQuad = 4 steps stay in flight in a
// register ring. At the start of each 4-step chunk a lane reads the chunk's 16
// bytes of E8M0 scales of its rows from LDS and packs its own K block's byte of
// the four steps into one register; the MFMA's op_sel picks byte d for step d. The
// activation scales come in one dword per chunk (byte d for step d). Prefetch step
// indices are clamped on the wave-uniform offset, so the loop is branch-free; the
// clamped reloads hit the cache and go unused.
// Other K (short or not a multiple of 4 steps): a plain per-step loop.
constexpr int kQuad = 4;

// byte q of each of the four dwords of v, packed as bytes 0..3
__device__ __forceinline__ int pack_lane_bytes(v4i v, int qshift) {
  uint32_t r = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) r |= (((uint32_t)v[d] >> qshift) & 0xFFu) << (8 * d);
  return (int)r;
}

template <int NF, int D>
__device__ __forceinline__ void mma_quad_step(const Codes<NF>& r, const int* sc, int xsc, v4f* acc) {
#pragma unroll
  for (int f = 0; f < NF; ++f)
    acc[f] = mfma_scale_16x16x128<kFmtE2M1, kFmtE4M3, D, D>(fp4_operand(r.w[f]), r.x, acc[f], sc[f], xsc);
}

template <int NF, bool COH>
__device__ __forceinline__ void stream_k(v4f* acc, const Stream<NF>& p, int KS, int qshift) {
  if (KS % kQuad != 0) {
    wait_vmcnt<0>();   // the weight-scale copies into LDS
    for (int s = 0; s < KS; ++s) {
      Step<NF> r;
      load_step<NF, COH>(r, p, s);
      mma_step(r, qshift, acc);
    }
    return;
  }
  Codes<NF> buf[kQuad];
  int sc[NF];
#pragma unroll
  for (int d = 0; d < kQuad; ++d) load_codes<NF, COH>(buf[d], p, d);
  int xsc = buf_load4<kActPolicy<COH>>(p.xs, p.xso, 0);
  wait_vmcnt<0>();   // the weight-scale copies into LDS (and the first codes)
  for (int s0 = 0; s0 < KS; s0 += kQuad) {
#pragma unroll
    for (int f = 0; f < NF; ++f) sc[f] = pack_lane_bytes(*reinterpret_cast<const v4i*>(p.sl[f] + s0 * 4), qshift);
    const int nxt = min(s0 + kQuad, KS - kQuad);
    const int xscn = buf_load4<kActPolicy<COH>>(p.xs, p.xso, nxt);
    mma_quad_step<NF, 0>(buf[0], sc, xsc, acc);
    load_codes<NF, COH>(buf[0], p, min(s0 + kQuad + 0, KS - 1));
    mma_quad_step<NF, 1>(buf[1], sc, xsc, acc);
    load_codes<NF, COH>(buf[1], p, min(s0 + kQuad + 1, KS - 1));
    mma_quad_step<NF, 2>(buf[2], sc, xsc, acc);
    load_codes<NF, COH>(buf[2], p, min(s0 + kQuad + 2, KS - 1));
    mma_quad_step<NF, 3>(buf[3], sc, xsc, acc);
    load_codes<NF, COH>(buf[3], p, min(s0 + kQuad + 3, KS - 1));
    xsc = xscn;
  }
}

// One W13 work unit: 128 h columns (nb) of one item (an expert's routed rows
// it.y .. it.y + item_rows - 1, walked in 16-row tiles), WAVES waves, each streaming
// NF/2 gate and NF/2 up fragments. sS: the workgroup's LDS for weight scales (WAVES
// * 2 * staged_bytes(128 / WAVES * H/32) bytes); red: WAVES * 16 floats of LDS. Every
// thread of the workgroup calls it (two barriers per 16-row tile).
template <int WAVES, bool COH = false>
__device__ __forceinline__ void w13_small_unit(
    const int2 it, int item_rows, int nb,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
    const uint8_t* __restrict__ x_q, const uint8_t* __restrict__ x_s, const uint8_t* __restrict__ w13,
    const uint8_t* __restrict__ w13_s, uint8_t* __restrict__ h_q, uint8_t* __restrict__ h_s, int H, int I,
    int K, uint8_t* sS, float* red) {
  constexpr int NF = 256 / (16 * WAVES);    // weight fragments per wave: NF/2 gate + NF/2 up
  constexpr int HC = 128 / WAVES;            // h columns per wave
  const int e = it.x;
  const int e_begin = offsets[e], e_end = offsets[e + 1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  const int KS = H / 128;
  const int64_t wrow = H / 2, srow = H / 32;

  // 8-bit activation operand of a K step: bytes [16q, 16q+16) and [64+16q, 64+16q+16)
  Stream<NF> p;
  p.w = make_rsrc(w13 + (int64_t)e * 2 * I * wrow, (uint32_t)(2 * I * wrow));
  p.x = make_rsrc(x_q, 0xFFFFFFFFu);
  p.xs = make_rsrc(x_s, 0xFFFFFFFFu);
  // Weight scales of the wave's 64 rows (gate rows nb*128 + wave*32 + [0, 32) and
  // the matching up rows) into LDS rows wave*64 .. +63: two contiguous runs of
  // 32 * srow bytes, copied in full 1 KB instructions (each cache line once; read
  // per 4-step chunk straight from memory, a row's scale lines were refetched).
  const int run = staged_bytes(HC * (int)srow);
  stage_scales(w13_s + ((int64_t)e * 2 * I + nb * 128 + wave * HC) * srow,
               w13_s + ((int64_t)e * 2 * I + I + nb * 128 + wave * HC) * srow, HC * (int)srow,
               sS + wave * 2 * run, lane);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int up = f >= NF / 2, fi = f % (NF / 2);
    const int n0 = (up ? I : 0) + nb * 128 + wave * HC + fi * 16;   // first row of the fragment
    p.wo[f] = n0 * (int)wrow + lane * 16;
    p.sl[f] = sS + wave * 2 * run + up * run + (fi * 16 + c) * srow;
  }

  for (int m0 = it.y; m0 < it.y + item_rows && e_begin + m0 < e_end; m0 += kSmallRows) {
    const int row0 = e_begin + m0;
    const int mcount = min(kSmallRows, e_end - row0);
    const bool has = c < mcount;
    // an absent token column repeats the first row (valid data, result unused)
    const int tok = sorted_pairs[row0 + (has ? c : 0)] / K;
    p.xo = tok * H + q * 16;
    p.xso = tok * KS;

    v4f acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};
    stream_k<NF, false>(acc, p, KS, 8 * q);

    // SwiGLU + FP8 requantization: lane (c, q) holds h columns 4q..4q+3 of each
    // 16-column fragment pair, for routed row c.
    float h[NF / 2][4];
    float amax = 0.f;
#pragma unroll
    for (int g = 0; g < NF / 2; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[g][j] = silu_mul(acc[g][j], acc[g + NF / 2][j]);
        amax = fmaxf(amax, fabsf(h[g][j]));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (q == 0) red[wave * 16 + c] = amax;
    __syncthreads();
    amax = red[c];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) amax = fmaxf(amax, red[w * 16 + c]);
    __syncthreads();
    const int ex = e8m0_exponent(amax);
    const float inv = exp2_neg(ex);
    if (has) {
      uint8_t* dst = h_q + (int64_t)(row0 + c) * I + nb * 128 + wave * HC + q * 4;
#pragma unroll
      for (int g = 0; g < NF / 2; ++g) {
        store_row<COH>(reinterpret_cast<uint32_t*>(dst + g * 16),
                       e4m3_pack4(h[g][0] * inv, h[g][1] * inv, h[g][2] * inv, h[g][3] * inv));
      }
      if (wave == 0 && q == 0) store_row<COH>(&h_s[(int64_t)(row0 + c) * (I / 128) + nb], (uint8_t)(ex + 127));
    }
  }
}


// One wave's share of a W2 work unit: output columns n_wave .. n_wave + 16*NF - 1
// (wave-uniform; nothing if n_wave >= H) of one item, walked in 16-row tiles. sW:
// this wave's LDS for its weight scales (staged_bytes(16 * NF * I/32) bytes). No
// barriers: each wave works alone.
template <int NF, bool COH = false>
__device__ __forceinline__ void w2_small_wave(
    const int2 it, int item_rows, int n_wave,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
    const uint8_t* __restrict__ h_q, const uint8_t* __restrict__ h_s, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ w2_s, uint16_t* __restrict__ o, uint8_t* __restrict__ os, int H, int I,
    uint8_t* sW) {
  static_assert(NF == 2, "a wave's 16 * NF columns form one 32-column scale block of the per-pair output");
  const int lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  if (n_wave >= H) return;
  const int e = it.x;
  const int e_begin = offsets[e], e_end = offsets[e + 1];
  const int KS = I / 128;
  const int64_t wrow = I / 2, srow = I / 32;

  Stream<NF> p;
  p.w = make_rsrc(w2 + (int64_t)e * H * wrow, (uint32_t)(H * wrow));
  p.x = make_rsrc(h_q, 0xFFFFFFFFu);
  p.xs = make_rsrc(h_s, 0xFFFFFFFFu);
  // weight scales of the wave's 16*NF rows (one contiguous run) into LDS
  stage_scales(w2_s + ((int64_t)e * H + n_wave) * srow, nullptr, 16 * NF * (int)srow, sW, lane);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    p.wo[f] = (n_wave + f * 16) * (int)wrow + lane * 16;
    p.sl[f] = sW + (f * 16 + c) * srow;
  }

  for (int m0 = it.y; m0 < it.y + item_rows && e_begin + m0 < e_end; m0 += kSmallRows) {
    const int row0 = e_begin + m0;
    const int mcount = min(kSmallRows, e_end - row0);
    const bool has = c < mcount;
    const int hrow = row0 + (has ? c : 0);
    p.xo = hrow * I + q * 16;
    p.xso = hrow * KS;

    v4f acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};
    stream_k<NF, COH>(acc, p, KS, 8 * q);
    // fp16 codes + one scale per 32 columns (the wave's two fragments)
    float m = 0.f;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int k = 0; k < 4; ++k) m = fmaxf(m, fabsf(acc[f][k]));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    const int ex = o_exponent(m);
    const float inv = exp2_neg(ex);
    if (has) {
      const int64_t slot = sorted_pairs[row0 + c];
      uint16_t* dst = o + slot * H + n_wave + q * 4;
#pragma unroll
      for (int f = 0; f < NF; ++f)
        store_row<COH>(reinterpret_cast<uint64_t*>(dst + f * 16),
                       __builtin_bit_cast(uint64_t, f16_pack4(acc[f][0] * inv, acc[f][1] * inv, acc[f][2] * inv,
                                                              acc[f][3] * inv)));
      if (q == 0) store_row<COH>(&os[slot * (H / 32) + n_wave / 32], (uint8_t)(ex + 127));
    }
  }
}


}  // namespace small
}  // namespace moe
