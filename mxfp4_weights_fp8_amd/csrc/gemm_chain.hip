// Persistent decode chain: W13 + SwiGLU/requant, W2 and the top-k combine of a
// decode step in one launch, each W2 work unit starting as soon as the W13 units
// of its expert have signalled, and each output column block combined by the W2
// unit that finishes it ("Pushing the Limits of Serving DeepSeek-V4-Pro", section
// 4.3: W2 starts earlier once the fused SwiGLU quantization has written its
// operand, and the combine starts per finished W2 output tile; "Optimization
// progress report", Optimization 14: the route planned ahead, the expert work then
// runs without host involvement).
//
// Work units, handed out in order by an atomic ticket:
//   [0, n*U13)             W13 unit (item, 128 h columns), U13 = I/128
//   [n*U13, n*(U13+U2))    W2 unit (item, 128 output columns), U2 = ceil(H/128)
// Four waves per workgroup, the split of the separate small-M kernels (each W13 wave
// two gate and two up fragments, each W2 wave two fragments); measured on decode7
// against eight waves of one gate/up pair and 256-column W2 units: 0.2300 vs 0.2381
// ms per step (W2 units of two 128-column blocks in a row: 0.2359 ms).
// n = the plan's items of every list (16-row, 128-row and 256-row items, all
// walked in 16-row tiles: the chain runs for decode shapes, at most kFoldPairs
// pairs). Items are heavy-first and units item-major, so the first W2 units
// belong to the items whose W13 units were handed out first.
//
// Dependencies, with counters the activation quantizer zeroes at the start of
// every call (in stream order before this launch). The rows passed between
// units (SwiGLU codes and scales, per-pair rows and scales) are written and read
// with device-scope coherent accesses (sc1: past the non-coherent L1 and the
// per-XCD L2 copies), so the signals need no cache maintenance: every wave waits
// until its stores are complete (vmcnt counts stores too), the workgroup meets at
// a barrier, and one thread bumps a counter. (Device-scope fences instead wrote
// back and invalidated an XCD's whole L2 per signal and made the chain slower than
// the separate kernels.)
//   * a W13 unit, once its SwiGLU rows are stored, adds 1 to its item's counter; a
//     W2 unit first polls that counter until it reaches U13, then reads the rows.
//     Units are handed out in ticket order, so every W13 unit a W2 unit waits for
//     is already held by a running workgroup, which never waits itself: the chain
//     cannot deadlock. (Taking the next ticket while a unit runs, to hide the
//     atomic's round trip, made decode7's chain slower, 0.279 against 0.238 ms:
//     workgroups then hold units they cannot start yet, and the tail grows.) A poll gives up after kSpinLimit tries (marking sync[1]), so
//     every workgroup always exits.
//   * a W2 unit, once its per-pair rows are stored, adds 1 to its column block's
//     counter; the unit that brings it to n combines that column block for every
//     token (combine_group: fixed pick order, no atomics on values), so results
//     are bitwise those of the separate kernels.
// With no items at all (every pick dropped), U2 combine-only units write y.
#include "combine_group.h"
#include "small_unit.h"

namespace moe {
namespace {

using namespace small;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kW2NF = 2;                       // fragments per wave in a W2 unit
constexpr int kW2Cols = kWaves * 16 * kW2NF;   // output columns of a W2 unit
constexpr int kSpinLimit = 1 << 22;            // polls (about 0.1 s) before a wait gives up

struct ChainArgs {
  const int2* items[3];      // small, 128-row and 256-row item lists of the plan
  const int32_t* n_items[3];
  int rows[3];
  const int32_t* offsets;
  const int32_t* sorted_pairs;
  const int32_t* pair_rows;
  const uint8_t* x_q;
  const uint8_t* x_s;
  const uint8_t* w13;
  const uint8_t* w13_s;
  uint8_t* h_q;
  uint8_t* h_s;
  const uint8_t* w2;
  const uint8_t* w2_s;
  uint16_t* o;
  uint8_t* os;
  const float* topk_weights;
  const uint16_t* so;        // shared expert rows (nullable), added last by the combine
  const uint8_t* sos;
  uint16_t* y;
  int32_t* sync;             // [0] ticket, [1] gave-up flag, [2, 2+U2) column counters, then item counters
  int T, H, I, K;
};

__device__ __forceinline__ int poll(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void combine_columns(const ChainArgs& a, int cb) {
  const int gpr = a.H / 8;
  const int g0 = cb * (kW2Cols / 8);
  const int ng = min(kW2Cols / 8, gpr - g0);
  for (int i = threadIdx.x; i < a.T * ng; i += kThreads) {
    const int t = i / ng;
    combine_group<true>(a.o, a.os, a.topk_weights, a.pair_rows, a.so, a.sos, a.y, t, g0 + i % ng, gpr, a.K);
  }
}

__global__ __launch_bounds__(kThreads) void k_decode_chain(const ChainArgs a) {
  __shared__ float red[kWaves * 16];
  __shared__ int s_unit, s_last;
  extern __shared__ __attribute__((aligned(16))) uint8_t sS[];   // weight scales of the current unit
  const int n0 = a.n_items[0][0], n1 = a.n_items[1][0], n2 = a.n_items[2][0];
  const int n = n0 + n1 + n2;
  const int U13 = a.I / 128;
  const int U2 = (a.H + kW2Cols - 1) / kW2Cols;
  const int total13 = n * U13;
  const int total = n > 0 ? total13 + n * U2 : U2;
  int32_t* ticket = a.sync;
  int32_t* gave_up = a.sync + 1;
  int32_t* col_done = a.sync + 2;
  int32_t* item_done = a.sync + 2 + U2;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  for (;;) {
    if (threadIdx.x == 0) s_unit = atomicAdd(ticket, 1);
    __syncthreads();
    const int u = s_unit;
    if (u >= total) break;
    if (n == 0) {
      combine_columns(a, u);
    } else {
      const bool is13 = u < total13;
      const int v = is13 ? u : u - total13;
      const int item = is13 ? v / U13 : v / U2;
      const int sub = is13 ? v % U13 : v % U2;
      const int l = item < n0 ? 0 : (item < n0 + n1 ? 1 : 2);
      const int idx = item - (l == 0 ? 0 : (l == 1 ? n0 : n0 + n1));
      const int2 it = a.items[l][idx];
      if (is13) {
        w13_small_unit<kWaves, true>(it, a.rows[l], sub, a.offsets, a.sorted_pairs, a.x_q, a.x_s, a.w13,
                                     a.w13_s, a.h_q, a.h_s, a.H, a.I, a.K, sS, red);
        wait_vmcnt<0>();
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_fetch_add(&item_done[item], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        if (threadIdx.x == 0) {
          for (int tries = 0; poll(&item_done[item]) < U13; ++tries) {
            if (tries >= kSpinLimit) {
              atomicOr(gave_up, 1);
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
        }
        __syncthreads();
        w2_small_wave<kW2NF, true>(it, a.rows[l], sub * kW2Cols + wave * 16 * kW2NF, a.offsets, a.sorted_pairs, a.h_q,
                             a.h_s, a.w2, a.w2_s, a.o, a.os, a.H, a.I,
                             sS + wave * staged_bytes(16 * kW2NF * (a.I / 32)));
        wait_vmcnt<0>();
        __syncthreads();
        if (threadIdx.x == 0)
          s_last = __hip_atomic_fetch_add(&col_done[sub], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
        __syncthreads();
        if (s_last) combine_columns(a, sub);
      }
    }
    __syncthreads();   // s_unit, s_last and the scale LDS are reused by the next unit
  }
}

}  // namespace

size_t chain_sync_words(const moe_dims& d) {
  return 2 + (size_t)ceil_div(d.H, kW2Cols) + (size_t)(small_items_bound(d) + large_items_bound(d) +
                                                       xl_items_bound(d));
}

hipError_t launch_decode_chain(const moe_dims& d, const PlanWs& pw, const int32_t* offsets,
                               const int32_t* sorted_pairs, const int32_t* pair_rows, const uint8_t* x_q,
                               const uint8_t* x_s, const uint8_t* w13, const uint8_t* w13_s, uint8_t* h_q,
                               uint8_t* h_s, const uint8_t* w2, const uint8_t* w2_s, uint16_t* o, uint8_t* os,
                               const float* topk_weights, const uint16_t* so, const uint8_t* sos, uint16_t* y,
                               int32_t* sync, hipStream_t s) {
  ChainArgs a;
  a.items[0] = pw.small_items;
  a.items[1] = pw.large_items;
  a.items[2] = pw.xl_items;
  a.n_items[0] = pw.hdr + 0;
  a.n_items[1] = pw.hdr + 1;
  a.n_items[2] = pw.hdr + 2;
  a.rows[0] = kSmallRows;
  a.rows[1] = kLargeRows;
  a.rows[2] = kXlRows;
  a.offsets = offsets;
  a.sorted_pairs = sorted_pairs;
  a.pair_rows = pair_rows;
  a.x_q = x_q;
  a.x_s = x_s;
  a.w13 = w13;
  a.w13_s = w13_s;
  a.h_q = h_q;
  a.h_s = h_s;
  a.w2 = w2;
  a.w2_s = w2_s;
  a.o = o;
  a.os = os;
  a.topk_weights = topk_weights;
  a.so = so;
  a.sos = sos;
  a.y = y;
  a.sync = sync;
  a.T = d.T;
  a.H = d.H;
  a.I = d.I;
  a.K = d.K;
  // LDS: the larger of a W13 unit's weight scales (per wave two runs of 128/kWaves
  // rows x H/32) and a W2 unit's (per wave 16 kW2NF rows x I/32)
  const size_t lds13 = (size_t)kWaves * 2 * staged_bytes(128 / kWaves * (d.H / 32));
  const size_t lds2 = (size_t)kWaves * staged_bytes(16 * kW2NF * (d.I / 32));
  const size_t lds = lds13 > lds2 ? lds13 : lds2;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k_decode_chain),
                                                     kThreads, lds);
  if (e != hipSuccess) return e;
  const int64_t n_max = small_items_bound(d) + large_items_bound(d) + xl_items_bound(d);
  const int64_t units = n_max * (d.I / 128 + ceil_div(d.H, kW2Cols)) + ceil_div(d.H, kW2Cols);
  const int64_t resident = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
  const int64_t grid = units < resident ? units : resident;
  hipLaunchKernelGGL(k_decode_chain, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace moe
