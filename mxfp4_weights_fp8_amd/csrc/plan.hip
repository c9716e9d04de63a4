// Route planner: pack the (token, pick) pairs by expert ahead of the expert GEMMs
// without changing the token-to-expert mapping ("Optimization progress report",
// Optimization 14), and build the device-side tile work lists the grouped GEMMs
// drain, so no host readback is needed between planning and the FFN.
//
// Pair p = t*K + j. Output order: by expert, then by p (stable counting sort).
//   1. local ranks: each block takes kPlanChunk consecutive pairs; every wave
//      takes 64 of them at a time and finds, per lane, the lanes holding the same
//      expert with one ballot per key bit ("peer mask"); the rank inside the wave
//      is the popcount of the lower peers; waves of the same round are ordered
//      through a small LDS table; a per-expert LDS cursor carries the count across
//      rounds. No atomics decide an order, so the result is deterministic.
//   2. scan: per expert, an exclusive scan over blocks (one wave per expert),
//      then over experts -> expert_offsets; the work lists are built from the
//      per-expert counts.
//   3. scatter: position = expert offset + block base of the pair's expert +
//      local rank.
// One block (P <= kPlanChunk, the decode shapes) runs all three phases in a
// single fused launch; larger P uses four launches (the scan takes two).
#include "device_common.h"
#include "host_internal.h"

namespace moe {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kScanThreads = 1024;

// Exclusive scan of a[0..n) in LDS with all threads of the block; returns the total.
// Each thread sums a contiguous run, the runs are scanned within each wave with
// lane shuffles and across waves through part[] (at least blockDim/64 entries),
// then each thread writes its run's prefixes: two barriers per scan.
__device__ int block_exclusive_scan(int32_t* a, int n, int32_t* part) {
  const int t = threadIdx.x, nt = blockDim.x, lane = t & 63, wave = t >> 6, nw = nt >> 6;
  const int per = (n + nt - 1) / nt;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += a[i];
  int v = s;                                   // inclusive scan within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) part[wave] = v;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < nw; ++w) {
    const int pw = part[w];
    base += w < wave ? pw : 0;
    total += pw;
  }
  int run = base + v - s;
  for (int i = lo; i < hi; ++i) {
    const int x = a[i];
    a[i] = run;
    run += x;
  }
  __syncthreads();
  return total;
}

// The same for two arrays at once (one pass, two barriers): exclusive scans of a[0..n)
// and b[0..n); returns the total of a, the total of b in *total_b and the largest
// element of a in *max_a. part[] holds at least 3 blockDim/64 entries.
__device__ int block_exclusive_scan2(int32_t* a, int32_t* b, int n, int32_t* part, int* total_b, int* max_a) {
  const int t = threadIdx.x, nt = blockDim.x, lane = t & 63, wave = t >> 6, nw = nt >> 6;
  const int per = (n + nt - 1) / nt;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  int sa = 0, sb = 0, mx = 0;
  for (int i = lo; i < hi; ++i) {
    sa += a[i];
    sb += b[i];
    mx = max(mx, a[i]);
  }
  int va = sa, vb = sb;                        // inclusive scans within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ua = __shfl_up(va, off), ub = __shfl_up(vb, off);
    if (lane >= off) {
      va += ua;
      vb += ub;
    }
    mx = max(mx, __shfl_xor(mx, off));
  }
  if (lane == 63) {
    part[wave] = va;
    part[nw + wave] = vb;
    part[2 * nw + wave] = mx;
  }
  __syncthreads();
  int base_a = 0, base_b = 0, tot_a = 0, tot_b = 0, max_all = 0;
  for (int w = 0; w < nw; ++w) {
    const int pa = part[w], pb = part[nw + w];
    base_a += w < wave ? pa : 0;
    base_b += w < wave ? pb : 0;
    tot_a += pa;
    tot_b += pb;
    max_all = max(max_all, part[2 * nw + w]);
  }
  int ra = base_a + va - sa, rb = base_b + vb - sb;
  for (int i = lo; i < hi; ++i) {
    const int xa = a[i], xb = b[i];
    a[i] = ra;
    b[i] = rb;
    ra += xa;
    rb += xb;
  }
  __syncthreads();
  *total_b = tot_b;
  *max_a = max_all;
  return tot_a;
}

// Sum of v over the block (every thread gets it); part[] as for the scan.
__device__ int block_sum(int v, int32_t* part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if (lane == 0) part[wave] = v;
  __syncthreads();
  int total = 0;
  for (int w = 0; w < nw; ++w) total += part[w];
  __syncthreads();
  return total;
}

// Sorts the distinct keys v[0..n2) ascending (n2 a power of two), with all threads
// of the block: a bitonic network. Element i of a register pass lives in lane i % 64
// of its wave, so the stages whose partner distance j is below 64 exchange through
// lane shuffles with no barrier (all of them for the merges of up to 64 elements,
// the last six of every larger merge); the other stages go through LDS with one
// barrier each (6 of the 45 stages at 512 keys).
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int j) {
  const int lo = __shfl_xor((int)(uint32_t)x, j), hi = __shfl_xor((int)(uint32_t)(x >> 32), j);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ void block_sort_keys(uint64_t* v, int n2) {
  const int t = threadIdx.x, nt = blockDim.x;
  // merges k_lo..k_hi, stages j = min(k/2, 32) .. 1, in registers (n2 and nt are
  // powers of two: one round when n2 <= nt, otherwise whole rounds; elements past n2
  // hold the largest key and are not written back)
  auto reg_pass = [&](int k_lo, int k_hi) {
    for (int base = 0; base < n2; base += nt) {
      const int i = base + t;
      uint64_t x = i < n2 ? v[i] : ~0ull;
      for (int k = k_lo; k <= k_hi; k <<= 1)
        for (int j = min(k >> 1, 32); j > 0; j >>= 1) {
          const uint64_t y = shfl_xor_u64(x, j);
          // the lower index of the pair keeps the smaller key in an ascending run
          const bool keep_min = ((i & j) == 0) == ((i & k) == 0);
          x = keep_min ? (y < x ? y : x) : (y > x ? y : x);
        }
      if (i < n2) v[i] = x;
    }
    __syncthreads();
  };
  reg_pass(2, n2 < 64 ? n2 : 64);
  for (int k = 128; k <= n2; k <<= 1) {
    for (int j = k >> 1; j >= 64; j >>= 1) {
      for (int i = t; i < n2 / 2; i += nt) {
        const int a = 2 * i - (i & (j - 1)), b = a + j;   // bit log2(j) of a clear
        const uint64_t x = v[a], y = v[b];
        if ((a & k) == 0 ? y < x : x < y) {
          v[a] = y;
          v[b] = x;
        }
      }
      __syncthreads();
    }
    reg_pass(k, k);
  }
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Phase 1 for pairs [begin, end): local_rank[p - rank_base] = number of earlier
// pairs of the same expert inside [begin, end); key[p - rank_base] (when given) =
// the pair's expert, or -1 for an id outside [0, E). cursor[E] must start at zero
// and ends holding the per-expert counts of the range; wcnt[kPlanWaves * E] must
// start at zero and ends at zero.
__device__ void local_ranks(const int32_t* __restrict__ ids, int begin, int end, int E, int nbits,
                            int32_t* __restrict__ local_rank, int rank_base, int32_t* key_out, int32_t* cursor,
                            int32_t* wcnt) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = begin; base < end; base += kPlanThreads) {
    const int p = base + tid;
    int key = -1;
    if (p < end) {
      const int v = ids[p];
      key = (v >= 0 && v < E) ? v : -1;
    }
    const bool valid = key >= 0;
    if (key_out && p < end) key_out[p - rank_base] = key;
    uint64_t peer = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool b = valid && ((key >> bit) & 1);
      const uint64_t m = __ballot(b);
      peer &= b ? m : ~m;
    }
    const int rank = __popcll(peer & lower);
    const int cnt = __popcll(peer);
    const bool leader = valid && rank == 0;
    if (leader) wcnt[wave * E + key] = cnt;
    __syncthreads();
    if (valid) {
      int r = cursor[key] + rank;
      for (int w = 0; w < wave; ++w) r += wcnt[w * E + key];
      local_rank[p - rank_base] = r;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&cursor[key], cnt);   // integer adds commute: order-independent
      wcnt[wave * E + key] = 0;
    }
    __syncthreads();
  }
}

// 16-row small-M tiles of an expert with m pairs (none above small_max).
__device__ __forceinline__ int small_tiles(int m, int small_max) {
  return (m >= 1 && m <= small_max) ? (m + kSmallRows - 1) / kSmallRows : 0;
}

// Work lists from per-expert counts cnt[E] (LDS): small-M tiles of kSmallRows rows
// for experts with 1..small_max pairs (expert order); the rest in 256-row items (the
// last one when more than 128 rows remain), heaviest expert first (ties: lower id
// first), and at most one 128-row item per expert for a remainder of 1..128 rows,
// ordered by rows (ties: heavier expert, then lower id), so that the items of at
// most t13 (t2) rows, which W13 (W2) walks as 16-row tiles, are a prefix whose
// length goes to hdr[3] (hdr[4]). Both orders come from bitonic sorts of the
// compacted experts, O(E log^2 E) work (a count of the experts ahead of each one,
// O(E^2), took 3.7 ms at 4096 experts). a1: E words holding on entry the exclusive
// scan of small_tiles() (n_small in all); any_big: some expert has more than
// small_max pairs; a2: E words, part: blockDim words, keys: LDS for 2 E sort keys
// (8-byte aligned).
__device__ void build_worklists(const int32_t* cnt, int E, int small_max, int t13, int t2,
                                int2* __restrict__ small_items, int64_t small_cap, int2* __restrict__ large_items,
                                int64_t large_cap, int2* __restrict__ xl_items, int64_t xl_cap,
                                int32_t* __restrict__ hdr, int32_t* a1, int n_small, bool any_big, int32_t* a2,
                                int32_t* part, uint64_t* keys) {
  const int t = threadIdx.x, nt = blockDim.x;
  for (int e = t; e < E; e += nt) {
    const int m = cnt[e];
    if (m >= 1 && m <= small_max) {
      const int s = a1[e];
      for (int i = 0; i * kSmallRows < m; ++i)
        if (s + i < small_cap) small_items[s + i] = make_int2(e, i * kSmallRows);
    }
  }
  // no expert above small_max (decode batches): empty large-M lists, done
  if (!any_big) {
    if (t == 0) {
      hdr[0] = n_small < small_cap ? n_small : (int)small_cap;
      hdr[1] = 0;
      hdr[2] = 0;
      hdr[3] = 0;
      hdr[4] = 0;
    }
    return;
  }
  // The large experts (more than small_max pairs) in heavy-first order (ties: lower
  // id): compacted in id order as keys (INT_MAX - pairs, id), then sorted (a2[r] =
  // the expert of rank r). An id takes the low 24 bits of either key (E <= 4096).
  for (int e = t; e < E; e += nt) a1[e] = cnt[e] > small_max ? 1 : 0;
  __syncthreads();
  const int n_big = block_exclusive_scan(a1, E, part);
  const int n2 = pow2_at_least(n_big);
  for (int e = t; e < E; e += nt)
    if (cnt[e] > small_max) keys[a1[e]] = ((uint64_t)(0x7FFFFFFF - cnt[e]) << 32) | (uint32_t)e;
  for (int i = n_big + t; i < n2; i += nt) keys[i] = ~0ull;   // padding, sorted last
  __syncthreads();
  block_sort_keys(keys, n2);
  for (int r = t; r < n_big; r += nt) a2[r] = (int)(keys[r] & 0xFFFFFF);
  __syncthreads();
  // 128-row items: the large experts with a remainder of 1..128 rows, by rows (ties:
  // heavier, then lower id): keys (rows, INT_MAX - pairs, id), compacted and sorted
  // the same way
  for (int e = t; e < E; e += nt) {
    const int m = cnt[e], rem = m % kXlRows;
    a1[e] = m > small_max && rem >= 1 && rem <= kXlRows / 2;
  }
  __syncthreads();
  const int n_rem = block_exclusive_scan(a1, E, part);
  const int n2r = pow2_at_least(n_rem);
  for (int e = t; e < E; e += nt) {
    const int m = cnt[e], rem = m % kXlRows;
    if (m > small_max && rem >= 1 && rem <= kXlRows / 2)
      keys[a1[e]] = ((uint64_t)rem << 56) | ((uint64_t)(0x7FFFFFFF - m) << 24) | (uint32_t)e;
  }
  for (int i = n_rem + t; i < n2r; i += nt) keys[i] = ~0ull;
  __syncthreads();
  block_sort_keys(keys, n2r);
  for (int i = t; i < n_rem && i < large_cap; i += nt) {
    const int e = (int)(keys[i] & 0xFFFFFF), m = cnt[e];
    large_items[i] = make_int2(e, m - m % kXlRows);
  }
  // 256-row items: a1[r] = the first item of rank r; item i belongs to the last rank r
  // with a1[r] <= i (ranks without 256-row items share the next rank's start), found by
  // binary search, one thread per item
  for (int r = t; r < E; r += nt) a1[r] = r < n_big ? (cnt[a2[r]] + kXlRows / 2 - 1) / kXlRows : 0;
  __syncthreads();
  const int n_xl = block_exclusive_scan(a1, E, part);
  for (int i = t; i < n_xl && i < xl_cap; i += nt) {
    int lo = 0, hi = n_big - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a1[mid] <= i) lo = mid; else hi = mid - 1;
    }
    xl_items[i] = make_int2(a2[lo], (i - a1[lo]) * kXlRows);
  }
  // 128-row items (written above): their number, and how many have at most t13 / t2 rows
  int c13 = 0, c2 = 0, n_large = 0;
  for (int e = t; e < E; e += nt) {
    const int m = cnt[e], rem = m % kXlRows;
    if (m > small_max && rem >= 1 && rem <= kXlRows / 2) {
      n_large += 1;
      c13 += rem <= t13;
      c2 += rem <= t2;
    }
  }
  n_large = block_sum(n_large, part);
  c13 = block_sum(c13, part);
  c2 = block_sum(c2, part);
  if (t == 0) {
    const int nl = n_large < large_cap ? n_large : (int)large_cap;
    hdr[0] = n_small < small_cap ? n_small : (int)small_cap;
    hdr[1] = nl;
    hdr[2] = n_xl < xl_cap ? n_xl : (int)xl_cap;
    hdr[3] = c13 < nl ? c13 : nl;
    hdr[4] = c2 < nl ? c2 : nl;
  }
}

struct PlanArgs {
  const int32_t* ids;
  int32_t* offsets;
  int32_t* sorted_pairs;
  int32_t* pair_rows;
  int32_t* status;
  int32_t* hdr;
  int2* small_items;
  int2* large_items;
  int2* xl_items;
  int32_t* local_rank;
  int32_t* block_counts;
  int32_t* block_base;
  int64_t small_cap, large_cap, xl_cap;
  int P, E, nbits, small_max, nb;
  int t13, t2;   // tile_small_rows of W13 and W2
};

// Single-block plan: all three phases in one launch (P <= kPlanChunk).
__global__ __launch_bounds__(kPlanThreads) void k_plan_fused(PlanArgs a) {
  extern __shared__ __attribute__((aligned(16))) int32_t lds[];
  const int E = a.E;
  int32_t* wcnt = lds;                        // [kPlanWaves * E]; later the sort keys
  int32_t* cnt = wcnt + kPlanWaves * E;       // [E]
  int32_t* off = cnt + E;                     // [E + 1]
  int32_t* a1 = off + E + 1;                  // [E]
  int32_t* a2 = a1 + E;                       // [E]
  int32_t* part = a2 + E;                     // [kPlanThreads]
  int32_t* rank = part + kPlanThreads;        // [P] local ranks
  int32_t* key = rank + a.P;                  // [P] experts (-1: dropped)
  const int t = threadIdx.x;
  for (int i = t; i < (kPlanWaves + 1) * E; i += kPlanThreads) lds[i] = 0;
  __syncthreads();
  local_ranks(a.ids, 0, a.P, E, a.nbits, rank, 0, key, cnt, wcnt);
  for (int e = t; e < E; e += kPlanThreads) {
    off[e] = cnt[e];
    a1[e] = small_tiles(cnt[e], a.small_max);
  }
  __syncthreads();
  int n_small, max_cnt;
  const int n_valid = block_exclusive_scan2(off, a1, E, part, &n_small, &max_cnt);
  if (t == 0) {
    off[E] = n_valid;
    a.status[0] = a.P - n_valid;
  }
  __syncthreads();
  for (int e = t; e <= E; e += kPlanThreads) a.offsets[e] = off[e];
  for (int p = t; p < a.P; p += kPlanThreads) {   // the thread that ranked pair p
    const int v = key[p];
    if (v >= 0) {
      const int pos = off[v] + rank[p];
      a.sorted_pairs[pos] = p;
      a.pair_rows[p] = pos;
    } else {
      a.pair_rows[p] = -1;
    }
    if (p >= n_valid) a.sorted_pairs[p] = -1;
  }
  // wcnt (4 E words at the start of LDS) is free: room for 2 E sort keys
  build_worklists(cnt, E, a.small_max, a.t13, a.t2, a.small_items, a.small_cap, a.large_items, a.large_cap, a.xl_items, a.xl_cap,
                  a.hdr, a1, n_small, max_cnt > a.small_max, a2, part, reinterpret_cast<uint64_t*>(wcnt));
}

// Multi-block phase 1.
__global__ __launch_bounds__(kPlanThreads) void k_plan_local(PlanArgs a) {
  extern __shared__ __attribute__((aligned(16))) int32_t lds[];
  const int E = a.E;
  int32_t* cnt = lds;
  int32_t* wcnt = cnt + E;
  const int t = threadIdx.x, b = blockIdx.x;
  for (int i = t; i < (kPlanWaves + 1) * E; i += kPlanThreads) lds[i] = 0;
  __syncthreads();
  const int begin = b * kPlanChunk;
  const int end = min(a.P, begin + kPlanChunk);
  local_ranks(a.ids, begin, end, E, a.nbits, a.local_rank, 0, nullptr, cnt, wcnt);
  for (int e = t; e < E; e += kPlanThreads) a.block_counts[(int64_t)e * a.nb + b] = cnt[e];   // [E][nb]
}

// Multi-block phase 2: per expert, the exclusive scan of its block counts over the
// blocks (the rank of a block's first pair of that expert among the expert's pairs),
// one wave per expert, 64 blocks per round with lane shuffles; counts and bases are
// stored [expert][block], so a wave's load covers 64 consecutive words. The expert's
// total goes to offsets[e] for the next phase, which turns it into the offset.
// (Done by the next phase's single workgroup, this took 10 us of a 32K-token plan at
// 384 experts and most of its 0.39 ms at 4096.)
__global__ __launch_bounds__(kPlanThreads) void k_plan_expert_scan(PlanArgs a) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * kPlanWaves + (threadIdx.x >> 6);
  if (e >= a.E) return;                                   // wave-uniform
  const int nb = a.nb;
  int run = 0;
  for (int b0 = 0; b0 < nb; b0 += 64) {
    const int b = b0 + lane;
    const int c = b < nb ? a.block_counts[(int64_t)e * nb + b] : 0;
    int v = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(v, o);
      if (lane >= o) v += u;
    }
    if (b < nb) a.block_base[(int64_t)e * nb + b] = run + v - c;
    run += __shfl(v, 63);
  }
  if (lane == 0) a.offsets[e] = run;
}

// Multi-block phase 3 (one block of kScanThreads): expert offsets and work lists
// from the per-expert totals.
__global__ __launch_bounds__(kScanThreads) void k_plan_scan(PlanArgs a) {
  extern __shared__ __attribute__((aligned(16))) int32_t lds[];
  const int E = a.E;
  uint64_t* keys = reinterpret_cast<uint64_t*>(lds);   // [2 E] sort keys
  int32_t* cnt = lds + 4 * E;       // [E]
  int32_t* off = cnt + E;           // [E + 1]
  int32_t* a1 = off + E + 1;        // [E]
  int32_t* a2 = a1 + E;             // [E]
  int32_t* part = a2 + E;           // [kScanThreads]
  const int t = threadIdx.x;
  for (int e = t; e < E; e += kScanThreads) {
    const int m = a.offsets[e];       // the expert's total, from the previous phase
    cnt[e] = m;
    off[e] = m;
    a1[e] = small_tiles(m, a.small_max);
  }
  __syncthreads();
  int n_small, max_cnt;
  const int n_valid = block_exclusive_scan2(off, a1, E, part, &n_small, &max_cnt);
  if (t == 0) {
    off[E] = n_valid;
    a.status[0] = a.P - n_valid;
  }
  __syncthreads();
  for (int e = t; e <= E; e += kScanThreads) a.offsets[e] = off[e];
  build_worklists(cnt, E, a.small_max, a.t13, a.t2, a.small_items, a.small_cap, a.large_items, a.large_cap, a.xl_items, a.xl_cap,
                  a.hdr, a1, n_small, max_cnt > a.small_max, a2, part, keys);
}

// Multi-block phase 4.
__global__ __launch_bounds__(256) void k_plan_scatter(PlanArgs a) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= a.P) return;
  const int v = a.ids[p];
  if (v >= 0 && v < a.E) {
    const int pos = a.offsets[v] + a.block_base[(int64_t)v * a.nb + p / kPlanChunk] + a.local_rank[p];
    a.sorted_pairs[pos] = p;
    a.pair_rows[p] = pos;
  } else {
    a.pair_rows[p] = -1;
  }
  if (p >= a.offsets[a.E]) a.sorted_pairs[p] = -1;
}

}  // namespace

namespace {
// The tuned exact-shape table: for a shape (H, I), the largest 128-row item (rows)
// that W13 and W2 walk as 16-row small-M tiles rather than one 128-row tile; 0 =
// none. Measured on MI355X with tune_tiles.py on the routing histograms of the
// 32K-token prefill chunk (236 such items, 10 of them at most 16 rows), one MoE-TP8
// rank of it and the 256-token decode step. A 16-row pass re-streams the expert's
// weight slice, so only items of at most 16 rows gain, and only in W13 at the full
// intermediate size (9.44 vs 9.53 ms); every larger limit is slower in both GEMMs.
struct TileRule {
  int H, I, w13, w2;
};
constexpr TileRule kTileTable[] = {
    {7168, 3072, 16, 0},
    {7168, 384, 0, 0},
};
}  // namespace

int tile_small_rows(const moe_dims& d, bool w13) {
  const int64_t P = (int64_t)d.T * d.K;
  if (P <= kFoldPairs || !large_path_supported(d)) return kLargeRows;
  const int v = w13 ? d.tile_w13 : d.tile_w2;
  if (v < 0) return 0;
  if (v > 0) return v < kLargeRows ? v : kLargeRows;
  for (const TileRule& r : kTileTable)
    if (r.H == d.H && r.I == d.I) return w13 ? r.w13 : r.w2;
  return 0;
}

size_t plan_ws_layout(const moe_dims& d, void* base, PlanWs* out) {
  const int64_t P = (int64_t)d.T * d.K;
  const int64_t nb = ceil_div(P, kPlanChunk) < 1 ? 1 : ceil_div(P, kPlanChunk);
  const int64_t sc = small_items_bound(d), lc = large_items_bound(d), xc = xl_items_bound(d);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t o_hdr = take(64);
  const size_t o_small = take(sizeof(int2) * (size_t)(sc > 0 ? sc : 1));
  const size_t o_large = take(sizeof(int2) * (size_t)(lc > 0 ? lc : 1));
  const size_t o_xl = take(sizeof(int2) * (size_t)(xc > 0 ? xc : 1));
  const size_t o_rank = take(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
  const size_t o_bc = take(sizeof(int32_t) * (size_t)(nb * d.E));
  const size_t o_bb = take(sizeof(int32_t) * (size_t)(nb * d.E));
  if (out) {
    char* b = static_cast<char*>(base);
    out->hdr = reinterpret_cast<int32_t*>(b + o_hdr);
    out->small_items = reinterpret_cast<int2*>(b + o_small);
    out->large_items = reinterpret_cast<int2*>(b + o_large);
    out->xl_items = reinterpret_cast<int2*>(b + o_xl);
    out->local_rank = reinterpret_cast<int32_t*>(b + o_rank);
    out->block_counts = reinterpret_cast<int32_t*>(b + o_bc);
    out->block_base = reinterpret_cast<int32_t*>(b + o_bb);
    out->small_cap = sc;
    out->large_cap = lc;
    out->xl_cap = xc;
    out->nb = nb;
  }
  return off;
}

hipError_t launch_plan(const moe_dims& d, const int32_t* ids, int32_t* offsets, int32_t* sorted_pairs,
                       int32_t* pair_rows, int32_t* status, const PlanWs& ws, hipStream_t s) {
  PlanArgs a;
  a.ids = ids;
  a.offsets = offsets;
  a.sorted_pairs = sorted_pairs;
  a.pair_rows = pair_rows;
  a.status = status;
  a.hdr = ws.hdr;
  a.small_items = ws.small_items;
  a.large_items = ws.large_items;
  a.xl_items = ws.xl_items;
  a.local_rank = ws.local_rank;
  a.block_counts = ws.block_counts;
  a.block_base = ws.block_base;
  a.small_cap = ws.small_cap;
  a.large_cap = ws.large_cap;
  a.xl_cap = ws.xl_cap;
  a.P = d.T * d.K;
  a.E = d.E;
  int nbits = 0;
  while ((1 << nbits) < d.E) ++nbits;
  a.nbits = nbits;
  a.small_max = small_max_of(d);
  a.t13 = tile_small_rows(d, true);
  a.t2 = tile_small_rows(d, false);
  a.nb = (int)ws.nb;
  if (a.P <= kPlanChunk) {
    const size_t lds = sizeof(int32_t) * ((size_t)(kPlanWaves + 4) * d.E + 1 + kPlanThreads + 2 * (size_t)a.P);
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)k_plan_fused, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_plan_fused, dim3(1), dim3(kPlanThreads), lds, s, a);
    return hipGetLastError();
  }
  const size_t lds_local = sizeof(int32_t) * (size_t)(kPlanWaves + 1) * d.E;
  hipError_t err = hipSuccess;
  if (lds_local > 65536) {
    err = hipFuncSetAttribute((const void*)k_plan_local, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_local);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_plan_local, dim3(a.nb), dim3(kPlanThreads), lds_local, s, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds_scan = sizeof(int32_t) * ((size_t)8 * d.E + 1 + kScanThreads);
  if (lds_scan > 65536) {
    err = hipFuncSetAttribute((const void*)k_plan_scan, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_scan);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_plan_expert_scan, dim3((unsigned)ceil_div(d.E, kPlanWaves)), dim3(kPlanThreads), 0, s, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_plan_scan, dim3(1), dim3(kScanThreads), lds_scan, s, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_plan_scatter, dim3((unsigned)ceil_div(a.P, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
