// Affinity of every level row, then Grid -> Chunk -> Page top-K.
//
// Page "Key-Key Semantic Affinity: Key vectors replace attention scores for
// KV-cache importance" (10100.com): section 2.2 step 3 (affinity of anchor
// and block vector, normalised), section 5.1 (all three levels scored in a
// single pass, children of unselected parents masked to zero) and section
// 5.2 step 4 (keep the K highest-affinity blocks).
//
// Scoring: a batched GEMV with one right-hand side per sequence, bound by
// HBM bandwidth.  Each sequence's present rows are cut into tiles spread
// over the whole chip; in a tile, 8 lanes share one row (16 above head_dim
// 512; each lane reads 16-byte pieces 128 bytes apart, so 8 lanes read
// whole 128-byte lines) and every lane keeps 4 non-temporal loads in flight
// per pass over its tile (few registers, so eight waves per SIMD stay
// resident; rows are read once per step, and a serving batch's level rows
// exceed the last-level cache anyway); the fused kernel issues all 8 of a
// lane's loads in one pass.  A tile requests its first rows together with
// the page count and the anchor, taking level row v for physical row v
// (true below the page count and whenever the sequence fills its
// capacity) and loading them again in the rare tile where the count proves
// otherwise.  Dot product and row norm are reduced over the row's lanes
// with a fixed butterfly.
//
// Selection, written for latency: for batches whose tiles all fit on the
// chip at once, the work-group that finishes a sequence's last scoring
// tile (a per-sequence counter) selects that sequence in the same launch
// (score_select_kernel); larger batches whose levels are small (the serving
// workload) score and select in one launch too, with a selecting
// work-group per sequence that re-scores its few candidate rows beside the
// scoring tiles (score_topk_kernel, see the small coarse-to-fine selection
// below); other batches run the lighter score_kernel and then
// select_kernel, one work-group per sequence.  The sequence's
// affinity rows are staged into LDS in one round of loads (sequences of
// more than kLdsRows rows are selected from memory), then each level is
// selected: up to 64 candidates (children of kept parents, or every row)
// are ranked from per-wave LDS copies with one barrier, up to 512 in
// groups of 64 that are ranked, written back as sorted runs and merged by
// counting, larger sets are compacted with wave ballots and ranked or
// radix-selected (MSB first).  A rank is the number of larger keys, so rank
// < k places the element at its final position.  Keys are (affinity bits
// << 32 | ~index): unique, and larger means higher score then lower index.
// When fewer than k candidates score above zero, the lowest-index rows
// scoring exactly 0 (masked or zero affinity) fill the remaining slots in
// index order.  Small hierarchical levels (at most 64 grids, 64 chunk and
// 256 page candidates, k at most 64: the 128K and serving shapes) take a
// leaner path in the one-launch, two-launch and lazy selectors: wavefront
// 0 ranks grids and chunks alone while the others stage the page rows, and
// four wavefronts rank the pages (see the lean selection below).  The
// latency-bound paths read rows and anchors through buffer resources: a
// lane without a row issues the same load with an offset past the range
// and reads zeros, so no load waits behind a branch or a select.
#include <atomic>

#include "kka_internal.h"

namespace kka {
namespace {

#ifndef KKA_SELECT_THREADS
#define KKA_SELECT_THREADS 512
#endif
constexpr int kSelThreads = KKA_SELECT_THREADS;
constexpr int kRankMax = 512;
constexpr int kLdsRows = kSelectLdsRows;  // affinity rows staged per sequence (36 KB)
constexpr int kPlainTileMax = 256;        // rows of one score_kernel tile (one per thread)
constexpr int kBitmapWords = kMaxParents / 32;

// float4 row loads each lane keeps in flight in the scoring pass, and how
// many passes of the row-groups one scoring work-group makes.
#ifndef KKA_SCORE_LOADS
#define KKA_SCORE_LOADS 4
#endif
#ifndef KKA_SCORE_PASSES
#define KKA_SCORE_PASSES 2
#endif
// whether row loads bypass cache allocation
#ifndef KKA_SCORE_NT
#define KKA_SCORE_NT 1
#endif

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 load_row4(const f32x4* p) {
#if KKA_SCORE_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// Sorted groups of a level of 65-512 candidates: the keys, and every
// eighth key of each group (the last key of each block of 8).
struct SortedRuns {
  alignas(16) uint64_t key[kSelThreads];
  alignas(16) uint64_t piv[kSelThreads / 8];
};

struct SelectShared {
  float aff[kLdsRows];
  alignas(16) uint64_t ck[kRankMax];   // compacted candidate keys, or 64 keys per wave (copies)
  union {
    SortedRuns runs;                      // levels of 65-512 candidates
    int32_t part[kSelThreads / 64][64];   // per-wave counts (sorting up to 64 results)
  };
  uint64_t buf[kMaxK];
  uint32_t kept_grid[kBitmapWords];   // grids kept (parents of chunks)
  uint32_t kept_chunk[kBitmapWords];  // chunks kept (parents of pages)
  int32_t plist[kMaxK];
  uint32_t hist[256];
  uint32_t digit, above, bucket;
  int32_t cnt[4];
  int32_t wave_tot[kSelThreads / 64];
  uint32_t last;  // this work-group finished its sequence's scoring
};

struct Level {
  const float* aff;        // global scores: element e at aff[e] (used when not staged)
  int32_t off;             // row offset of element 0 in the staged LDS copy
  int32_t n;               // elements in the level
  int32_t fanout;          // children per parent; 0 = no parent level (all live)
  int32_t shift;           // log2(fanout) when fanout is a power of two, else -1
  int32_t n_par;           // kept parents listed in plist (fanout > 0)
  const uint32_t* parent;  // keep flags of the parent level (fanout > 0)
  int32_t slot;            // counter of sm.cnt this level uses
};

// Affinities cross work-groups inside one launch (scoring tiles on any
// XCD, the selecting work-group on another): device-scope stores and loads
// (store_agent, load_agent), ordered by the tile counters (arrive).

// Score bits of element e: from the LDS copy (STG) or from global memory.
// The two sources are separate instantiations so that LDS reads compile to
// LDS instructions rather than generic-address loads.
template <bool STG>
__device__ __forceinline__ uint32_t aff_key(const Level& L, const SelectShared& sm, int32_t e) {
  if constexpr (STG) return __float_as_uint(sm.aff[L.off + e]);
  else return __float_as_uint(load_agent(L.aff + e));
}

// Parent slot of child c (a shift for power-of-two fan-outs).
__device__ __forceinline__ int32_t parent_of(const Level& L, int32_t c) {
  return L.shift >= 0 ? (c >> L.shift) : c / L.fanout;
}

__device__ __forceinline__ bool is_live(const Level& L, int32_t e) {
  if (L.fanout == 0) return true;
  const int32_t p = parent_of(L, e);
  return (L.parent[p >> 5] >> (p & 31)) & 1u;
}

// Candidate c -> element index (or -1 when past the level's end).
__device__ __forceinline__ int32_t cand(const Level& L, const SelectShared& sm, int64_t c) {
  if (L.fanout == 0) return (int32_t)c;
  const int32_t pi = L.shift >= 0 ? (int32_t)(c >> L.shift) : (int32_t)(c / L.fanout);
  const int32_t e = sm.plist[pi] * L.fanout + (int32_t)(c - (int64_t)pi * L.fanout);
  return e < L.n ? e : -1;
}

__device__ __forceinline__ int32_t cand32(const Level& L, const SelectShared& sm, int32_t c) {
  if (L.fanout == 0) return c;
  const int32_t pi = parent_of(L, c);
  const int32_t e = sm.plist[pi] * L.fanout + (c - pi * L.fanout);
  return e < L.n ? e : -1;
}

__device__ __forceinline__ uint64_t composite(uint32_t key, int32_t e) {
  return ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)e);
}

// Puts key x in slot `slot` of the level's result; on a level that parents
// the next one (`kept` set) its element also becomes parent `slot` of the
// next level, with its keep flag set.
__device__ __forceinline__ void put_kept(SelectShared& sm, int32_t slot, uint64_t x, uint32_t* kept) {
  sm.buf[slot] = x;
  if (kept) {
    const int32_t e = (int32_t)(~(uint32_t)x);
    sm.plist[slot] = e;
    atomicOr(&kept[e >> 5], 1u << (e & 31));
  }
}

// Records the kept elements of a level (sm.buf[0, k_eff)) as the parents of
// the next level: their indices in plist and their bits in `kept` (clear on
// entry).
__device__ void keep_parents(SelectShared& sm, int32_t k_eff, uint32_t* kept) {
  const int tid = threadIdx.x;
  for (int32_t i = tid; i < k_eff; i += kSelThreads) {
    const int32_t e = (int32_t)(~(uint32_t)sm.buf[i]);
    sm.plist[i] = e;
    atomicOr(&kept[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
}

// Wave 0 finds the digit whose bucket holds the kk-th largest key.
__device__ void pick_digit(SelectShared& sm, int32_t kk) {
  const int lane = threadIdx.x;  // called with threadIdx.x < 64
  const uint32_t h0 = sm.hist[4 * lane], h1 = sm.hist[4 * lane + 1];
  const uint32_t h2 = sm.hist[4 * lane + 2], h3 = sm.hist[4 * lane + 3];
  const uint32_t local = h0 + h1 + h2 + h3;
  uint32_t suf = local;  // sum over lanes >= lane
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_down(suf, off, 64);
    if (lane + off < 64) suf += t;
  }
  uint32_t above = suf - local;  // keys in bins above this lane's four
  const uint32_t hb[4] = {h0, h1, h2, h3};
  const uint32_t want = (uint32_t)kk;
#pragma unroll
  for (int b = 3; b >= 0; --b) {
    const uint32_t upto = above + hb[b];
    if (above < want && want <= upto) {
      sm.digit = (uint32_t)(4 * lane + b);
      sm.above = above;
      sm.bucket = hb[b];
    }
    above = upto;
  }
}

// Sorts sm.buf[0, n) in descending key order (bitonic, padded with 0 keys).
__device__ void sort_desc(SelectShared& sm, int32_t n) {
  const int tid = threadIdx.x;
  int32_t N = 1;
  while (N < n) N <<= 1;
  for (int32_t i = n + tid; i < N; i += kSelThreads) sm.buf[i] = 0ull;
  __syncthreads();
  for (int32_t size = 2; size <= N; size <<= 1) {
    for (int32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (int32_t i = tid; i < (N >> 1); i += kSelThreads) {
        const int32_t lo = 2 * i - (i & (stride - 1));
        const int32_t hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t x = sm.buf[lo], y = sm.buf[hi];
        if (desc ? (x < y) : (x > y)) {
          sm.buf[lo] = y;
          sm.buf[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

// Sorts sm.buf[0, n) in descending order for n <= 64 distinct keys that
// all lie above 2^32 (positive scores): every wave holds the n keys (lane =
// key) and counts, for each, how many keys of its share of the lanes are
// larger, reading them with lane broadcasts; the counts are summed through
// LDS and give each key's slot.
__device__ void sort_desc_small(SelectShared& sm, int32_t n) {
  constexpr int W = kSelThreads / 64;
  constexpr int J = 64 / W;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint64_t x = lane < n ? sm.buf[lane] : (uint64_t)lane;  // padding below every real key
  const uint32_t xlo = (uint32_t)x, xhi = (uint32_t)(x >> 32);
  int32_t c = 0;
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    const int j = wave * J + jj;
    const uint64_t y = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)xhi, j) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)xlo, j);
    c += (int32_t)(y > x);
  }
  sm.part[wave][lane] = c;
  __syncthreads();
  if (wave == 0) {
    int32_t r = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) r += sm.part[w][lane];
    if (lane < n) sm.ck[r] = x;
  }
  __syncthreads();
  if (tid < n) sm.buf[tid] = sm.ck[tid];
  __syncthreads();
}

// Radix select over every positive candidate (re-enumerated each pass), for
// candidate sets too large to rank; leaves the top k_eff sorted in sm.buf.
// Bytes that every positive key shares (scores of one sequence often agree
// in their leading bits) are fixed up front from an AND / OR reduction, so
// the digit passes start at the first byte that tells keys apart.
template <bool STG>
__device__ void radix_top(const Level& L, int64_t m, int32_t k_eff, SelectShared& sm) {
  constexpr int W = kSelThreads / 64;
  const int tid = threadIdx.x;
  uint64_t all_and = ~0ull, any_or = 0ull;
  for (int64_t c = tid; c < m; c += kSelThreads) {
    const int32_t e = cand(L, sm, c);
    if (e < 0) continue;
    const uint32_t key = aff_key<STG>(L, sm, e);
    if (key == 0u) continue;
    const uint64_t comp = composite(key, e);
    all_and &= comp;
    any_or |= comp;
  }
  for (int o = 1; o < 64; o <<= 1) {
    all_and &= __shfl_xor(all_and, o, 64);
    any_or |= __shfl_xor(any_or, o, 64);
  }
  if ((tid & 63) == 0) {
    sm.ck[tid >> 6] = all_and;
    sm.ck[W + (tid >> 6)] = any_or;
  }
  __syncthreads();
  for (int w = 0; w < W; ++w) {
    all_and &= sm.ck[w];
    any_or |= sm.ck[W + w];
  }
  // keys are distinct, so some bit differs: digits of up to 8 bits start at
  // the highest differing bit and go down (a byte-aligned first digit would
  // put scores on either side of 0.5, which differ in the exponent's last
  // bit, into two bins and serialise the LDS atomics on them)
  const int hb = 63 - __clzll((long long)(all_and ^ any_or));
  uint64_t mask = hb >= 63 ? 0ull : ~((2ull << hb) - 1ull);
  uint64_t prefix = any_or & mask;
  int32_t kk = k_eff;
  for (int top = hb; top >= 0;) {
    const int sh = top >= 7 ? top - 7 : 0;
    const uint32_t dmask = (2u << (top - sh)) - 1u;
    for (int b = tid; b < 256; b += kSelThreads) sm.hist[b] = 0u;
    __syncthreads();
    for (int64_t c = tid; c < m; c += kSelThreads) {
      const int32_t e = cand(L, sm, c);
      if (e < 0) continue;
      const uint32_t key = aff_key<STG>(L, sm, e);
      if (key == 0u) continue;
      const uint64_t comp = composite(key, e);
      if ((comp & mask) == prefix) atomicAdd(&sm.hist[(uint32_t)(comp >> sh) & dmask], 1u);
    }
    __syncthreads();
    if (tid < 64) pick_digit(sm, kk);
    __syncthreads();
    prefix |= (uint64_t)sm.digit << sh;
    mask |= (uint64_t)dmask << sh;
    kk -= (int32_t)sm.above;
    const bool done = sm.bucket == (uint32_t)kk;
    __syncthreads();
    if (done) break;
    top = sh - 1;
  }
  if (tid == 0) sm.cnt[3] = 0;
  __syncthreads();
  for (int64_t c = tid; c < m; c += kSelThreads) {
    const int32_t e = cand(L, sm, c);
    if (e < 0) continue;
    const uint32_t key = aff_key<STG>(L, sm, e);
    if (key == 0u) continue;
    const uint64_t comp = composite(key, e);
    if (comp >= prefix) {
      const int32_t slot = atomicAdd(&sm.cnt[3], 1);
      if (slot < k_eff) sm.buf[slot] = comp;
    }
  }
  __syncthreads();
  if (k_eff <= 64) sort_desc_small(sm, k_eff);
  else sort_desc(sm, k_eff);
}

// When only P < k_eff candidates score above zero, the lowest-index rows
// scoring exactly 0 (masked, or live with zero affinity) take slots
// P .. k_eff-1 of sm.buf in index order (recorded as parents when `kept`
// is set).
template <bool STG>
__device__ void fill_zeros(const Level& L, SelectShared& sm, int32_t P, int32_t k_eff, uint32_t* kept) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const int32_t need = k_eff - P;
  int32_t found = 0;
  for (int32_t e0 = 0; e0 < L.n && found < need; e0 += kSelThreads) {
    const int32_t e = e0 + tid;
    const bool zero = e < L.n && (!is_live(L, e) || aff_key<STG>(L, sm, e) == 0u);
    const uint64_t bal = __ballot(zero);
    if (lane == 0) sm.wave_tot[wave] = (int32_t)__popcll(bal);
    __syncthreads();
    int32_t before = 0, tot = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) {
      if (w < wave) before += sm.wave_tot[w];
      tot += sm.wave_tot[w];
    }
    const int32_t rank = found + before + (int32_t)__popcll(bal & lt_mask);
    if (zero && rank < need) put_kept(sm, P + rank, composite(0u, e), kept);
    found += tot;
    __syncthreads();
  }
}

// Ranks the P <= kRankMax compacted positive keys sm.ck[0, P): rank r goes
// to sm.buf[r] when r < k_eff.  tpc consecutive lanes share a key, each
// counting a strided part with 8 LDS reads in flight.
__device__ void rank_compacted(SelectShared& sm, int32_t P, int32_t k_eff) {
  const int tid = threadIdx.x;
  int32_t tpc = 1;
  while (tpc < 16 && P * tpc * 2 <= kSelThreads) tpc <<= 1;
  for (int32_t t0 = 0; t0 < P * tpc; t0 += kSelThreads) {
    const int32_t t = t0 + tid;
    const int32_t i = t / tpc, q = t - i * tpc;
    const uint64_t x = i < P ? sm.ck[i] : ~0ull;
    int32_t r = 0;
    int32_t j = q;
    for (; j + 7 * tpc < P; j += 8 * tpc) {
      uint64_t y[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) y[u] = sm.ck[j + u * tpc];
#pragma unroll
      for (int u = 0; u < 8; ++u) r += (int32_t)(y[u] > x);
    }
    for (; j < P; j += tpc) r += (int32_t)(sm.ck[j] > x);
    for (int32_t o = 1; o < tpc; o <<= 1) r += __shfl_xor(r, o);
    if (q == 0 && i < P && r < k_eff) sm.buf[r] = x;
  }
  __syncthreads();
}

// Rows each thread covers in the flat staged path (row r * kSelThreads + tid).
constexpr int kKeysPerThread = (kLdsRows + kSelThreads - 1) / kSelThreads;

// Top k_eff of a flat level of m <= kKeysPerThread * kSelThreads rows staged
// in LDS, sorted, in sm.buf.  Every pass (positive count with the fixed
// leading bits, the radix digits, the gather) reads a thread's rows
// r * kSelThreads + tid straight from the LDS copy with all reads in
// flight; up to kRankMax positive scores are compacted and ranked instead.
__device__ int32_t select_flat_staged(const Level& L, int32_t m, int32_t k_eff, SelectShared& sm) {
  constexpr int W = kSelThreads / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const float* row = sm.aff + L.off;
  const int nr = (m + kSelThreads - 1) / kSelThreads;  // row slots in use (<= kKeysPerThread)
  auto key_at = [&](int r) -> uint32_t {
    const int32_t e = r * kSelThreads + tid;
    return e < m ? __float_as_uint(row[e]) : 0u;
  };
  uint64_t a_and = ~0ull, a_or = 0ull;
  int32_t npos = 0;
  for (int r = 0; r < nr; ++r) {
    const uint32_t kb = key_at(r);
    if (kb != 0u) {
      const uint64_t comp = composite(kb, r * kSelThreads + tid);
      a_and &= comp;
      a_or |= comp;
      ++npos;
    }
  }
  for (int o = 1; o < 64; o <<= 1) {
    a_and &= __shfl_xor(a_and, o, 64);
    a_or |= __shfl_xor(a_or, o, 64);
    npos += __shfl_xor(npos, o, 64);
  }
  if (lane == 0) {
    sm.ck[wave] = a_and;
    sm.ck[W + wave] = a_or;
    sm.wave_tot[wave] = npos;
  }
  __syncthreads();
  int32_t P = 0;
  for (int w = 0; w < W; ++w) {
    a_and &= sm.ck[w];
    a_or |= sm.ck[W + w];
    P += sm.wave_tot[w];
  }
  __syncthreads();  // sm.ck and sm.wave_tot are reused below
  if (P <= kRankMax) {
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    int32_t* cnt = &sm.cnt[L.slot];
    for (int r = 0; r < nr; ++r) {
      const uint32_t kb = key_at(r);
      const bool pos = kb != 0u;
      const uint64_t bal = __ballot(pos);
      int32_t base = 0;
      if (lane == 0 && bal) base = atomicAdd(cnt, (int32_t)__popcll(bal));
      base = __shfl(base, 0, 64);
      if (pos) sm.ck[base + (int32_t)__popcll(bal & lt_mask)] = composite(kb, r * kSelThreads + tid);
    }
    __syncthreads();
    rank_compacted(sm, P, k_eff);
  } else {
    // radix select of the top min(k_eff, P), as in radix_top
    const int32_t take = P >= k_eff ? k_eff : P;
    const int hb = 63 - __clzll((long long)(a_and ^ a_or));
    uint64_t mask = hb >= 63 ? 0ull : ~((2ull << hb) - 1ull);
    uint64_t prefix = a_or & mask;
    int32_t kk = take;
    for (int top = hb; top >= 0;) {
      const int sh = top >= 7 ? top - 7 : 0;
      const uint32_t dmask = (2u << (top - sh)) - 1u;
      for (int b = tid; b < 256; b += kSelThreads) sm.hist[b] = 0u;
      __syncthreads();
      for (int r = 0; r < nr; ++r) {
        const uint32_t kb = key_at(r);
        const uint64_t comp = composite(kb, r * kSelThreads + tid);
        if (kb != 0u && (comp & mask) == prefix) atomicAdd(&sm.hist[(uint32_t)(comp >> sh) & dmask], 1u);
      }
      __syncthreads();
      if (tid < 64) pick_digit(sm, kk);
      __syncthreads();
      prefix |= (uint64_t)sm.digit << sh;
      mask |= (uint64_t)dmask << sh;
      kk -= (int32_t)sm.above;
      const bool done = sm.bucket == (uint32_t)kk;
      __syncthreads();
      if (done) break;
      top = sh - 1;
    }
    if (tid == 0) sm.cnt[3] = 0;
    __syncthreads();
    for (int r = 0; r < nr; ++r) {
      const uint32_t kb = key_at(r);
      const uint64_t comp = composite(kb, r * kSelThreads + tid);
      if (kb != 0u && comp >= prefix) {
        const int32_t slot = atomicAdd(&sm.cnt[3], 1);
        if (slot < take) sm.buf[slot] = comp;
      }
    }
    __syncthreads();
    if (take <= 64) sort_desc_small(sm, take);
    else sort_desc(sm, take);
  }
  if (P < k_eff) fill_zeros<true>(L, sm, P, k_eff, nullptr);
  return k_eff;
}

// Keeps the top min(k, n) elements of a level with more candidates than
// threads, sorted, in sm.buf.  sm.cnt[L.slot] must be zero on entry.
template <bool STG>
__device__ int32_t select_big_sorted(const Level& L, int32_t k, SelectShared& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const int32_t k_eff = k < L.n ? k : L.n;
  if (k_eff <= 0) return 0;
  const int64_t m = L.fanout ? (int64_t)L.n_par * L.fanout : (int64_t)L.n;
  if constexpr (STG) {
    if (L.fanout == 0 && m <= (int64_t)kKeysPerThread * kSelThreads)
      return select_flat_staged(L, (int32_t)m, k_eff, sm);
  }
  int32_t* cnt = &sm.cnt[L.slot];
  // compact the candidates scoring above zero
  for (int64_t c0 = 0; c0 < m; c0 += kSelThreads) {
    const int64_t c = c0 + tid;
    const int32_t e = c < m ? cand(L, sm, c) : -1;
    const uint32_t key = e >= 0 ? aff_key<STG>(L, sm, e) : 0u;
    const bool pos = key != 0u;
    const uint64_t bal = __ballot(pos);
    int32_t base = 0;
    if (lane == 0 && bal) base = atomicAdd(cnt, (int32_t)__popcll(bal));
    base = __shfl(base, 0, 64);
    const int32_t slot = base + (int32_t)__popcll(bal & lt_mask);
    if (pos && slot < kRankMax) sm.ck[slot] = composite(key, e);
  }
  __syncthreads();
  const int32_t P = *cnt;
  if (P > kRankMax) {
    // too many to rank: radix select the top k_eff, or (when k_eff is larger
    // still) all P positive candidates, sorted; zeros fill the rest below
    const int32_t take = P >= k_eff ? k_eff : P;
    radix_top<STG>(L, m, take, sm);
    if (P >= k_eff) return k_eff;
  } else {
    // rank the positive candidates: rank r goes to slot r when r < k_eff
    rank_compacted(sm, P, k_eff);
    if (P >= k_eff) return k_eff;
  }
  fill_zeros<STG>(L, sm, P, k_eff, nullptr);
  return k_eff;
}

// select_big_sorted, then (on a level that parents the next one) its
// results recorded as parents.
template <bool STG>
__device__ int32_t select_level_big(const Level& L, int32_t k, SelectShared& sm, uint32_t* kept) {
  const int32_t k_eff = select_big_sorted<STG>(L, k, sm);
  if (kept) keep_parents(sm, k_eff, kept);
  return k_eff;
}

// Sum of v over lanes [lane, lane + n) of the same 16-lane row (n = 1, 2, 4
// or 8; exact for lanes that start an aligned group of n).
__device__ __forceinline__ int32_t group_sum(int32_t v, int32_t n) {
  if (n >= 2) v += __builtin_amdgcn_update_dpp(0, v, 0x101, 0xF, 0xF, false);  // row_shl:1
  if (n >= 4) v += __builtin_amdgcn_update_dpp(0, v, 0x102, 0xF, 0xF, false);  // row_shl:2
  if (n >= 8) v += __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, false);  // row_shl:4
  return v;
}

// Keys of the strictly descending run g that exceed x, from two rounds of
// 16-byte LDS reads: the run's 8 block-end keys give the number c of whole
// blocks of 8 above x (the same addresses for every lane counting run g),
// then the 8 keys of block c give the position inside it.
__device__ __forceinline__ int32_t run_count_above(const SortedRuns& R, int32_t g, uint64_t x) {
  const u64x2* pv = reinterpret_cast<const u64x2*>(R.piv + 8 * g);
  int32_t c = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const u64x2 v = pv[p];
    c += (int32_t)(v.x > x) + (int32_t)(v.y > x);
  }
  const u64x2* bk = reinterpret_cast<const u64x2*>(R.key + 64 * g + 8 * (c < 8 ? c : 7));
  int32_t f = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const u64x2 v = bk[p];
    f += (int32_t)(v.x > x) + (int32_t)(v.y > x);
  }
  return c == 8 ? 64 : 8 * c + f;
}

// Lanes that share one key when NG groups of 64 keys are ranked by
// kSelThreads threads: the largest power of two up to 8 that fits.
constexpr int rank_tpc(int ng) {
  int t = 1;
  while (t < 8 && ng * 64 * t * 2 <= kSelThreads) t <<= 1;
  return t;
}

// Keeps the top k_eff of a level's 64 < m <= NG * 64 candidates, sorted,
// in sm.buf.  The candidates form NG groups of 64 (slots past the
// candidates hold distinct keys below every real one).  TPC waves rank a
// group: each stores the group's keys to a copy of its own in LDS, and TPC
// lanes rank each key within the group, each comparing a contiguous share.
// Each group is written back as a strictly descending run (with its
// block-end keys) and a key's rank in the level is the number of keys above
// it summed over all runs, its own included (run_count_above), the runs
// split among its TPC lanes.  Keys without a positive score rank below all
// positive ones and are never kept here (the zero fill handles them).
template <bool STG, int NG>
__device__ int32_t select_small(const Level& L, int32_t m, int32_t k_eff, SelectShared& sm, uint32_t* kept) {
  constexpr int TPC = rank_tpc(NG);
  constexpr int SPAN = 64 / TPC;            // keys of its group one lane compares
  constexpr int RPL = (NG + TPC - 1) / TPC;  // runs one lane counts in
  static_assert(NG >= 2 && NG * 64 * TPC <= kSelThreads && SPAN % 8 == 0, "rank layout");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int32_t g = wave / TPC;   // group this wave ranks
  const bool active = g < NG;     // whole waves
  const int32_t q = lane % TPC;   // this lane's share of its key's comparisons
  uint64_t x = 0;
  if (active) {
    const int32_t c = 64 * g + lane;
    const int32_t e = c < m ? cand32(L, sm, c) : -1;
    const uint32_t key = e >= 0 ? aff_key<STG>(L, sm, e) : 0u;
    const uint64_t bal = __ballot(key != 0u);
    if (lane == 0 && wave % TPC == 0) sm.wave_tot[g] = (int32_t)__popcll(bal);
    uint64_t* copy = sm.ck + 64 * wave;
    copy[lane] = e >= 0 ? composite(key, e) : (uint64_t)c;
    // lanes of this wave read each other's stores: wave-scope synchronisation
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // the wave's 64 / TPC keys are consecutive in the group
    x = copy[SPAN * (wave % TPC) + lane / TPC];
    const u64x2* share = reinterpret_cast<const u64x2*>(copy + q * SPAN);
    int32_t r = 0;
#pragma unroll
    for (int j = 0; j < SPAN / 2; j += 4) {
      u64x2 y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) y[u] = share[j + u];
#pragma unroll
      for (int u = 0; u < 4; ++u) r += (int32_t)(y[u].x > x) + (int32_t)(y[u].y > x);
    }
    r = group_sum(r, TPC);
    if (q == 0) {
      sm.runs.key[64 * g + r] = x;
      if ((r & 7) == 7) sm.runs.piv[8 * g + (r >> 3)] = x;
    }
  }
  __syncthreads();
  int32_t P = 0;
  for (int w = 0; w < NG; ++w) P += sm.wave_tot[w];
  // rank in the level; lane q counts in runs q, q + TPC, ...
  if (active) {
    int32_t R = 0;
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
      const int32_t gg = q + t * TPC;
      const int32_t above = run_count_above(sm.runs, gg < NG ? gg : NG - 1, x);
      R += gg < NG ? above : 0;
    }
    R = group_sum(R, TPC);
    if (q == 0 && (x >> 32) != 0ull && R < k_eff) put_kept(sm, R, x, kept);
  }
  __syncthreads();
  if (P < k_eff) fill_zeros<STG>(L, sm, P, k_eff, kept);
  return k_eff;
}

// Keeps the top k_eff of a level of at most 64 candidates, sorted, in
// sm.buf.  Every wave builds the 64 candidate keys (lane = candidate; lanes
// past the candidates hold distinct keys below every real one) and stores
// them to a copy of its own in LDS; then each wave ranks its share of the
// candidates: W lanes share a key, each counting the larger keys among a
// contiguous share of the copy, and a DPP sum over the W lanes gives the
// rank, which is the key's result slot.  One barrier per level (two when
// the level both reads and rewrites the parent list).
template <bool STG>
__device__ int32_t select_one_group(const Level& L, int32_t m, int32_t k_eff, SelectShared& sm, uint32_t* kept) {
  constexpr int W = kSelThreads / 64;  // waves = lanes per key
  constexpr int CPW = 64 / W;          // keys each wave ranks = keys each lane compares
  static_assert(W * CPW == 64 && W <= 8 && CPW % 4 == 0, "wave layout");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int32_t e = lane < m ? cand32(L, sm, lane) : -1;
  const uint32_t key = e >= 0 ? aff_key<STG>(L, sm, e) : 0u;
  const int32_t P = (int32_t)__popcll(__ballot(key != 0u));
  uint64_t* copy = sm.ck + 64 * wave;
  copy[lane] = e >= 0 ? composite(key, e) : (uint64_t)lane;
  // lanes of this wave read each other's stores: wave-scope synchronisation
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t x = copy[CPW * wave + lane / W];
  const u64x2* share = reinterpret_cast<const u64x2*>(copy + CPW * (lane % W));
  int32_t r = 0;
#pragma unroll
  for (int u = 0; u < CPW / 2; ++u) {
    const u64x2 y = share[u];
    r += (int32_t)(y.x > x) + (int32_t)(y.y > x);
  }
  r = group_sum(r, W);
  // The kept elements overwrite the parent list that other waves may still
  // be reading for this level's candidates: wait for every wave first.
  if (kept && L.fanout > 0) __syncthreads();
  if (lane % W == 0 && (x >> 32) != 0ull && r < k_eff) put_kept(sm, r, x, kept);
  __syncthreads();
  if (P < k_eff) fill_zeros<STG>(L, sm, P, k_eff, kept);
  return k_eff;
}

// Picks the group count: the smallest NG >= 2 with m <= NG * 64.
template <bool STG, int NG>
__device__ __forceinline__ int32_t select_small_ng(const Level& L, int32_t m, int32_t k_eff, SelectShared& sm,
                                                   uint32_t* kept) {
  if constexpr (NG * 64 < kSelThreads) {
    if (m > NG * 64) return select_small_ng<STG, NG + 1>(L, m, k_eff, sm, kept);
  }
  return select_small<STG, NG>(L, m, k_eff, sm, kept);
}

// Keeps the top min(k, n) elements of a level, sorted, in sm.buf: levels
// with at most kSelThreads candidates are ranked, larger ones compacted and
// ranked or radix-selected.  With `kept` set (a level that parents the next
// one) the kept elements are also recorded as the next level's parents: in
// plist, in rank order, and as bits of `kept` (clear on entry).  Everything
// is visible to the whole work-group on return.
template <bool STG>
__device__ int32_t select_level(const Level& L, int32_t k, SelectShared& sm, uint32_t* kept) {
  const int32_t k_eff = k < L.n ? k : L.n;
  if (k_eff <= 0) return 0;
  const int64_t m64 = L.fanout ? (int64_t)L.n_par * L.fanout : (int64_t)L.n;
  if (m64 > kSelThreads) return select_level_big<STG>(L, k, sm, kept);
  if (m64 <= 64) return select_one_group<STG>(L, (int32_t)m64, k_eff, sm, kept);
  return select_small_ng<STG, 2>(L, (int32_t)m64, k_eff, sm, kept);
}

struct SeqGeom {
  int32_t n_p, n_c, n_g;
};

// Level sizes of a sequence of n_p pages (the value read from a.n_pages).
__device__ __forceinline__ SeqGeom geom_of(const ScoreArgs& a, int32_t n_p, bool report) {
  SeqGeom g;
  g.n_p = n_p;
  if (g.n_p < 0 || g.n_p > a.max_pages) {
    if (report) raise_err(a.err, KKA_DEVERR_PAGES);
    g.n_p = g.n_p < 0 ? 0 : a.max_pages;
  }
  g.n_c = a.hier ? (g.n_p + a.ppc - 1) / a.ppc : 0;
  g.n_g = a.hier ? (g.n_c + a.cpg - 1) / a.cpg : 0;
  return g;
}

__device__ __forceinline__ SeqGeom seq_geom(const ScoreArgs& a, int32_t s, bool report) {
  return geom_of(a, a.n_pages[s], report);
}

// Copies a sequence's whole affinity row block src[0, n) (n <= kLdsRows)
// into LDS with one round of device-scope loads, every load issued before
// the first store.  Rows that are not present are copied too and never
// read.
__device__ __forceinline__ void stage_rows(float* dst, const float* src, int32_t n) {
  constexpr int U = (kLdsRows + kSelThreads - 1) / kSelThreads;
  const int tid = threadIdx.x;
  if (n <= 0) return;
  // Clamped indices make every load and store unconditional; the clamped
  // copies write the value the last slot holds anyway.
  float t[U];
#pragma unroll
  for (int u = 0; u < U; ++u) t[u] = load_agent(src + min(u * kSelThreads + tid, n - 1));
#pragma unroll
  for (int u = 0; u < U; ++u) dst[min(u * kSelThreads + tid, n - 1)] = t[u];
}

// Level `lev` (0 grids, 1 chunks of kept grids, 2 pages of kept chunks or
// every page when flat) of sequence geometry g; kp = kept count of the
// level above.
__device__ __forceinline__ Level make_level(const ScoreArgs& a, const SeqGeom& g, int32_t lev, const float* aff,
                                            int32_t kp, SelectShared& sm) {
  Level L;
  L.slot = lev;
  if (lev == 0) {
    L.off = a.max_pages + a.c_cap;
    L.n = g.n_g;
    L.fanout = 0;
    L.parent = nullptr;
  } else if (lev == 1) {
    L.off = a.max_pages;
    L.n = g.n_c;
    L.fanout = a.cpg;
    L.parent = sm.kept_grid;
  } else {
    L.off = 0;
    L.n = g.n_p;
    L.fanout = a.hier ? a.ppc : 0;
    L.parent = sm.kept_chunk;
  }
  L.aff = aff + L.off;
  L.n_par = kp;
  L.shift = (L.fanout > 0 && (L.fanout & (L.fanout - 1)) == 0) ? __builtin_ctz((unsigned)L.fanout) : -1;
  return L;
}

__device__ __forceinline__ void clear_select_state(const ScoreArgs& a, const SeqGeom& g, SelectShared& sm) {
  const int tid = threadIdx.x;
  if (tid < 4) sm.cnt[tid] = 0;
  if (a.hier) {
    for (int32_t w = tid; w < (g.n_g + 31) / 32; w += kSelThreads) sm.kept_grid[w] = 0u;
    for (int32_t w = tid; w < (g.n_c + 31) / 32; w += kSelThreads) sm.kept_chunk[w] = 0u;
  }
}

__device__ __forceinline__ void write_selection(const ScoreArgs& a, const SelectShared& sm, int32_t s, int32_t kp) {
  const int tid = threadIdx.x;
  for (int32_t i = tid; i < a.k_p; i += kSelThreads) {
    int32_t idx = -1;
    float sc = 0.f;
    if (i < kp) {
      const uint64_t c = sm.buf[i];
      idx = (int32_t)(~(uint32_t)c);
      sc = __uint_as_float((uint32_t)(c >> 32));
    }
    a.idx_out[(int64_t)s * a.k_p + i] = idx;
    if (a.score_out) a.score_out[(int64_t)s * a.k_p + i] = sc;
  }
  if (tid == 0 && a.cnt_out) a.cnt_out[s] = kp;
}

// Selects grids, chunks of kept grids and pages of kept chunks (pages only
// when flat); returns the kept page count.
template <bool STG>
__device__ __forceinline__ int32_t select_levels(const ScoreArgs& a, const SeqGeom& g, const float* aff, SelectShared& sm) {
  int32_t kp = 0;
  for (int32_t lev = a.hier ? 0 : 2; lev < 3; ++lev) {
    const Level L = make_level(a, g, lev, aff, kp, sm);
    kp = select_level<STG>(L, lev == 0 ? a.k_g : (lev == 1 ? a.k_c : a.k_p), sm,
                           lev == 0 ? sm.kept_grid : (lev == 1 ? sm.kept_chunk : nullptr));
  }
  return kp;
}

// ------------------------------------------- lean selection of small levels
//
// Hierarchical levels small enough to rank without the general machinery:
// at most 64 grids, at most 64 chunk candidates (children of the kept
// grids) and at most 256 page candidates, at most 64 kept per level (the
// serving and 128K shapes: 32 grids, 4 x 16 chunks, 16 x 16 pages, top
// 4 / 16 / 64).  Wavefront 0 stages the chunk and grid rows and ranks
// grids and chunks alone, with no work-group barrier, while the page rows
// are still arriving; four wavefronts then rank the page candidates, each
// its 64 among themselves (a sorted run), then against the other three
// runs.  A level with fewer positive-score candidates than it keeps needs
// the zero fill, and the general path selects instead, from the same
// staged rows.

// x / d for a wave-uniform d >= 1: a shift when d is a power of two.
__device__ __forceinline__ int32_t div_fan(int32_t x, int32_t d) {
  return (d & (d - 1)) == 0 ? x >> __builtin_ctz((unsigned)d) : x / d;
}

// Lanes of one wavefront read each other's LDS stores.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Keys among the wavefront's first m (lane l's key stored at copy[l]; m
// wave-uniform, a multiple of 32 at most 64) larger than this lane's x.
// The rank is a chain of LDS round trips and compares, so it is written
// for latency: up to 32 keys (16 reads) in flight at once, and four
// independent counts.
__device__ __forceinline__ int32_t rank_in_wave(uint64_t x, uint64_t* copy, int32_t m) {
  wave_sync();  // earlier reads of the copy are done
  copy[threadIdx.x & 63] = x;
  wave_sync();
  const u64x2* p = reinterpret_cast<const u64x2*>(copy);
  int32_t r[4] = {0, 0, 0, 0};
  for (int u = 0; u < m / 2; u += 16) {
    u64x2 y[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) y[v] = p[u + v];
#pragma unroll
    for (int v = 0; v < 16; ++v) r[v & 3] += (int32_t)(y[v].x > x) + (int32_t)(y[v].y > x);
    // the scheduler would otherwise hoist the next 16 reads too (spills)
    __builtin_amdgcn_sched_barrier(0);
  }
  return (r[0] + r[1]) + (r[2] + r[3]);
}

// Top k of up to 64 candidates on one wavefront: lane l < m holds
// candidate l (element e, or -1, and its score bits); the kept elements go
// to list[rank].  Candidates without a positive score take keys below every
// positive one (the lane number).  False when fewer than k score above 0.
__device__ __forceinline__ bool rank_level64(int32_t e, uint32_t bits, int32_t k, int32_t m, uint64_t* copy,
                                             int32_t* list) {
  const int lane = threadIdx.x & 63;
  const bool pos = e >= 0 && bits != 0u;
  const uint64_t x = pos ? composite(bits, e) : (uint64_t)lane;
  // lanes from m on hold no candidate: their keys (below every positive
  // one) need not be compared
  const int32_t r = rank_in_wave(x, copy, min((m + 31) & ~31, 64));
  if ((int32_t)__popcll(__ballot(pos)) < k) return false;
  if (pos && r < k) list[r] = e;
  wave_sync();
  return true;
}

// Keys of the three runs other than run w (of four strictly descending runs
// of 64, with their block-end keys) larger than x: as run_count_above for
// each, with the three runs' reads of a round in flight together.
__device__ __forceinline__ int32_t count_above_other_runs(const SortedRuns& R, int32_t w, uint64_t x) {
  int32_t c[3];
  {
    u64x2 pv[3][4];
#pragma unroll
    for (int v = 0; v < 3; ++v) {
      const u64x2* p = reinterpret_cast<const u64x2*>(R.piv + 8 * ((w + 1 + v) & 3));
#pragma unroll
      for (int q = 0; q < 4; ++q) pv[v][q] = p[q];
    }
#pragma unroll
    for (int v = 0; v < 3; ++v) {
      int32_t n = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) n += (int32_t)(pv[v][q].x > x) + (int32_t)(pv[v][q].y > x);
      c[v] = n;
    }
  }
  u64x2 bk[3][4];
#pragma unroll
  for (int v = 0; v < 3; ++v) {
    const u64x2* p = reinterpret_cast<const u64x2*>(R.key + 64 * ((w + 1 + v) & 3) + 8 * (c[v] < 8 ? c[v] : 7));
#pragma unroll
    for (int q = 0; q < 4; ++q) bk[v][q] = p[q];
  }
  int32_t total = 0;
#pragma unroll
  for (int v = 0; v < 3; ++v) {
    int32_t f = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) f += (int32_t)(bk[v][q].x > x) + (int32_t)(bk[v][q].y > x);
    total += c[v] == 8 ? 64 : 8 * c[v] + f;
  }
  return total;
}

// Top k (<= 64) of up to 256 candidates: thread t < 256 holds candidate t;
// every thread of the work-group calls it.  Each of wavefronts 0-3 ranks
// its 64 keys, writes them as a strictly descending run (with every eighth
// key), and a key's rank is its place in its run plus the keys above it in
// the other three runs.  Kept keys go to sm.buf[rank].  False (in every
// thread) when fewer than k score above 0.
__device__ __forceinline__ bool rank_level256(int32_t e, uint32_t bits, int32_t k, SelectShared& sm) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pos = e >= 0 && bits != 0u;
  const uint64_t x = pos ? composite(bits, e) : (uint64_t)tid;
  int32_t r = 0;
  if (wave < 4) {
    r = rank_in_wave(x, sm.ck + 64 * wave, 64);
    const uint64_t bal = __ballot(pos);
    if (lane == 0) sm.wave_tot[wave] = (int32_t)__popcll(bal);
    sm.runs.key[64 * wave + r] = x;
    if ((r & 7) == 7) sm.runs.piv[8 * wave + (r >> 3)] = x;
  }
  __syncthreads();
  const int32_t P = sm.wave_tot[0] + sm.wave_tot[1] + sm.wave_tot[2] + sm.wave_tot[3];
  if (P < k) return false;
  if (wave < 4) {
    const int32_t R = r + count_above_other_runs(sm.runs, wave, x);
    if (pos && R < k) sm.buf[R] = x;
  }
  __syncthreads();
  return true;
}

// Stages the sequence's affinity rows into LDS and selects its levels on
// the lean path; returns the kept page count, or -1 when a level needs the
// zero fill (every row is staged either way).
__device__ __forceinline__ int32_t select_lean_levels(const ScoreArgs& a, const SeqGeom& g, const float* aff,
                                                      SelectShared& sm) {
  constexpr int NP = kSelThreads - 64;          // threads staging the page rows
  constexpr int UP = (kLdsRows + NP - 1) / NP;  // page rows per thread, at most
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t n_lo = a.max_pages;                             // page rows
  const int32_t n_hi = (int32_t)a.rows_per_seq - a.max_pages;  // chunk and grid rows
  const int32_t kg = min(a.k_g, g.n_g), kc = min(a.k_c, g.n_c), kp = min(a.k_p, g.n_p);
  if (wave == 0) {
    // wavefront 0 stages the chunk and grid rows and ranks grids and chunks
    // while the other wavefronts stage the page rows
    // clamped, unconditional loads and stores (a slot past the rows repeats
    // the last one): each store then waits for its own load only
    float hi[kLeanHiRows / 64];
#pragma unroll
    for (int u = 0; u < kLeanHiRows / 64; ++u) hi[u] = load_agent(aff + n_lo + min(u * 64 + lane, n_hi - 1));
#pragma unroll
    for (int u = 0; u < kLeanHiRows / 64; ++u) sm.aff[n_lo + min(u * 64 + lane, n_hi - 1)] = hi[u];
    wave_sync();
    const int32_t off_g = a.max_pages + a.c_cap;
    const int32_t eg = lane < g.n_g ? lane : -1;
    bool good = rank_level64(eg, eg >= 0 ? __float_as_uint(sm.aff[off_g + eg]) : 0u, kg, g.n_g, sm.ck, sm.plist);
    if (good) {
      const int32_t pr = div_fan(lane, a.cpg);
      int32_t ec = -1;
      if (pr < kg) {
        const int32_t c = sm.plist[pr] * a.cpg + (lane - pr * a.cpg);
        ec = c < g.n_c ? c : -1;
      }
      good = rank_level64(ec, ec >= 0 ? __float_as_uint(sm.aff[a.max_pages + ec]) : 0u, kc, kg * a.cpg, sm.ck,
                          sm.plist + 64);
    }
    if (lane == 0) sm.cnt[0] = good ? 1 : 0;
  } else {
    const int t = tid - 64;
    float lo[UP];
#pragma unroll
    for (int u = 0; u < UP; ++u) lo[u] = load_agent(aff + min(u * NP + t, n_lo - 1));
#pragma unroll
    for (int u = 0; u < UP; ++u) sm.aff[min(u * NP + t, n_lo - 1)] = lo[u];
  }
  __syncthreads();
  if (sm.cnt[0] == 0) return -1;
  int32_t ep = -1;
  if (tid < 256) {
    const int32_t pr = div_fan(tid, a.ppc);
    if (pr < kc) {
      const int32_t p = sm.plist[64 + pr] * a.ppc + (tid - pr * a.ppc);
      ep = p < g.n_p ? p : -1;
    }
  }
  if (!rank_level256(ep, ep >= 0 ? __float_as_uint(sm.aff[ep]) : 0u, kp, sm)) return -1;
  return kp;
}

// The general path restricted to the levels of a lean layout (at most 256
// candidates a level): for the rare lean sequence that needs the zero fill.
__device__ __forceinline__ int32_t select_level_lean(const Level& L, int32_t k, SelectShared& sm, uint32_t* kept) {
  const int32_t k_eff = k < L.n ? k : L.n;
  if (k_eff <= 0) return 0;
  const int32_t m = L.fanout ? L.n_par * L.fanout : L.n;
  if (m <= 64) return select_one_group<true>(L, m, k_eff, sm, kept);
  if (m <= 128) return select_small<true, 2>(L, m, k_eff, sm, kept);
  if (m <= 192) return select_small<true, 3>(L, m, k_eff, sm, kept);
  return select_small<true, 4>(L, m, k_eff, sm, kept);
}

// Selection of sequence s from its affinity rows in a.aff, by the whole
// work-group.  LEAN: the layout passes lean_levels_fit.
template <bool LEAN>
__device__ __forceinline__ void select_sequence(const ScoreArgs& a, int32_t s, SelectShared& sm) {
  const float* aff = a.aff + (int64_t)s * a.rows_per_seq;
  const SeqGeom g = seq_geom(a, s, false);  // issued before the staging loads
  if constexpr (LEAN) {
    int32_t kp = select_lean_levels(a, g, aff, sm);  // stages every row
    if (kp < 0) {
      // a level needs the zero fill: the general path on the staged rows
      clear_select_state(a, g, sm);
      __syncthreads();
      kp = 0;
      for (int32_t lev = 0; lev < 3; ++lev) {
        const Level L = make_level(a, g, lev, aff, kp, sm);
        kp = select_level_lean(L, lev == 0 ? a.k_g : (lev == 1 ? a.k_c : a.k_p), sm,
                               lev == 0 ? sm.kept_grid : (lev == 1 ? sm.kept_chunk : nullptr));
      }
    }
    write_selection(a, sm, s, kp);
  } else {
    const bool staged = a.rows_per_seq <= kLdsRows;
    if (staged) stage_rows(sm.aff, aff, (int32_t)a.rows_per_seq);
    clear_select_state(a, g, sm);
    __syncthreads();
    const int32_t kp = staged ? select_levels<true>(a, g, aff, sm) : select_levels<false>(a, g, aff, sm);
    write_selection(a, sm, s, kp);
  }
}

template <bool LEAN>
__global__ __launch_bounds__(kSelThreads) void select_kernel(ScoreArgs a) {
  __shared__ SelectShared sm;
  select_sequence<LEAN>(a, blockIdx.x, sm);
}

// (1 + cos) / 2 clamped to [0, 1]; NaN and -0 become +0.
__device__ __forceinline__ float affinity_of(float dot, float nr, float sqrt_na, float na) {
  const float c = (nr > 0.f && na > 0.f) ? dot / (sqrtf(nr) * sqrt_na) : 0.f;
  const float v = 0.5f * (1.0f + c);
  return v > 0.f ? (v < 1.f ? v : 1.f) : 0.f;
}

// Buffer-resource loads: a raw buffer load whose byte offset lies past the
// resource's range (at most 2^31 - 1 bytes) reads zero and touches no
// memory, so a lane without data issues the same load as the others, with
// no branch and no select, and every load of a pass is in flight at once.
constexpr int32_t kOutOfRange = 0x7ffffff0;  // a byte offset past any range here
constexpr int kBufAux = KKA_SCORE_NT ? 2 : 0;  // cache policy bits of row loads: 2 = non-temporal

// The row buffers built here span a lean layout's rows (at most
// kSelectLdsRows of at most head_dim 1024 floats): within the 2^31 bytes a
// resource's range and its 32-bit offsets cover.
static_assert((int64_t)kSelectLdsRows * 1024 * 4 < ((int64_t)1 << 31), "lean row buffers exceed a buffer resource");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int64_t bytes) {
  // gfx9 raw buffer: stride 0, `bytes` records of one byte, default format word
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int32_t)bytes, 0x00020000);
}

// The anchor as held by one lane of an LPR-lane row group: float4 pieces
// lg, lg + LPR, ... of the row, plus the squared norm (every lane of the
// group holds the full sum after a fixed butterfly).
template <int LPR, int NQ>
struct AnchorRegs {
  f32x4 av[NQ];
  float na, sqrt_na;
};

// The anchor's pieces go through a buffer resource over its head_dim
// floats: a piece past head_dim reads zero without a branch, so the loads
// never wait for one another (nor for row loads already in flight).
// issue_anchor requests the pieces, finish_anchor forms the norm once they
// are needed; load_anchor does both.
template <int LPR, int NQ>
__device__ __forceinline__ void issue_anchor(const ScoreArgs& a, int32_t s, int32_t lg, AnchorRegs<LPR, NQ>& r) {
  const int32_t Q = a.D >> 2;
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(a.anchors + (int64_t)s * a.D, (int64_t)a.D * 4);
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int32_t qi = lg + LPR * j;
    const int32_t off = qi < Q ? qi * 16 : kOutOfRange;
    r.av[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  }
}

template <int LPR, int NQ>
__device__ __forceinline__ void finish_anchor(AnchorRegs<LPR, NQ>& r) {
  r.na = 0.f;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    r.na = fmaf(r.av[j].x, r.av[j].x, r.na);
    r.na = fmaf(r.av[j].y, r.av[j].y, r.na);
    r.na = fmaf(r.av[j].z, r.av[j].z, r.na);
    r.na = fmaf(r.av[j].w, r.av[j].w, r.na);
  }
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) r.na += __shfl_xor(r.na, o);
  r.sqrt_na = sqrtf(r.na);
}

template <int LPR, int NQ>
__device__ __forceinline__ AnchorRegs<LPR, NQ> load_anchor(const ScoreArgs& a, int32_t s, int32_t lg) {
  AnchorRegs<LPR, NQ> r;
  issue_anchor<LPR, NQ>(a, s, lg, r);
  finish_anchor<LPR, NQ>(r);
  return r;
}

// Loads this lane's pieces of one row (unconditional, from a clamped
// in-bounds address; pieces past head_dim read as zero).
template <int LPR, int NQ>
__device__ __forceinline__ void load_row(const f32x4* rowp, int32_t lg, int32_t Q, f32x4 (&x)[NQ]) {
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int32_t qi = lg + LPR * j;
    const f32x4 t = load_row4(rowp + min(qi, Q - 1));
    x[j] = qi < Q ? t : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// This lane's pieces of row `row` of the resource (row < 0: zeros, nothing
// read); pieces past head_dim read as zero.
template <int LPR, int NQ>
__device__ __forceinline__ void load_row_buf(__amdgpu_buffer_rsrc_t rs, int32_t row, int32_t lg, int32_t Q,
                                             f32x4 (&x)[NQ]) {
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int32_t qi = lg + LPR * j;
    const int32_t off = row >= 0 && qi < Q ? (row * Q + qi) * 16 : kOutOfRange;
    x[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kBufAux));
  }
}

// Affinity of one row from its loaded pieces: fixed FMA order per lane,
// fixed butterfly over the group, so every caller gets the same bits.
template <int LPR, int NQ>
__device__ __forceinline__ float row_affinity(const f32x4 (&x)[NQ], const AnchorRegs<LPR, NQ>& A) {
  float dot = 0.f, nr = 0.f;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    dot = fmaf(x[j].x, A.av[j].x, dot);
    dot = fmaf(x[j].y, A.av[j].y, dot);
    dot = fmaf(x[j].z, A.av[j].z, dot);
    dot = fmaf(x[j].w, A.av[j].w, dot);
    nr = fmaf(x[j].x, x[j].x, nr);
    nr = fmaf(x[j].y, x[j].y, nr);
    nr = fmaf(x[j].z, x[j].z, nr);
    nr = fmaf(x[j].w, x[j].w, nr);
  }
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) {
    dot += __shfl_xor(dot, o);
    nr += __shfl_xor(nr, o);
  }
  return affinity_of(dot, nr, A.sqrt_na, A.na);
}

// Stability window of one page after this step (section 5.3): the word
// shifts by one step and takes the new step's bit (affinity above theta);
// the score is the fraction of set bits over the window length.
__device__ __forceinline__ void stability_step(const ScoreArgs& a, uint32_t h, float v_aff, uint32_t* hist,
                                               float* stab) {
  const uint32_t nh = ((h << 1) | (v_aff > a.theta ? 1u : 0u)) & a.stab_mask;
  *hist = nh;
  if (stab) *stab = (float)__popc(nh) / (float)a.stab_w;
}

// One scoring tile: rows [tile * rows_per_tile, ...) of sequence s, by NT
// threads in row groups of LPR lanes, R rows per group per pass.  Used by
// the scoring launch of the two-launch path and by the streaming
// work-groups of the one-launch path.  With the stability filter a tile's
// affinities are gathered in LDS (g_aff) and the affinities, window words
// and scores are read and written one row per thread, as whole lines: one
// lane per row group would write a quarter line per store (measured 2.5 %
// slower on the serving batch).  Without affinity_out and without the
// filter there is nothing to write and the caller does not launch tiles.
template <int NT, int LPR, int NQ, int R, bool STAB>
__device__ __forceinline__ void score_tile(const ScoreArgs& a, int32_t s, int32_t tile, float* g_aff) {
  constexpr int NG = NT / LPR;  // row groups per work-group
  const int tid = threadIdx.x;
  const int32_t v0 = tile * a.rows_per_tile;
  const int32_t Q = a.D >> 2;
  const f32x4* seq = reinterpret_cast<const f32x4*>(a.lvl + (int64_t)s * a.rows_per_seq * a.D);
  float* aff = a.aff ? a.aff + (int64_t)s * a.rows_per_seq : nullptr;
  const int32_t grp = tid / LPR, lg = tid % LPR;
  // The first pass's rows are requested together with the page count and
  // the anchor: row v is physical row v whenever v < n_p or the sequence
  // fills its capacity (every level full), the case of most tiles; a tile
  // whose guess the page count proves wrong loads them again.
  if (a.rows_per_seq <= 0) return;
  const int32_t n_p_v = __hip_atomic_load(a.n_pages + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  AnchorRegs<LPR, NQ> A;
  issue_anchor<LPR, NQ>(a, s, lg, A);
  f32x4 x[R][NQ];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t vr = v0 + grp + NG * r;
    load_row<LPR, NQ>(seq + (vr < a.rows_per_seq ? vr : a.rows_per_seq - 1) * Q, lg, Q, x[r]);
  }
  __builtin_amdgcn_sched_barrier(0);
  finish_anchor<LPR, NQ>(A);
  const SeqGeom g = geom_of(a, __builtin_amdgcn_readfirstlane(n_p_v), false);
  const int32_t nv = g.n_p + g.n_c + g.n_g;
  if (v0 >= nv) return;
  const int32_t v1 = min(nv, v0 + a.rows_per_tile);
  bool loaded = !(v1 > g.n_p && g.n_p != a.max_pages);  // the first pass's rows are the right ones

  uint32_t* hist = STAB ? a.hist + (int64_t)s * a.max_pages : nullptr;
  float* stab = STAB && a.stab_out ? a.stab_out + (int64_t)s * a.max_pages : nullptr;

  for (int32_t v = v0 + grp; v < v1; v += NG * R) {
    int64_t row[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // a row past the tile is replaced by row 0 (loaded, never written back)
      const int32_t vr = v + NG * r;
      const bool ok = vr < v1;
      row[r] = !ok ? 0
               : vr < g.n_p ? vr
               : vr < g.n_p + g.n_c ? (int64_t)a.max_pages + (vr - g.n_p)
                                    : (int64_t)a.max_pages + a.c_cap + (vr - g.n_p - g.n_c);
      if (!loaded) load_row<LPR, NQ>(seq + row[r] * Q, lg, Q, x[r]);
    }
    loaded = false;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v_aff = row_affinity<LPR, NQ>(x[r], A);
      const int32_t vr = v + NG * r;
      if (lg == 0 && vr < v1) {
        if constexpr (STAB) g_aff[vr - v0] = v_aff;
        else aff[row[r]] = v_aff;
      }
    }
  }
  if constexpr (STAB) {
    __syncthreads();
    for (int32_t i = tid; i < v1 - v0; i += NT) {
      const int32_t vr = v0 + i;
      const int64_t row = vr < g.n_p ? vr
                          : vr < g.n_p + g.n_c ? (int64_t)a.max_pages + (vr - g.n_p)
                                               : (int64_t)a.max_pages + a.c_cap + (vr - g.n_p - g.n_c);
      if (aff) aff[row] = g_aff[i];
      if (vr < g.n_p) stability_step(a, hist[vr], g_aff[i], hist + vr, stab ? stab + vr : nullptr);
    }
  }
}

// Scoring pass of the two-launch path: 256-thread work-groups without LDS
// (more of them resident per compute unit), each scoring one tile; the
// kernel boundary publishes the affinities to the selection launch that
// follows.
template <int LPR, int NQ, int R, bool STAB>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  __shared__ float g_aff[STAB ? kPlainTileMax : 1];
  const int32_t s = blockIdx.x / a.tiles_per_seq;
  const int32_t tile = blockIdx.x - s * a.tiles_per_seq;
  if (threadIdx.x == 0 && tile == 0) seq_geom(a, s, true);  // reports a bad page count once
  score_tile<256, LPR, NQ, R, STAB>(a, s, tile, g_aff);
}

// Scoring tile, then selection: every work-group scores one tile of one
// sequence's rows; the work-group that finishes a sequence's last tile (a
// per-sequence counter, incremented once each tile's device-scope
// affinity stores have completed) selects that sequence.  Other sequences'
// tiles keep streaming meanwhile, and the selection needs no second launch.
template <int LPR, int NQ, int R, bool STAB, bool LEAN>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(NQ * R <= 8 && !LEAN ? 4 : 1)))
void score_select_kernel(ScoreArgs a) {
  __shared__ SelectShared sm;
  constexpr int NG = kSelThreads / LPR;  // row groups per work-group
  const int tid = threadIdx.x;
  const int32_t s = blockIdx.x / a.tiles_per_seq;
  const int32_t tile = blockIdx.x - s * a.tiles_per_seq;
  const int32_t v0 = tile * a.rows_per_tile;
  const int32_t Q = a.D >> 2;
  const f32x4* seq = reinterpret_cast<const f32x4*>(a.lvl + (int64_t)s * a.rows_per_seq * a.D);
  float* aff = a.aff + (int64_t)s * a.rows_per_seq;
  const int32_t grp = tid / LPR, lg = tid % LPR;
  SeqGeom g;
  int32_t v1;

  if constexpr (!STAB && LEAN) {
    // One pass covers the tile (rows_per_tile = NG * R).  Its rows are
    // requested together with the page count and the anchor: row v is
    // physical row v whenever v < n_p or the sequence fills its capacity
    // (every level full), the case of most tiles.  A tile whose guess the
    // page count proves wrong (it reaches past a ragged sequence's pages)
    // loads its rows again.  Loads go through a buffer resource over the
    // sequence's rows (fewer than 2^31 bytes on this path): a row past the
    // buffer reads zeros.
    const int32_t n_p_v = __hip_atomic_load(a.n_pages + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(seq, a.rows_per_seq * a.D * 4);
    const int32_t n_rows = (int32_t)a.rows_per_seq;
    AnchorRegs<LPR, NQ> A;
    issue_anchor<LPR, NQ>(a, s, lg, A);
    f32x4 x[R][NQ];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int32_t vr = v0 + grp + NG * r;
      load_row_buf<LPR, NQ>(rs, vr < n_rows ? vr : -1, lg, Q, x[r]);
    }
    __builtin_amdgcn_sched_barrier(0);
    finish_anchor<LPR, NQ>(A);
    g = geom_of(a, __builtin_amdgcn_readfirstlane(n_p_v), tid == 0 && tile == 0);
    const int32_t nv = g.n_p + g.n_c + g.n_g;
    v1 = min(nv, v0 + a.rows_per_tile);
    if (v0 < v1) {
      if (v1 > g.n_p && g.n_p != a.max_pages) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int32_t vr = v0 + grp + NG * r;
          const int32_t row = vr >= v1 ? -1
                              : vr < g.n_p ? vr
                              : vr < g.n_p + g.n_c ? a.max_pages + (vr - g.n_p)
                                                   : a.max_pages + a.c_cap + (vr - g.n_p - g.n_c);
          load_row_buf<LPR, NQ>(rs, row, lg, Q, x[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v_aff = row_affinity<LPR, NQ>(x[r], A);
        const int32_t vr = v0 + grp + NG * r;
        if (lg == 0 && vr < v1) sm.aff[vr - v0] = v_aff;
      }
    }
  } else {
    g = seq_geom(a, s, tid == 0 && tile == 0);
    const int32_t nv = g.n_p + g.n_c + g.n_g;
    v1 = min(nv, v0 + a.rows_per_tile);
    if (v0 < v1) {
      const AnchorRegs<LPR, NQ> A = load_anchor<LPR, NQ>(a, s, lg);
      uint32_t* hist = STAB ? a.hist + (int64_t)s * a.max_pages : nullptr;
      float* stab = STAB && a.stab_out ? a.stab_out + (int64_t)s * a.max_pages : nullptr;
      for (int32_t v = v0 + grp; v < v1; v += NG * R) {
        f32x4 x[R][NQ];
        int64_t row[R];
        uint32_t h[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          // a row past the tile is replaced by row 0 (loaded, never written back)
          const int32_t vr = v + NG * r;
          const bool ok = vr < v1;
          row[r] = !ok ? 0
                   : vr < g.n_p ? vr
                   : vr < g.n_p + g.n_c ? (int64_t)a.max_pages + (vr - g.n_p)
                                        : (int64_t)a.max_pages + a.c_cap + (vr - g.n_p - g.n_c);
          load_row<LPR, NQ>(seq + row[r] * Q, lg, Q, x[r]);
          // page rows also load their window word (others load word 0: max_pages >= 1 here)
          if constexpr (STAB) h[r] = hist[ok && vr < g.n_p ? vr : 0];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float v_aff = row_affinity<LPR, NQ>(x[r], A);
          const int32_t vr = v + NG * r;
          if (lg == 0 && vr < v1) {
            sm.aff[vr - v0] = v_aff;
            if constexpr (STAB) {
              if (vr < g.n_p) stability_step(a, h[r], v_aff, hist + vr, stab ? stab + vr : nullptr);
            }
          }
        }
      }
    }
  }
  // The tile's affinities leave in whole lines: consecutive rows of a level
  // are consecutive in memory, so consecutive lanes write consecutive words.
  __syncthreads();
  for (int32_t i = tid; i < v1 - v0; i += kSelThreads) {
    const int32_t vr = v0 + i;
    const int64_t row = vr < g.n_p ? vr
                        : vr < g.n_p + g.n_c ? (int64_t)a.max_pages + (vr - g.n_p)
                                             : (int64_t)a.max_pages + a.c_cap + (vr - g.n_p - g.n_c);
    store_agent(aff + row, sm.aff[i]);
  }
  // Every tile of the launch counts, scored or empty: the work-group that
  // completes the sequence's last tile selects it.
  if (!arrive(a.done + s, (uint32_t)a.tiles_per_seq, a.err, sm.last)) return;
  select_sequence<LEAN>(a, s, sm);
}

// Affinity v of element e of a level (lazy scoring) to LDS (STG) or to
// `aff`, and to `out` when it is set.
template <bool STG>
__device__ __forceinline__ void lazy_put(const Level& L, int32_t e, float v, float* aff, float* out, SelectShared& sm) {
  if constexpr (STG) sm.aff[L.off + e] = v;
  else store_agent(aff + L.off + e, v);
  if (out) out[L.off + e] = v;
}

// Lazy hierarchical scoring: one work-group per sequence scores the grids,
// selects, scores only the chunks of kept grids, selects, scores only the
// pages of kept chunks and selects (the page's coarse-to-fine order).  Rows
// under unkept parents are never read; their score is +0 by definition, so
// the selection equals the one over every row.  Scored affinities land in
// LDS when the sequence's rows fit (STG), else in `a.aff`; when `lazy_out`
// is set they are also written there (other rows untouched).  With EARLY,
// v0 holds the affinities of the first pass of rows of the first scored
// level (grids, or the pages of a flat layout), scored by the caller (the
// widest rows, 16 pieces per lane, keep the plain order: their registers
// are full).
template <bool STG, bool EARLY, int LPR, int NQ, int R>
__device__ __forceinline__ int32_t lazy_levels(const ScoreArgs& a, const SeqGeom& g, const f32x4* seq, float* aff,
                                               float* out, const AnchorRegs<LPR, NQ>& A, SelectShared& sm,
                                               const float (&v0)[R]) {
  constexpr int NG = kSelThreads / LPR;
  const int tid = threadIdx.x;
  const int32_t grp = tid / LPR, lg = tid % LPR;
  const int32_t Q = a.D >> 2;
  const int32_t lev0 = a.hier ? 0 : 2;
  Level L = make_level(a, g, lev0, aff, 0, sm);
  int32_t c_start = grp;
  if constexpr (EARLY) {
    // the first pass of the first level, from v0 (no parents: element = candidate)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int32_t c = grp + NG * r;
      if (lg == 0 && c < L.n) lazy_put<STG>(L, c, v0[r], aff, out, sm);
    }
    c_start += NG * R;
  }
  int32_t kp = 0;
  for (int32_t lev = lev0; lev < 3; ++lev) {
    if (lev != lev0) {
      L = make_level(a, g, lev, aff, kp, sm);
      c_start = grp;
    }
    const int32_t m = L.fanout ? L.n_par * L.fanout : L.n;
    for (int32_t c0 = c_start; c0 < m; c0 += NG * R) {
      f32x4 x[R][NQ];
      int32_t e[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int32_t c = c0 + NG * r;
        e[r] = c < m ? cand32(L, sm, c) : -1;
        // lanes past the candidates load row 0 (unconditional loads issue
        // back to back; exec-masked ones measured 15 % slower on a batch)
        load_row<LPR, NQ>(seq + (int64_t)(L.off + (e[r] >= 0 ? e[r] : 0)) * Q, lg, Q, x[r]);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v_aff = row_affinity<LPR, NQ>(x[r], A);
        if (lg == 0 && e[r] >= 0) lazy_put<STG>(L, e[r], v_aff, aff, out, sm);
      }
    }
    __syncthreads();
    kp = select_level<STG>(L, lev == 0 ? a.k_g : (lev == 1 ? a.k_c : a.k_p), sm,
                           lev == 0 ? sm.kept_grid : (lev == 1 ? sm.kept_chunk : nullptr));
  }
  return kp;
}

// One round of lazy scoring on the lean path: candidates c = grp + NG * r
// (r < P) of a level, element cand(c) (or -1), scored from their rows in
// the buffer `rs` into sm.aff[off + element].  Straight-line code: every
// lane issues the same P * NQ buffer loads (a lane without a candidate
// reads zeros, nothing from memory), all in flight before the first use.
// FIN: the anchor's pieces were only requested (issue_anchor); its norm is
// formed here, after the row loads have gone out.
template <int LPR, int NQ, int P, bool FIN, class Cand>
__device__ __forceinline__ void lean_round(__amdgpu_buffer_rsrc_t rs, int32_t Q, int32_t off,
                                           AnchorRegs<LPR, NQ>& A, Cand cand, float* dst) {
  constexpr int NG = kSelThreads / LPR;
  const int32_t grp = threadIdx.x / LPR, lg = threadIdx.x % LPR;
  f32x4 x[P][NQ];
  int32_t e[P];
#pragma unroll
  for (int r = 0; r < P; ++r) {
    e[r] = cand(grp + NG * r);
    load_row_buf<LPR, NQ>(rs, e[r] >= 0 ? off + e[r] : -1, lg, Q, x[r]);
  }
  if constexpr (FIN) {
    // kept after the row loads: the scheduler would otherwise start the
    // norm, and so wait for the anchor, before issuing them
    __builtin_amdgcn_sched_barrier(0);
    finish_anchor<LPR, NQ>(A);
  }
#pragma unroll
  for (int r = 0; r < P; ++r) {
    const float v = row_affinity<LPR, NQ>(x[r], A);
    if (lg == 0 && e[r] >= 0) dst[off + e[r]] = v;
  }
}

// Lazy scoring of the m (<= NG * R) candidates of one lean level: the round
// of the fewest passes, among 1, 2, 4, ... R, that covers them (the count
// is the work-group's, so the choice is uniform).  Each pass of loads costs
// its data return whether the lanes read rows or zeros, so passes without a
// candidate are not issued.
template <int LPR, int NQ, int R, bool FIN, class Cand>
__device__ __forceinline__ void lean_level_rows(int32_t m, __amdgpu_buffer_rsrc_t rs, int32_t Q, int32_t off,
                                                AnchorRegs<LPR, NQ>& A, Cand cand, float* dst) {
  constexpr int NG = kSelThreads / LPR;
  if (m <= NG) {
    lean_round<LPR, NQ, 1, FIN>(rs, Q, off, A, cand, dst);
    return;
  }
  if constexpr (R >= 2) {
    if (m <= 2 * NG) {
      lean_round<LPR, NQ, 2, FIN>(rs, Q, off, A, cand, dst);
      return;
    }
  }
  if constexpr (R >= 4) {
    if (m <= 4 * NG) {
      lean_round<LPR, NQ, 4, FIN>(rs, Q, off, A, cand, dst);
      return;
    }
  }
  if constexpr (R >= 8) {
    if (m <= 8 * NG) {
      lean_round<LPR, NQ, 8, FIN>(rs, Q, off, A, cand, dst);
      return;
    }
  }
  if constexpr (R >= 16) lean_round<LPR, NQ, R, FIN>(rs, Q, off, A, cand, dst);
}

// Lazy scoring of a lean layout (lean_levels_fit; NG * R >= 256): the
// grids' affinities are in sm.aff already (scored by the caller as soon as
// the anchor arrived); the chunks of the kept grids and then the pages of
// the kept chunks are scored in one round each into the LDS row copy,
// wavefront 0 ranks grids and chunks and four wavefronts the pages (as in
// select_lean_levels); the scored affinities go to `out` at the end.
// Returns the kept page count, or -1 when a level needs the zero fill
// (`out` is then left to the general path).
template <int LPR, int NQ, int R>
__device__ __forceinline__ int32_t lazy_lean_levels(const ScoreArgs& a, const SeqGeom& g, const f32x4* seq, float* out,
                                                    AnchorRegs<LPR, NQ>& A, SelectShared& sm) {
  constexpr int NG = kSelThreads / LPR;
  static_assert(NG * R >= 256, "one round of the row groups covers a lean level");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t Q = a.D >> 2;
  const int32_t kg = min(a.k_g, g.n_g), kc = min(a.k_c, g.n_c), kp = min(a.k_p, g.n_p);
  const int32_t off_g = a.max_pages + a.c_cap;
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(seq, a.rows_per_seq * a.D * 4);
  __syncthreads();
  if (wave == 0) {
    const int32_t eg = lane < g.n_g ? lane : -1;
    const bool good = rank_level64(eg, eg >= 0 ? __float_as_uint(sm.aff[off_g + eg]) : 0u, kg, g.n_g, sm.ck, sm.plist);
    if (lane == 0) sm.cnt[0] = good ? 1 : 0;
  }
  __syncthreads();
  if (sm.cnt[0] == 0) return -1;
  // chunks of the kept grids, then pages of the kept chunks
  for (int32_t lev = 1; lev < 3; ++lev) {
    const int32_t fan = lev == 1 ? a.cpg : a.ppc;
    const int32_t n_lev = lev == 1 ? g.n_c : g.n_p;
    const int32_t n_par = lev == 1 ? kg : kc;
    const int32_t* par = sm.plist + (lev == 1 ? 0 : 64);
    const int32_t off = lev == 1 ? a.max_pages : 0;
    const int32_t m = n_par * fan;
    auto child = [&](int32_t c) -> int32_t {
      if (c >= m) return -1;
      const int32_t pr = div_fan(c, fan);
      const int32_t el = par[pr] * fan + (c - pr * fan);
      return el < n_lev ? el : -1;
    };
    lean_level_rows<LPR, NQ, R, false>(m, rs, Q, off, A, child, sm.aff);
    __syncthreads();
    const int32_t ec = (tid < m && (lev == 2 || wave == 0)) ? child(tid) : -1;
    const uint32_t bits = ec >= 0 ? __float_as_uint(sm.aff[off + ec]) : 0u;
    if (lev == 1) {
      if (wave == 0) {
        const bool good = rank_level64(ec, bits, kc, m, sm.ck, sm.plist + 64);
        if (lane == 0) sm.cnt[0] = good ? 1 : 0;
      }
      __syncthreads();
      if (sm.cnt[0] == 0) return -1;
    } else if (!rank_level256(ec, bits, kp, sm)) {
      return -1;
    }
  }
  if (out) {
    // the scored affinities, stored once the selection is done: a store
    // issued between two rounds of row loads would hold up the wait for
    // the second round (memory operations complete in order)
    if (tid < g.n_g) out[off_g + tid] = sm.aff[off_g + tid];
    if (tid < kg * a.cpg) {
      const int32_t pr = div_fan(tid, a.cpg);
      const int32_t c = sm.plist[pr] * a.cpg + (tid - pr * a.cpg);
      if (c < g.n_c) out[a.max_pages + c] = sm.aff[a.max_pages + c];
    }
    if (tid < kc * a.ppc) {
      const int32_t pr = div_fan(tid, a.ppc);
      const int32_t p = sm.plist[64 + pr] * a.ppc + (tid - pr * a.ppc);
      if (p < g.n_p) out[p] = sm.aff[p];
    }
  }
  return kp;
}

// Work-group of the lazy pass's first sequence.  Group i runs on XCD i mod 8,
// and a lone latency-bound group measured slower on XCD 0 than on any other
// (one 128K sequence: 11.2-11.35 against 10.85-11.1 us on one device, 12.0
// against 11.35 on XCD 1 on another), so a batch of fewer than 8 sequences
// starts at group 1 and group 0 does nothing; larger batches spread from 0.
__host__ __device__ constexpr int32_t lazy_first_group(int32_t S) { return S < 8 ? 1 : 0; }

template <int LPR, int NQ, int R, bool LEAN>
__global__ __launch_bounds__(kSelThreads) void lazy_kernel(ScoreArgs a, float* lazy_out) {
  __shared__ SelectShared sm;
  constexpr int NG = kSelThreads / LPR;
  const int tid = threadIdx.x;
  const int32_t s = (int32_t)blockIdx.x - lazy_first_group(a.S);
  if (s < 0) return;
  const int32_t grp = tid / LPR, lg = tid % LPR;
  const int32_t Q = a.D >> 2;
  const f32x4* seq = reinterpret_cast<const f32x4*>(a.lvl + (int64_t)s * a.rows_per_seq * a.D);
  // The first scored level starts at a fixed row whatever the sequence's
  // length, so its first pass of rows is requested together with the page
  // count and the anchor, and scored as soon as they arrive; affinities of
  // rows past the level's end (known from the page count) are dropped.  The
  // count is read with a relaxed atomic load, which keeps its place before
  // the row loads (a plain load was issued where the count is first used,
  // after the round), and moved to a scalar register after the round; its
  // scope is the work-group's, so it may hit in the L2 (the counts are
  // written before the launch).
  const int32_t n_p_v = __hip_atomic_load(a.n_pages + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const int32_t off0 = a.hier ? a.max_pages + a.c_cap : 0;
  const int64_t cap0 = a.hier ? a.rows_per_seq - off0 : a.max_pages;
  // the general path scores the first pass of its first level early
  constexpr bool EARLY = !LEAN && NQ < 16;
  float v0[R] = {};
  AnchorRegs<LPR, NQ> A;
  if constexpr (LEAN) {
    // every grid row (at most 64 of them) in one round with the anchor,
    // straight into the LDS row copy
    issue_anchor<LPR, NQ>(a, s, lg, A);
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(seq, a.rows_per_seq * a.D * 4);
    lean_level_rows<LPR, NQ, R, true>((int32_t)cap0, rs, Q, off0, A,
                                      [&](int32_t c) -> int32_t { return c < cap0 ? c : -1; }, sm.aff);
  } else if constexpr (EARLY) {
    // Only the passes that reach the level's rows load (a count the whole
    // work-group shares), every lane of such a pass unconditionally: a lane
    // past the level reloads the level's first row (the anchor when the
    // level has no rows) and its score is dropped.  A per-lane load with
    // the other lanes' registers zeroed made each pass's loads wait for the
    // previous pass's.
    f32x4 x0[R][NQ] = {};
    const f32x4* base = cap0 > 0 ? seq + (int64_t)off0 * Q
                                 : reinterpret_cast<const f32x4*>(a.anchors + (int64_t)s * a.D);
    const int64_t lim = cap0 > 0 ? cap0 : 1;
    const int32_t passes = (int32_t)min<int64_t>(R, (lim + NG - 1) / NG);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int32_t c = grp + NG * r;
      if (r < passes) load_row<LPR, NQ>(base + (int64_t)(c < lim ? c : 0) * Q, lg, Q, x0[r]);
    }
    A = load_anchor<LPR, NQ>(a, s, lg);
#pragma unroll
    for (int r = 0; r < R; ++r) v0[r] = r < passes ? row_affinity<LPR, NQ>(x0[r], A) : 0.f;
  } else {
    A = load_anchor<LPR, NQ>(a, s, lg);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int32_t n_p = __builtin_amdgcn_readfirstlane(n_p_v);
  const SeqGeom g = geom_of(a, n_p, tid == 0);
  float* aff = a.aff + (int64_t)s * a.rows_per_seq;
  float* out = lazy_out ? lazy_out + (int64_t)s * a.rows_per_seq : nullptr;
  int32_t kp = -1;
  if constexpr (LEAN) kp = lazy_lean_levels<LPR, NQ, R>(a, g, seq, out, A, sm);
  if (kp < 0) {
    // the general path (also when a lean level needs the zero fill)
    clear_select_state(a, g, sm);
    __syncthreads();
    kp = a.rows_per_seq <= kLdsRows ? lazy_levels<true, EARLY, LPR, NQ, R>(a, g, seq, aff, out, A, sm, v0)
                                    : lazy_levels<false, EARLY, LPR, NQ, R>(a, g, seq, aff, out, A, sm, v0);
  }
  write_selection(a, sm, s, kp);
}

// ------------------------------------------- small coarse-to-fine selection
//
// For batches too large for the one-launch handoff (more tiles than fit on
// the chip at once) whose levels are small (a few hundred candidates per
// level, k up to a few hundred: the serving workload), one work-group per
// sequence selects on its own beside the scoring tiles: it scores every
// grid, keeps the top k_grid, scores the chunks of the kept grids, keeps the
// top k_chunk, scores the pages of the kept chunks and keeps the top k_page
// (section 5.1's order), with the same row code as the scoring tiles, so the
// affinities it selects on are bit for bit the ones the tiles write.  Rows
// under unkept parents score +0 by definition and are never read; the
// selection equals the one over every row.  Nothing passes between
// work-groups, and the selecting groups' latency hides behind the stream of
// the batch's rows.

// Candidates per level, and kept elements per level, that the small
// selector holds (the host sends larger geometries to the two-launch path).
constexpr int kSmallCand = kSmallSelect;

struct SmallSel {
  alignas(16) uint64_t key[kSmallCand];  // candidate keys (0: the candidate scores 0, or is absent)
  alignas(16) uint64_t res[kSmallCand];  // kept keys in rank order
  int32_t kept[kSmallCand];              // kept elements of the level above, in rank order
  int32_t zero_e[kSmallCand];            // live candidates scoring exactly 0
  uint32_t pbits[kBitmapWords];          // keep flags of the level above's elements
  float g_aff[kPlainTileMax];            // scoring tiles: a tile's affinities (stability filter)
  int32_t n_zero;
  int32_t wcnt[16];                      // per-wave counts (up to 1024 threads)
};

// Value of lane (lane ^ J) of one 32-bit register of the wavefront: DPP quad
// permutes for J = 1, 2, swizzles (xor within 32 lanes) for J = 4 .. 16, a
// permute through LDS for J = 32.
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  if constexpr (J == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  else if constexpr (J == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  else if constexpr (J < 32) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (J << 10) | 0x1F);
  else return (uint32_t)__builtin_amdgcn_ds_bpermute((int)((((int)threadIdx.x & 63) ^ J) << 2), (int)v);
}

// One compare-exchange step of a bitonic network over the lanes: blocks of
// SIZE lanes alternate direction (the block of 64 is descending), partners J
// lanes apart.
template <int SIZE, int J>
__device__ __forceinline__ uint64_t bitonic_step(uint64_t x) {
  const int lane = threadIdx.x & 63;
  const uint32_t lo = xor_lane<J>((uint32_t)x);
  const uint32_t hi = xor_lane<J>((uint32_t)(x >> 32));
  const uint64_t y = ((uint64_t)hi << 32) | lo;
  const bool desc = (lane & SIZE) == 0 || SIZE == 64;
  const bool lower = (lane & J) == 0;
  return (lower == desc) ? (x > y ? x : y) : (x < y ? x : y);
}

template <int SIZE, int J>
__device__ __forceinline__ uint64_t bitonic_merge(uint64_t x) {
  x = bitonic_step<SIZE, J>(x);
  if constexpr (J > 1) x = bitonic_merge<SIZE, J / 2>(x);
  return x;
}

template <int SIZE>
__device__ __forceinline__ uint64_t bitonic_sort(uint64_t x) {
  if constexpr (SIZE > 2) x = bitonic_sort<SIZE / 2>(x);
  return bitonic_merge<SIZE, SIZE / 2>(x);
}

// Sorts one key per lane of a wavefront into descending order (lane j ends
// up with the j-th largest).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x) { return bitonic_sort<64>(x); }

// Keys greater than x in a descending run of 64 keys: binary search for the
// first key <= x over the 65 possible answers 0..64 (seven halvings).
__device__ __forceinline__ int32_t count_above(const uint64_t* run, uint64_t x) {
  int32_t lo = 0, hi = 64;
#pragma unroll
  for (int it = 0; it < 7; ++it) {
    if (lo < hi) {
      const int32_t mid = (lo + hi) >> 1;  // < 64 while lo < hi <= 64
      if (run[mid] > x) lo = mid + 1;
      else hi = mid;
    }
  }
  return lo;
}

// Ranks the m candidate keys sm.key[0, m) (m <= kSmallCand; non-zero keys
// are distinct, 0 marks a candidate scoring 0 or a slot past the
// candidates): the key with r larger keys goes to sm.res[r] when r <
// k_eff.  Wavefront w sorts keys [64w, 64w + 64) in registers; with more
// than one run, the sorted runs go to LDS and each key's rank is its place
// in its own run plus the keys above it in every other run.  Returns the
// number of non-zero (positive-score) keys.
template <int NT>
__device__ int32_t small_rank(SmallSel& sm, int32_t m, int32_t k_eff) {
  static_assert(NT / 64 >= kSmallCand / 64, "one wavefront per run of 64 candidates");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t n_runs = (m + 63) >> 6;
  uint64_t x = 0ull;
  if (wave < n_runs) {  // whole wavefronts
    const int32_t c = 64 * wave + lane;
    x = wave_sort_desc(c < m ? sm.key[c] : 0ull);
    const uint64_t bal = __ballot(x != 0ull);
    if (lane == 0) sm.wcnt[wave] = (int32_t)__popcll(bal);
  }
  if (n_runs > 1) {
    __syncthreads();  // every run has read its keys: overwrite with the sorted runs
    if (wave < n_runs) sm.key[64 * wave + lane] = x;
  }
  __syncthreads();
  int32_t P = 0;
  for (int32_t w = 0; w < n_runs; ++w) P += sm.wcnt[w];
  if (wave < n_runs && x != 0ull) {
    int32_t r = lane;
    for (int32_t v = 0; v < n_runs; ++v)
      if (v != wave) r += count_above(sm.key + 64 * v, x);
    if (r < k_eff) sm.res[r] = x;
  }
  __syncthreads();
  return P;
}

// When only P < k_eff candidates score above 0, slots P .. k_eff-1 take the
// lowest-index elements of the level scoring exactly 0: children of unkept
// parents (fan > 0 and their parent's bit clear in sm.pbits) and live
// candidates of zero affinity (sm.zero_e), in index order.
template <int NT>
__device__ void small_fill_zeros(SmallSel& sm, int32_t n_lev, int32_t fan, int32_t P, int32_t k_eff) {
  constexpr int W = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const int32_t need = k_eff - P;
  const int32_t nz = sm.n_zero;
  int32_t found = 0;
  for (int32_t e0 = 0; e0 < n_lev && found < need; e0 += NT) {
    const int32_t e = e0 + tid;
    bool zero = false;
    if (e < n_lev) {
      const int32_t par = fan > 0 ? e / fan : 0;
      if (fan > 0 && !((sm.pbits[par >> 5] >> (par & 31)) & 1u)) {
        zero = true;
      } else {
        for (int32_t z = 0; z < nz && !zero; ++z) zero = sm.zero_e[z] == e;
      }
    }
    const uint64_t bal = __ballot(zero);
    if (lane == 0) sm.wcnt[wave] = (int32_t)__popcll(bal);
    __syncthreads();
    int32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      if (w < wave) before += sm.wcnt[w];
      tot += sm.wcnt[w];
    }
    const int32_t rank = found + before + (int32_t)__popcll(bal & lt_mask);
    if (zero && rank < need) sm.res[P + rank] = composite(0u, e);
    found += tot;
    __syncthreads();
  }
}

// Selection of sequence s by one work-group of NT threads (see above).  The
// first scored level's rows sit at a fixed place, so its first pass of
// loads goes out with the page count and the anchor.  RS rows per row group
// are in flight per pass.
template <int NT, int LPR, int NQ, int RS>
__device__ void small_select(const ScoreArgs& a, int32_t s, SmallSel& sm) {
  constexpr int NG = NT / LPR;
  const int tid = threadIdx.x;
  const int32_t grp = tid / LPR, lg = tid % LPR;
  const int32_t Q = a.D >> 2;
  const f32x4* seq = reinterpret_cast<const f32x4*>(a.lvl + (int64_t)s * a.rows_per_seq * a.D);
  // The first level's rows (every grid, or every page of a flat layout) sit
  // at a fixed place whatever the sequence's length: its first pass of row
  // loads goes out with the page count and the anchor, and rows past the
  // level's end (known once the page count arrives) are dropped.
  const int32_t lev0 = a.hier ? 0 : 2;
  const int32_t off0 = a.hier ? a.max_pages + a.c_cap : 0;
  const int32_t cap0 = a.hier ? a.g_cap : a.max_pages;  // rows the first level can hold
  float v0[RS];
  f32x4 x0[RS][NQ];
  {
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      const int32_t c = grp + NG * r;
      if (cap0 > 0) {
        load_row<LPR, NQ>(seq + (int64_t)(off0 + (c < cap0 ? c : cap0 - 1)) * Q, lg, Q, x0[r]);
      } else {
#pragma unroll
        for (int j = 0; j < NQ; ++j) x0[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  const SeqGeom g = seq_geom(a, s, tid == 0);
  const AnchorRegs<LPR, NQ> A = load_anchor<LPR, NQ>(a, s, lg);
#pragma unroll
  for (int r = 0; r < RS; ++r) v0[r] = row_affinity<LPR, NQ>(x0[r], A);
  int32_t n_par = 0;  // kept elements of the level above
  for (int32_t lev = lev0; lev < 3; ++lev) {
    int32_t n_lev, fan, off;  // elements, children per parent (0: every element a candidate), first row
    if (lev == 0) {
      n_lev = g.n_g;
      fan = 0;
      off = a.max_pages + a.c_cap;
    } else if (lev == 1) {
      n_lev = g.n_c;
      fan = a.cpg;
      off = a.max_pages;
    } else {
      n_lev = g.n_p;
      fan = a.hier ? a.ppc : 0;
      off = 0;
    }
    const int32_t m = min(fan ? n_par * fan : n_lev, kSmallCand);
    if (tid == 0) sm.n_zero = 0;
    __syncthreads();  // n_zero, the kept list and keep flags of the level above
    int32_t c_start = grp;
    if (lev == lev0) {
      // the first pass, scored above (no parents: candidate = element)
#pragma unroll
      for (int r = 0; r < RS; ++r) {
        const int32_t c = grp + NG * r;
        if (lg == 0 && c < m) {
          const uint32_t bits = __float_as_uint(v0[r]);
          sm.key[c] = bits != 0u ? composite(bits, c) : 0ull;
          if (bits == 0u) sm.zero_e[atomicAdd(&sm.n_zero, 1)] = c;
        }
      }
      c_start += NG * RS;
    }
    for (int32_t c0 = c_start; c0 < m; c0 += NG * RS) {
      f32x4 x[RS][NQ];
      int32_t e[RS];
#pragma unroll
      for (int r = 0; r < RS; ++r) {
        const int32_t c = c0 + NG * r;
        int32_t el = -1;
        if (c < m) {
          el = fan ? sm.kept[c / fan] * fan + (c - (c / fan) * fan) : c;
          if (el >= n_lev) el = -1;  // past the end of a ragged last parent
        }
        e[r] = el;
        // candidates past the end load row `off` (unconditional loads issue back to back)
        load_row<LPR, NQ>(seq + (int64_t)(off + (el >= 0 ? el : 0)) * Q, lg, Q, x[r]);
      }
#pragma unroll
      for (int r = 0; r < RS; ++r) {
        const float v = row_affinity<LPR, NQ>(x[r], A);
        const int32_t c = c0 + NG * r;
        if (lg == 0 && c < m) {
          const uint32_t bits = __float_as_uint(v);
          sm.key[c] = (e[r] >= 0 && bits != 0u) ? composite(bits, e[r]) : 0ull;
          if (e[r] >= 0 && bits == 0u) sm.zero_e[atomicAdd(&sm.n_zero, 1)] = e[r];
        }
      }
    }
    __syncthreads();
    const int32_t k = lev == 0 ? a.k_g : (lev == 1 ? a.k_c : a.k_p);
    const int32_t k_eff = min(min(k, n_lev), kSmallCand);
    const int32_t P = k_eff > 0 ? small_rank<NT>(sm, m, k_eff) : 0;
    if (P < k_eff) small_fill_zeros<NT>(sm, n_lev, fan, P, k_eff);
    __syncthreads();
    if (lev < 2) {
      // the kept elements become the next level's parents
      for (int32_t w = tid; w < (n_lev + 31) / 32 && w < kBitmapWords; w += NT) sm.pbits[w] = 0u;
      __syncthreads();
      for (int32_t i = tid; i < k_eff; i += NT) {
        const int32_t el = (int32_t)(~(uint32_t)sm.res[i]);
        sm.kept[i] = el;
        atomicOr(&sm.pbits[el >> 5], 1u << (el & 31));
      }
    }
    n_par = k_eff;
  }
  __syncthreads();
  for (int32_t i = tid; i < a.k_p; i += NT) {
    int32_t idx = -1;
    float sc = 0.f;
    if (i < n_par) {
      const uint64_t c = sm.res[i];
      idx = (int32_t)(~(uint32_t)c);
      sc = __uint_as_float((uint32_t)(c >> 32));
    }
    a.idx_out[(int64_t)s * a.k_p + i] = idx;
    if (a.score_out) a.score_out[(int64_t)s * a.k_p + i] = sc;
  }
  if (tid == 0 && a.cnt_out) a.cnt_out[s] = n_par;
}

// One launch of scoring and selection: work-groups 0 .. S-1 select (one per
// sequence, small_select); the others, when a.tiles_per_seq > 0, score
// tile (blockIdx - S) % tiles_per_seq of sequence (blockIdx - S) /
// tiles_per_seq for affinity_out and the stability filter.  No work-group
// reads what another writes.
template <int NT, int LPR, int NQ, int RS, int RT, bool STAB>
__global__ __launch_bounds__(NT) void score_topk_kernel(ScoreArgs a) {
  __shared__ SmallSel sm;
  const int32_t b = blockIdx.x;
  if (b < a.S) {
    small_select<NT, LPR, NQ, RS>(a, b, sm);
    return;
  }
  const int32_t t = b - a.S;
  const int32_t s = t / a.tiles_per_seq;
  score_tile<NT, LPR, NQ, RT, STAB>(a, s, t - s * a.tiles_per_seq, sm.g_aff);
}

// Lanes sharing one row: 8 (whole 128-byte lines per row group), 16 above
// head_dim 512 so that a lane's row and anchor pieces stay in registers.
constexpr int32_t score_lpr(int32_t D) { return D / 4 > 8 * 16 ? 16 : 8; }


// Shape of the one-launch path for large batches, where the scoring tiles'
// stream is the call's time and the selecting groups run beside it: 256
// threads per group and score_kernel's loads (4 float4 per lane per pass,
// two passes per tile), so the kernel stays near score_kernel's register
// count and residency; the selecting groups read RS rows per row group per
// pass.
template <int LPR, int NQ>
struct FusedShape {
  static constexpr int NT = 256;
  static constexpr int RS = NQ >= KKA_SCORE_LOADS ? 1 : KKA_SCORE_LOADS / NQ;
  static constexpr int RT = RS;
  static constexpr int PT = KKA_SCORE_PASSES;
  static constexpr int32_t kTileRows = (NT / LPR) * RT * PT;
  static_assert(kTileRows <= kPlainTileMax, "tile rows exceed the gather buffer");
};

template <int LPR, int NQ>
hipError_t launch_small(const ScoreArgs& a0, hipStream_t st) {
  using F = FusedShape<LPR, NQ>;
  ScoreArgs a = a0;
  // without affinity_out and the stability filter there is nothing to score
  // for: the selecting groups alone
  const bool streams = a0.aff != nullptr || a0.hist != nullptr;
  int64_t tiles = 0;
  if (streams) {
    a.rows_per_tile = F::kTileRows;
    tiles = (a.rows_per_seq + a.rows_per_tile - 1) / a.rows_per_tile;
    a.tiles_per_seq = (int32_t)(tiles > 0 ? tiles : 1);
    tiles = a.tiles_per_seq;
  }
  const dim3 grid((unsigned)((int64_t)a.S * (1 + tiles)));
  if (a.hist)
    hipLaunchKernelGGL((score_topk_kernel<F::NT, LPR, NQ, F::RS, F::RT, true>), grid, dim3(F::NT), 0, st, a);
  else
    hipLaunchKernelGGL((score_topk_kernel<F::NT, LPR, NQ, F::RS, F::RT, false>), grid, dim3(F::NT), 0, st, a);
  return hipGetLastError();
}

template <int LPR, int NQ>
hipError_t launch_nq(const ScoreArgs& a0, bool lazy, float* lazy_out, hipStream_t st) {
  constexpr int R = NQ >= KKA_SCORE_LOADS ? 1 : KKA_SCORE_LOADS / NQ;
  if (lazy) {
    constexpr int RL = NQ >= 16 ? 1 : 16 / NQ;  // 16 row loads in flight per lane
    constexpr bool kLeanOk = NQ < 16 && (kSelThreads / LPR) * RL >= 256;  // early grid rows, one pass a level
    const dim3 grid((unsigned)(a0.S + lazy_first_group(a0.S)));
    if (kLeanOk && lean_levels_fit(a0))
      hipLaunchKernelGGL((lazy_kernel<LPR, NQ, RL, kLeanOk>), grid, dim3(kSelThreads), 0, st, a0, lazy_out);
    else
      hipLaunchKernelGGL((lazy_kernel<LPR, NQ, RL, false>), grid, dim3(kSelThreads), 0, st, a0, lazy_out);
    return hipGetLastError();
  }
  ScoreArgs a = a0;
  // Latency-bound batches (one wave of 512-thread work-groups, two per
  // compute unit, covers every tile) score and select in one launch, the
  // selection handed to the work-group that finishes a sequence's last tile.
  // All of a lane's row loads go out in one pass over its tile.
  constexpr int RF = NQ >= KKA_SCORE_LOADS * KKA_SCORE_PASSES ? 1 : KKA_SCORE_LOADS * KKA_SCORE_PASSES / NQ;
  constexpr int32_t kFusedRows = (kSelThreads / LPR) * RF;
  const int64_t fused_tiles = (a.rows_per_seq + kFusedRows - 1) / kFusedRows;
  if (a.done && (int64_t)a.S * fused_tiles <= 2 * (int64_t)device_cus()) {
    a.rows_per_tile = kFusedRows;
    a.tiles_per_seq = (int32_t)(fused_tiles > 0 ? fused_tiles : 1);
    const dim3 grid((unsigned)((int64_t)a.S * a.tiles_per_seq));
    // the lean selection (more registers: one work-group per compute unit)
    // when one work-group per compute unit covers every tile
    const bool lean = lean_levels_fit(a) && (int64_t)a.S * fused_tiles <= (int64_t)device_cus();
    if (a.hist && lean)
      hipLaunchKernelGGL((score_select_kernel<LPR, NQ, RF, true, true>), grid, dim3(kSelThreads), 0, st, a);
    else if (a.hist)
      hipLaunchKernelGGL((score_select_kernel<LPR, NQ, RF, true, false>), grid, dim3(kSelThreads), 0, st, a);
    else if (lean)
      hipLaunchKernelGGL((score_select_kernel<LPR, NQ, RF, false, true>), grid, dim3(kSelThreads), 0, st, a);
    else
      hipLaunchKernelGGL((score_select_kernel<LPR, NQ, RF, false, false>), grid, dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
  }
  // Larger batches whose levels fit the small selector: one launch, a
  // selecting group per sequence beside the scoring tiles (its latency hides
  // behind the stream of the batch's rows).
  if (a.small) return launch_small<LPR, NQ>(a, st);
  // Otherwise two launches: the scoring pass, then one selecting work-group
  // per sequence (the kernel boundary orders the affinities between them).
  constexpr int32_t kPlainRows = (256 / LPR) * R * KKA_SCORE_PASSES;
  static_assert(kPlainRows <= kPlainTileMax, "a score_kernel tile has at most one row per thread");
  const int64_t tiles = (a.rows_per_seq + kPlainRows - 1) / kPlainRows;
  a.rows_per_tile = kPlainRows;
  a.tiles_per_seq = (int32_t)(tiles > 0 ? tiles : 1);
  const dim3 grid((unsigned)((int64_t)a.S * a.tiles_per_seq));
  if (a.hist)
    hipLaunchKernelGGL((score_kernel<LPR, NQ, R, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((score_kernel<LPR, NQ, R, false>), grid, dim3(256), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (lean_levels_fit(a))
    hipLaunchKernelGGL(select_kernel<true>, dim3((unsigned)a.S), dim3(kSelThreads), 0, st, a);
  else
    hipLaunchKernelGGL(select_kernel<false>, dim3((unsigned)a.S), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t dispatch(const ScoreArgs& a, bool lazy, float* lazy_out, hipStream_t st) {
  if (a.S <= 0) return hipSuccess;
  if (score_lpr(a.D) == 16) return launch_nq<16, 16>(a, lazy, lazy_out, st);  // head_dim 516..1024
  const int32_t nq = (a.D / 4 + 7) / 8;
  if (nq <= 1) return launch_nq<8, 1>(a, lazy, lazy_out, st);
  if (nq <= 2) return launch_nq<8, 2>(a, lazy, lazy_out, st);
  if (nq <= 4) return launch_nq<8, 4>(a, lazy, lazy_out, st);
  if (nq <= 8) return launch_nq<8, 8>(a, lazy, lazy_out, st);
  return launch_nq<8, 16>(a, lazy, lazy_out, st);
}

}  // namespace

// Compute units of the current device (cached per device; callers on
// several host threads may fill an entry at once with the same value).
int32_t device_cus() {
  static std::atomic<int32_t> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int32_t n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    int q = 0;
    if (hipDeviceGetAttribute(&q, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || q <= 0) q = 256;
    n = q;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Rows the smaller (256-thread) scoring work-group covers for a given
// head_dim: the launch sizes its tiles from this or twice this.
int32_t score_rows_per_tile(int32_t D) {
  const int32_t lpr = score_lpr(D);
  const int32_t nq = (D / 4 + lpr - 1) / lpr;
  int32_t NQ = 1;
  while (NQ < nq) NQ <<= 1;
  const int32_t R = NQ >= KKA_SCORE_LOADS ? 1 : KKA_SCORE_LOADS / NQ;
  return (256 / lpr) * R * KKA_SCORE_PASSES;
}

// A fused tile's affinities are gathered in the selection's LDS row buffer.
static_assert((kSelThreads / 8) * KKA_SCORE_LOADS * KKA_SCORE_PASSES <= kLdsRows, "tile rows exceed LDS");

hipError_t launch_score_topk(const ScoreArgs& a, hipStream_t st) { return dispatch(a, false, nullptr, st); }

hipError_t launch_select(const ScoreArgs& a, hipStream_t st) {
  if (a.S <= 0) return hipSuccess;
  if (lean_levels_fit(a))
    hipLaunchKernelGGL(select_kernel<true>, dim3((unsigned)a.S), dim3(kSelThreads), 0, st, a);
  else
    hipLaunchKernelGGL(select_kernel<false>, dim3((unsigned)a.S), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_score_topk_lazy(const ScoreArgs& a, float* lazy_out, hipStream_t st) {
  return dispatch(a, true, lazy_out, st);
}

}  // namespace kka
