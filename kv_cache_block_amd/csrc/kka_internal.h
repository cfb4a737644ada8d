// Internal declarations shared by the libkka translation units: launch
// argument blocks, small device helpers and the launchers each kernel file
// provides to the C-ABI layer (kka_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kka.h"

namespace kka {

// Largest block size any pool kernel is launched with (one thread per 16-byte
// chunk of a token's H*D key row, H*D/8 <= 1024).
constexpr int kMaxPoolThreads = 1024;
// Target work-groups for one pooling launch (blocks are split over layers
// until there are about this many groups).
#ifndef KKA_POOL_TARGET_GROUPS
#define KKA_POOL_TARGET_GROUPS 2048
#endif
constexpr int kPoolTargetGroups = KKA_POOL_TARGET_GROUPS;
// Largest k at any selection level.
constexpr int kMaxK = 1024;
// Largest number of parents whose keep flags one selecting group tracks.
constexpr int kMaxParents = 16384;
// Largest chunks_per_grid * head_dim (LDS of the level builder, floats).
constexpr int kMaxGridFloats = 16384;
// Largest page count of one sequence (also rounded up to whole chunks).
constexpr int64_t kMaxPagesPerSeq = (int64_t)1 << 30;
// Affinity rows of one sequence a selecting work-group keeps in LDS.
constexpr int kSelectLdsRows = 9216;
// Candidates, and kept elements, per level that the one-launch selector
// holds (small_select_fits).
constexpr int kSmallSelect = 256;

// True when a selection fits the one-launch path: a hierarchical layout
// whose levels never offer more than kSmallSelect candidates (every grid;
// the chunks of at most k_grid kept grids; the pages of at most k_chunk
// kept chunks) or a flat one of at most kSmallSelect pages, and k at most
// kSmallSelect at every level.  c_cap, g_cap: chunk and grid rows of the
// layout; the counts of any sequence are at most these.
inline bool small_select_fits(bool hier, int64_t max_pages, int64_t c_cap, int64_t g_cap, int64_t ppc, int64_t cpg,
                              int64_t k_g, int64_t k_c, int64_t k_p) {
  if (k_p > kSmallSelect) return false;
  if (!hier) return max_pages <= kSmallSelect;
  if (k_g > kSmallSelect || k_c > kSmallSelect) return false;
  const int64_t kg = k_g < g_cap ? k_g : g_cap, kc = k_c < c_cap ? k_c : c_cap;
  return g_cap <= kSmallSelect && kg * cpg <= kSmallSelect && kc * ppc <= kSmallSelect;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Thread layout of the pooling kernels: a token's H*D key row is cut into
// H*D/8 chunks of 16 bytes; `rg` consecutive threads cover one row and `m`
// rows (tokens) are in flight per pass, nt = rg * m threads per group.
struct PoolShape {
  int32_t rg, m, nt;
};

inline PoolShape pool_shape(int32_t H, int32_t D) {
  PoolShape ps;
  ps.rg = H * (D / 8);
  ps.m = ps.rg >= 256 ? 1 : 256 / ps.rg;
  ps.nt = ps.rg * ps.m;
  return ps;
}

// Layer split of a pooling launch: enough groups to fill the chip, never a
// split finer than one layer (nor, with layer_bytes, shares smaller than
// kMinShareBytes).  Depends only on its arguments.
struct LayerSplit {
  int32_t n_split, lps;
};

// A layer-split launch of at most one work-group per compute unit that
// reads at most this many key bytes (pure latency: one sequence's anchor)
// combines its shares in the same launch through per-item arrival counters;
// others leave them to a second kernel.  The wait for the shares' write-
// through stores to be acknowledged and the last work-group's loads past
// the L2 cost more than the second launch once many work-groups take part
// (anchors of 32 sequences, 896 work-groups: 19.2 against 17.1 us; 7B
// K-pool of 32K tokens under a saturating read stream: 157 against 150 us)
// and less for one sequence's anchor (28 work-groups: 12.2 against 14.4).
constexpr double kSplitOneLaunchBytes = 32.0 * 1024 * 1024;

int32_t device_cus();  // compute units of the current device (cached; defined with the scoring launchers)

// KKA_NO_HANDOFF=1 in the environment: no launch hands values from one
// work-group to another (layer-split shares are added by a second kernel,
// small scoring batches select in a second launch); results are the same.
bool handoff_disabled();  // defined with the C-ABI layer

inline bool split_in_one_launch(int64_t items, int32_t n_split, double key_bytes) {
  return n_split > 1 && items * n_split <= device_cus() && key_bytes <= kSplitOneLaunchBytes && !handoff_disabled();
}

// Pooling splits a block's layers into shares of at least this many key
// bytes (layer_bytes: one layer of one item): a smaller share is dominated
// by its work-group's fixed costs (0.5B shape, blocks of 98 KB kept whole:
// 256 work-groups and no combine, 17.1 -> 13.1 us).  Anchors pass 0: their
// work-groups walk tokens and layers serially, and fewer, larger shares
// measured slower (one 32K sequence: 12.2 -> 21.0 us at this minimum).
constexpr int64_t kMinShareBytes = 128 * 1024;

inline LayerSplit layer_split(int64_t items, int32_t L, int64_t layer_bytes = 0) {
  LayerSplit ls;
  int64_t want = items >= kPoolTargetGroups ? 1 : (kPoolTargetGroups + items - 1) / (items > 0 ? items : 1);
  if (want > L) want = L;
  if (want < 1) want = 1;
  int64_t lps = (L + want - 1) / want;
  if (layer_bytes > 0) {
    const int64_t min_lps = (kMinShareBytes + layer_bytes - 1) / layer_bytes;
    if (lps < min_lps) lps = min_lps < L ? min_lps : L;
  }
  ls.lps = (int32_t)lps;
  ls.n_split = (int32_t)((L + lps - 1) / lps);
  return ls;
}

// Layer split of an anchor launch.  Anchors read a few tokens per sequence
// and are latency-bound: where the split above needs more work-groups than
// kAnchorFitGroups but shares of at most kAnchorFitLayers layers stay within
// it, those shares are taken instead, so that on a chip with that many
// compute units the shares are added in the same launch (32 sequences of the
// 7B shape: 7 shares of 4 layers, 224 work-groups, 14.2 us, against 28
// shares of one layer and a second kernel, 15.4 us).  Depends only on its
// arguments.
constexpr int64_t kAnchorFitGroups = 256;
constexpr int32_t kAnchorFitLayers = 4;

inline LayerSplit anchor_split(int64_t S, int32_t L) {
  LayerSplit ls = layer_split(S, L);
  if (S > 0 && S * ls.n_split > kAnchorFitGroups) {
    const int64_t shares = kAnchorFitGroups / S;
    if (shares >= 1) {
      const int64_t lps = (L + shares - 1) / shares;
      if (lps <= kAnchorFitLayers && lps > ls.lps) {
        ls.lps = (int32_t)lps;
        ls.n_split = (int32_t)((L + lps - 1) / lps);
      }
    }
  }
  return ls;
}

// Per-XCD shares of a pooling launch with one work-group per item.  The
// dispatcher hands work-group i to XCD i mod 8, and under the K-pool's read
// stream the XCDs do not stream equally fast (MI355X: every work-group on an
// odd-numbered XCD took about 8 % longer than on an even-numbered one, in
// every call on every device measured), so with equal counts the launch ends
// when the slowest XCDs do.  With shares, XCD x pools the contiguous items
// off[x] .. off[x] + n[x] - 1, n proportional to a weight per XCD, and
// work-group 8 r + x takes item off[x] + r (none when r >= n[x]): every item
// is pooled once, by the same arithmetic, whatever XCD it lands on.
constexpr int kXcds = 8;
constexpr int64_t kXcdShareMinItems = 2048;  // several dispatch rounds; smaller launches keep one item per group

struct XcdShares {
  int32_t on;
  int32_t n[kXcds], off[kXcds];
};

// Weights of the XCD shares for this process: KKA_XCD_WEIGHTS in the
// environment ("w0,...,w7", eight positive numbers; "off" for one item per
// work-group), else 1.1 for even-numbered and 1.0 for odd-numbered XCDs on a
// 256-compute-unit device (MI355X) and none elsewhere.  False: no shares.
bool xcd_weights(double (&w)[kXcds]);

// Shares of n_items items by weight w: floor of each XCD's part, the rest one
// item at a time from XCD 0 up.  Depends only on its arguments.
inline XcdShares xcd_shares(int64_t n_items, const double (&w)[kXcds]) {
  XcdShares xs = {};
  double tot = 0.0;
  for (int x = 0; x < kXcds; ++x) tot += w[x];
  int64_t given = 0;
  for (int x = 0; x < kXcds; ++x) {
    xs.n[x] = (int32_t)((double)n_items * w[x] / tot);
    given += xs.n[x];
  }
  for (int x = 0; given < n_items; x = (x + 1) % kXcds, ++given) ++xs.n[x];
  for (int x = 0, o = 0; x < kXcds; o += xs.n[x], ++x) xs.off[x] = o;
  xs.on = 1;
  return xs;
}

struct PoolArgs {
  const uint16_t* k;
  int64_t sL, sB, sT, sH;
  int32_t L, H, D, B;
  int64_t P;
  int32_t S, total_blocks;
  const int32_t* seq_len;
  const int32_t* offs;
  const int32_t* table;
  const int32_t* subset;  // global logical block per item, or null (item == block)
  int32_t n_items;
  int32_t n_split, lps;
  const float* weights;   // [S][L*H] (given-weight pooling and the anchor)
  float* out;             // v_b rows / anchor rows
  int64_t vb_stride;      // rows per sequence in `out`, 0 = row is the global block id
  float* partial;         // layer-split partial sums, or per-(l,h) token sums
  uint32_t* done;         // per-item arrival counters of a layer split (zero between calls)
  double* stats_q;        // per-(item, l, h) sums of squares of x - c (see pool_stats_kernel)
  uint32_t* err;
  PoolShape ps;
  int32_t window;         // anchor only
  XcdShares xs;           // item of work-group i (uniform and given-weight pooling, one share per item)
};

struct WeightArgs {
  const float* s1;  // [total_blocks][L*H][D] token sums of x - c (c: see shift_block)
  const double* q;  // [total_blocks][L*H] sums of (x - c)^2
  double* var;      // [S][L*H]
  double* csum;     // [S][D] sum over heads of weight * c
  float* head_weight;
  const int32_t* seq_len;
  const int32_t* offs;
  const int32_t* table;
  const uint16_t* k;
  int64_t sL, sB, sH, P;
  int32_t S, L, H, LH, D, B, total_blocks;
  uint32_t* err;
};

// Physical block holding the first token of sequence s, whose keys shift the
// head-variance statistics, or -1 (the shift is then 0) when the sequence
// has no token or its first table entry is unusable.  Every variance-mode
// kernel takes the shift from here, so they agree on it.
__device__ __forceinline__ int64_t shift_block(const int32_t* __restrict__ seq_len, const int32_t* __restrict__ offs,
                                               const int32_t* __restrict__ table, int32_t total_blocks, int64_t P,
                                               int32_t s) {
  const int32_t b0 = offs[s], b1 = offs[s + 1];
  if (seq_len[s] <= 0 || b0 < 0 || b0 >= b1 || b1 > total_blocks) return -1;
  const int64_t p = table[b0];
  return p >= 0 && p < P ? p : -1;
}

// Pool-on-write: one new token per sequence.
struct WriteArgs {
  const uint16_t* k_new;  // [S][L][H][D] new keys, or null (already in the pool)
  uint16_t* k;            // the pool; the new keys are stored into it
  int64_t sL, sB, sT, sH;
  int32_t L, H, D, B;
  int64_t P;
  int32_t S;
  const int32_t* seq_len;
  const int32_t* offs;
  const int32_t* table;
  const float* weights;   // [S][L*H] frozen head weights, or null (uniform)
  float* running;         // [S][D] the open block's key sum
  float* out;             // v_b rows
  int64_t vb_stride;      // rows per sequence in `out`, 0 = row is the global block id
  int32_t seed;           // 1: rebuild the running sum from the pool
  int32_t q8, m, nt;      // D/8 threads per key row, m rows in flight, nt = q8 * m
  uint32_t* err;
};

// Attention mass per block (one decode query per sequence).
struct AttnArgs {
  const uint16_t* k;
  int64_t sL, sB, sT, sH;
  int32_t L, H, D, B;
  int64_t P;
  int32_t S, total_blocks;
  const int32_t* seq_len;
  const int32_t* offs;
  const int32_t* table;
  const float* q;        // [S][L][Hq][D]
  int32_t Hq, G;         // query heads, query heads per KV head
  float scale;
  int32_t TB, TT;        // blocks and tokens per tile
  int32_t max_tiles;     // grid bound on tiles
  int32_t n_chunks;      // head chunks of the block-mass pass
  int32_t U, UPB;        // tokens per unit (a block or 16 tokens), units per block
  int32_t mfma;          // 1: matrix-core logits kernel, 0: vector kernel
  int32_t* tile_offs;    // [S+1] first tile of each sequence
  int32_t* n_blocks;     // [S] blocks holding tokens (selection candidates)
  float* um;             // [L*Hq][total_blocks*UPB] unit maximum logit (-inf: no token)
  float* ue;             // [L*Hq][total_blocks*UPB] unit sum of exp(logit - unit max)
  float* M;              // [S][L*Hq] sequence maximum logit
  float* Z;              // [S][L*Hq] softmax normaliser
  float* partial;        // [n_chunks][total_blocks] block mass per head chunk
  float* out;            // block scores, out + s * out_stride + j
  int64_t out_stride;
  uint32_t* err;
};

struct LevelArgs {
  float* lvl;
  int64_t rows_per_seq;
  int32_t S, max_pages, D, ppc, cpg, c_cap, g_cap;
  const int32_t* n_pages;
  const int32_t* first_dirty;
  uint32_t* err;
};

struct ScoreArgs {
  const float* lvl;
  int64_t rows_per_seq;
  int32_t S, max_pages, D, hier, ppc, cpg, c_cap, g_cap;
  const int32_t* n_pages;
  const float* anchors;
  float* aff;            // affinity rows, aff + s * rows_per_seq + row
  int32_t k_g, k_c, k_p;
  int32_t* idx_out;
  float* score_out;
  int32_t* cnt_out;
  int32_t tiles_per_seq, rows_per_tile;
  int32_t small;         // 1: every level fits the one-launch selector (small_select_fits)
  uint32_t* done;        // per-sequence count of finished scoring tiles (zero between calls), or null
  uint32_t* err;
  // stability filter (page rows only; hist == nullptr: off)
  uint32_t* hist;        // window words, hist + s * max_pages + page
  float* stab_out;       // stability scores, same indexing (may be null)
  uint32_t stab_mask;    // low `stab_w` bits set
  int32_t stab_w;
  float theta;
};

// Hierarchical levels small enough for the lean selection path of the
// per-sequence selectors (kka_score.hip): at most 64 grids, at most 64
// chunk candidates (children of the kept grids), at most 256 page
// candidates, at most 64 kept per level, at most kLeanHiRows chunk and grid
// rows, at least one page row and every row staged in LDS.  Kernel
// arguments only: the choice holds at any page count.
constexpr int kLeanHiRows = 1024;
inline __host__ __device__ bool lean_levels_fit(const ScoreArgs& a) {
  const int64_t kg = a.k_g < a.g_cap ? a.k_g : a.g_cap;
  const int64_t kc = a.k_c < a.c_cap ? a.k_c : a.c_cap;
  const int64_t kp = a.k_p < a.max_pages ? a.k_p : a.max_pages;
  return a.hier && a.max_pages >= 1 && a.rows_per_seq <= kSelectLdsRows &&
         a.rows_per_seq - a.max_pages <= kLeanHiRows && a.g_cap <= 64 && kg >= 0 && kg * a.cpg <= 64 && kc >= 0 &&
         kc <= 64 && kc * a.ppc <= 256 && kp >= 0 && kp <= 64;
}

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Largest s in [0, S) with offs[s] <= b (offsets nondecreasing).
__device__ __forceinline__ int32_t find_seq(const int32_t* __restrict__ offs, int32_t S, int32_t b) {
  int32_t lo = 0, hi = S - 1;
  while (lo < hi) {
    int32_t mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= b) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ void raise_err(uint32_t* err, uint32_t bit) { atomicOr(err, bit); }

// Values handed from one work-group to another inside one launch (work-
// groups on any XCD, and each XCD has its own L2) are stored and loaded
// with device-scope relaxed atomics, which write through and read past the
// non-coherent L2, instead of paying a device-scope release fence (a whole-
// L2 write-back) per work-group.  The handoff's order comes from the
// hardware rather than from release / acquire: the producer waits for its
// stores to be acknowledged (vmcnt 0) before its device-scope counter
// increment (arrive), and the consumer loads only after its own increment
// has returned the last count.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A work-group's arrival at the end of its share of an item split over n
// work-groups, once all of its device-scope stores have completed: true in
// every thread of the work-group that arrives last.  The counter wraps back
// to 0 on that arrival, ready for the next launch; a counter found at n or
// above (a workspace not zeroed before its first use) raises
// KKA_DEVERR_WORKSPACE.  `flag` is a __shared__ word of the work-group.
__device__ __forceinline__ bool arrive(uint32_t* done, uint32_t n, uint32_t* err, uint32_t& flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned top = n - 1u;
    const unsigned old = atomicInc(done, top);
    if (old > top) raise_err(err, KKA_DEVERR_WORKSPACE);
    flag = old == top;
  }
  __syncthreads();
  return flag != 0u;
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are already valid.

hipError_t launch_pool(const PoolArgs& a, int mode, hipStream_t st);          // uniform / given
hipError_t launch_pool_stats(const PoolArgs& a, hipStream_t st);              // variance pass 1
hipError_t launch_head_weights(const WeightArgs& w, hipStream_t st);          // variance pass 2
hipError_t launch_pool_combine(const PoolArgs& a, const float* w, const double* csum, hipStream_t st);  // pass 3
hipError_t launch_anchor(const PoolArgs& a, hipStream_t st);
hipError_t launch_levels(const LevelArgs& a, hipStream_t st);
hipError_t launch_pool_on_write(const WriteArgs& a, hipStream_t st);
hipError_t launch_attention_blocks(const AttnArgs& a, hipStream_t st);
int32_t attention_chunk_heads();  // (layer, query head) pairs per block-mass chunk
int32_t attention_tile_blocks(int32_t B, int32_t H, int32_t G, bool mfma);  // blocks per tile, 0 = too large
bool attention_mfma_ok(int32_t D, int32_t G, int32_t B);  // matrix-core logits apply
hipError_t launch_score_topk(const ScoreArgs& a, hipStream_t st);
// Lazy hierarchical variant: one work-group per sequence; scored affinities
// also go to lazy_out when it is set (a.aff is scratch for long sequences).
hipError_t launch_score_topk_lazy(const ScoreArgs& a, float* lazy_out, hipStream_t st);
int32_t score_rows_per_tile(int32_t D);  // rows one score work-group covers
// Selection only, over scores already in a.aff (non-negative, not NaN).
hipError_t launch_select(const ScoreArgs& a, hipStream_t st);

}  // namespace kka
