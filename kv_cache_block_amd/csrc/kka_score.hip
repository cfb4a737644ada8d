// Affinity of every level row, then Grid -> Chunk -> Page top-K.
//
// Page "Key-Key Semantic Affinity: Key vectors replace attention scores for
// KV-cache importance" (10100.com): section 2.2 step 3 (affinity of anchor
// and block vector, normalised), section 5.1 (all three levels scored in a
// single pass, children of unselected parents masked to zero) and section
// 5.2 step 4 (keep the K highest-affinity blocks).
//
// score_kernel: a batched GEMV with one right-hand side per sequence, bound
// by HBM bandwidth.  Each sequence's present rows are cut into tiles spread
// over the whole chip; in a tile, 8 lanes share one row (each lane reads
// 16-byte pieces 128 bytes apart, so 8 lanes read whole 128-byte lines) and
// every lane keeps 16 loads in flight.  Dot product and row norm are reduced
// over the 8 lanes with a fixed butterfly.  No cross-group communication:
// the kernel boundary publishes the affinities.
//
// select_kernel: one work-group per sequence.  The sequence's affinity rows
// are staged into LDS with one coalesced pass, then each level is selected
// from LDS: candidates (children of kept parents, or every row) with a
// positive score are compacted with wave ballots; up to 512 of them are
// ranked directly (rank = number of larger keys, so rank < k places the
// element at its final position); larger sets use an MSB-first radix select.
// Keys are (affinity bits << 32 | ~index): unique, and larger means higher
// score then lower index.  When fewer than k candidates score above zero,
// the lowest-index rows scoring exactly 0 (masked or zero affinity) fill the
// remaining slots in index order.
#include "kka_internal.h"

namespace kka {
namespace {

constexpr int kSelThreads = 256;
constexpr int kRankMax = 512;
constexpr int kLdsRows = 9216;  // affinity rows staged per sequence (36 KB)

struct SelectShared {
  float aff[kLdsRows];
  uint64_t ck[kRankMax];
  uint64_t buf[kMaxK];
  uint32_t bitmap[kMaxParents / 32];
  int32_t plist[kMaxK];
  uint32_t hist[256];
  uint32_t digit, above, bucket;
  int32_t cnt;
  int32_t np_sel;
  int32_t wave_tot[kSelThreads / 64];
};

struct Level {
  const float* aff;  // score of element e is aff[e] when live (LDS or global)
  int32_t n;         // elements in the level
  int32_t fanout;    // children per parent; 0 = no parent level (all live)
  int32_t n_par;     // kept parents listed in plist (fanout > 0)
};

__device__ __forceinline__ uint32_t aff_key(const Level& L, int32_t e) { return __float_as_uint(L.aff[e]); }

__device__ __forceinline__ bool is_live(const Level& L, const SelectShared& sm, int32_t e) {
  if (L.fanout == 0) return true;
  const int32_t p = e / L.fanout;
  return (sm.bitmap[p >> 5] >> (p & 31)) & 1u;
}

// Candidate c -> element index (or -1 when past the level's end).
__device__ __forceinline__ int32_t cand(const Level& L, const SelectShared& sm, int64_t c) {
  if (L.fanout == 0) return (int32_t)c;
  const int32_t pi = (int32_t)(c / L.fanout);
  const int32_t e = sm.plist[pi] * L.fanout + (int32_t)(c - (int64_t)pi * L.fanout);
  return e < L.n ? e : -1;
}

__device__ __forceinline__ uint64_t composite(uint32_t key, int32_t e) {
  return ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)e);
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

// Radix select over every positive candidate (re-enumerated each pass), for
// candidate sets too large to rank; leaves the top k_eff sorted in sm.buf.
__device__ void radix_top(const Level& L, int64_t m, int32_t k_eff, SelectShared& sm) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0, mask = 0;
  int32_t kk = k_eff;
  for (int shift = 56; shift >= 0; shift -= 8) {
    sm.hist[tid] = 0u;
    __syncthreads();
    for (int64_t c = tid; c < m; c += kSelThreads) {
      const int32_t e = cand(L, sm, c);
      if (e < 0) continue;
      const uint32_t key = aff_key(L, e);
      if (key == 0u) continue;
      const uint64_t comp = composite(key, e);
      if ((comp & mask) == prefix) atomicAdd(&sm.hist[(uint32_t)(comp >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) pick_digit(sm, kk);
    __syncthreads();
    prefix |= (uint64_t)sm.digit << shift;
    mask |= (uint64_t)255u << shift;
    kk -= (int32_t)sm.above;
    const bool done = sm.bucket == (uint32_t)kk;
    __syncthreads();
    if (done) break;
  }
  if (tid == 0) sm.cnt = 0;
  __syncthreads();
  for (int64_t c = tid; c < m; c += kSelThreads) {
    const int32_t e = cand(L, sm, c);
    if (e < 0) continue;
    const uint32_t key = aff_key(L, e);
    if (key == 0u) continue;
    const uint64_t comp = composite(key, e);
    if (comp >= prefix) {
      const int32_t slot = atomicAdd(&sm.cnt, 1);
      if (slot < k_eff) sm.buf[slot] = comp;
    }
  }
  __syncthreads();
  sort_desc(sm, k_eff);
}

// Keeps the top min(k, n) elements of a level, sorted, in sm.buf.
__device__ int32_t select_level(const Level& L, int32_t k, SelectShared& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const int32_t k_eff = k < L.n ? k : L.n;
  if (k_eff <= 0) return 0;
  const int64_t m = L.fanout ? (int64_t)L.n_par * L.fanout : (int64_t)L.n;
  if (tid == 0) sm.cnt = 0;
  __syncthreads();
  // compact the candidates scoring above zero
  for (int64_t c0 = 0; c0 < m; c0 += kSelThreads) {
    const int64_t c = c0 + tid;
    const int32_t e = c < m ? cand(L, sm, c) : -1;
    const uint32_t key = e >= 0 ? aff_key(L, e) : 0u;
    const bool pos = key != 0u;
    const uint64_t bal = __ballot(pos);
    int32_t base = 0;
    if (lane == 0 && bal) base = atomicAdd(&sm.cnt, (int32_t)__popcll(bal));
    base = __shfl(base, 0, 64);
    const int32_t slot = base + (int32_t)__popcll(bal & lt_mask);
    if (pos && slot < kRankMax) sm.ck[slot] = composite(key, e);
  }
  __syncthreads();
  const int32_t P = sm.cnt;
  __syncthreads();
  if (P > kRankMax) {
    // too many to rank: radix select the top k_eff, or (when k_eff is larger
    // still) all P positive candidates, sorted; zeros fill the rest below
    const int32_t take = P >= k_eff ? k_eff : P;
    radix_top(L, m, take, sm);
    if (P >= k_eff) return k_eff;
  } else {
    // rank the positive candidates: rank r goes to slot r when r < k_eff
    for (int32_t i = tid; i < P; i += kSelThreads) {
      const uint64_t x = sm.ck[i];
      int32_t r = 0;
      int32_t j = 0;
      for (; j + 4 <= P; j += 4)
        r += (int32_t)(sm.ck[j] > x) + (int32_t)(sm.ck[j + 1] > x) + (int32_t)(sm.ck[j + 2] > x) +
             (int32_t)(sm.ck[j + 3] > x);
      for (; j < P; ++j) r += (int32_t)(sm.ck[j] > x);
      if (r < k_eff) sm.buf[r] = x;
    }
    __syncthreads();
    if (P >= k_eff) return k_eff;
  }
  // lowest-index rows scoring exactly 0 fill the remaining slots, in order
  const int32_t need = k_eff - P;
  int32_t found = 0;
  for (int32_t e0 = 0; e0 < L.n && found < need; e0 += kSelThreads) {
    const int32_t e = e0 + tid;
    const bool zero = e < L.n && (!is_live(L, sm, e) || aff_key(L, e) == 0u);
    const uint64_t bal = __ballot(zero);
    if (lane == 0) sm.wave_tot[wave] = (int32_t)__popcll(bal);
    __syncthreads();
    int32_t before = 0, tot = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) {
      if (w < wave) before += sm.wave_tot[w];
      tot += sm.wave_tot[w];
    }
    const int32_t rank = found + before + (int32_t)__popcll(bal & lt_mask);
    if (zero && rank < need) sm.buf[P + rank] = composite(0u, e);
    found += tot;
    __syncthreads();
  }
  return k_eff;
}

// Marks the kept elements of a level as parents of the next one.
__device__ void keep_parents(SelectShared& sm, int32_t k_eff, int32_t n_parents) {
  const int tid = threadIdx.x;
  for (int32_t w = tid; w < (n_parents + 31) / 32; w += kSelThreads) sm.bitmap[w] = 0u;
  __syncthreads();
  for (int32_t i = tid; i < k_eff; i += kSelThreads) {
    const int32_t e = (int32_t)(~(uint32_t)sm.buf[i]);
    sm.plist[i] = e;
    atomicOr(&sm.bitmap[e >> 5], 1u << (e & 31));
  }
  if (tid == 0) sm.np_sel = k_eff;
  __syncthreads();
}

struct SeqGeom {
  int32_t n_p, n_c, n_g;
};

__device__ __forceinline__ SeqGeom seq_geom(const ScoreArgs& a, int32_t s, bool report) {
  SeqGeom g;
  g.n_p = a.n_pages[s];
  if (g.n_p < 0 || g.n_p > a.max_pages) {
    if (report) raise_err(a.err, KKA_DEVERR_PAGES);
    g.n_p = g.n_p < 0 ? 0 : a.max_pages;
  }
  g.n_c = a.hier ? (g.n_p + a.ppc - 1) / a.ppc : 0;
  g.n_g = a.hier ? (g.n_c + a.cpg - 1) / a.cpg : 0;
  return g;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(ScoreArgs a) {
  __shared__ SelectShared sm;
  const int tid = threadIdx.x;
  const int32_t s = blockIdx.x;
  const SeqGeom g = seq_geom(a, s, false);
  const float* aff = a.aff + (int64_t)s * a.rows_per_seq;
  const float* base = aff;
  if (a.rows_per_seq <= kLdsRows) {
    // stage the present rows of every level at their row offsets
    for (int32_t r = tid; r < g.n_p; r += kSelThreads) sm.aff[r] = aff[r];
    for (int32_t r = tid; r < g.n_c; r += kSelThreads) sm.aff[a.max_pages + r] = aff[a.max_pages + r];
    for (int32_t r = tid; r < g.n_g; r += kSelThreads)
      sm.aff[a.max_pages + a.c_cap + r] = aff[a.max_pages + a.c_cap + r];
    __syncthreads();
    base = sm.aff;
  }
  int32_t kp;
  if (a.hier) {
    Level G{base + a.max_pages + a.c_cap, g.n_g, 0, 0};
    const int32_t kg = select_level(G, a.k_g, sm);
    keep_parents(sm, kg, g.n_g);
    Level C{base + a.max_pages, g.n_c, a.cpg, sm.np_sel};
    const int32_t kc = select_level(C, a.k_c, sm);
    keep_parents(sm, kc, g.n_c);
    Level Pg{base, g.n_p, a.ppc, sm.np_sel};
    kp = select_level(Pg, a.k_p, sm);
  } else {
    Level Pg{base, g.n_p, 0, 0};
    kp = select_level(Pg, a.k_p, sm);
  }
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

// (1 + cos) / 2 clamped to [0, 1]; NaN and -0 become +0.
__device__ __forceinline__ float affinity_of(float dot, float nr, float sqrt_na, float na) {
  const float c = (nr > 0.f && na > 0.f) ? dot / (sqrtf(nr) * sqrt_na) : 0.f;
  const float v = 0.5f * (1.0f + c);
  return v > 0.f ? (v < 1.f ? v : 1.f) : 0.f;
}

template <int NQ, int R>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  const int tid = threadIdx.x;
  const int32_t s = blockIdx.x / a.tiles_per_seq;
  const int32_t tile = blockIdx.x - s * a.tiles_per_seq;
  const SeqGeom g = seq_geom(a, s, tid == 0 && tile == 0);
  const int32_t nv = g.n_p + g.n_c + g.n_g;
  const int32_t v0 = tile * a.rows_per_tile;
  if (v0 >= nv) return;
  const int32_t v1 = min(nv, v0 + a.rows_per_tile);
  const int32_t Q = a.D >> 2;
  const float4* seq = reinterpret_cast<const float4*>(a.lvl + (int64_t)s * a.rows_per_seq * a.D);
  float* aff = a.aff + (int64_t)s * a.rows_per_seq;

  const int32_t grp = tid >> 3, lg = tid & 7;
  float4 av[NQ];
  float na = 0.f;
  const float4* anc = reinterpret_cast<const float4*>(a.anchors + (int64_t)s * a.D);
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int32_t qi = lg + 8 * j;
    av[j] = qi < Q ? anc[qi] : make_float4(0.f, 0.f, 0.f, 0.f);
    na = fmaf(av[j].x, av[j].x, na);
    na = fmaf(av[j].y, av[j].y, na);
    na = fmaf(av[j].z, av[j].z, na);
    na = fmaf(av[j].w, av[j].w, na);
  }
  na += __shfl_xor(na, 1);
  na += __shfl_xor(na, 2);
  na += __shfl_xor(na, 4);
  const float sqrt_na = sqrtf(na);

  for (int32_t v = v0 + grp; v < v1; v += 32 * R) {
    float4 x[R][NQ];
    int64_t row[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int32_t vr = v + 32 * r;
      const bool ok = vr < v1;
      row[r] = !ok ? 0
               : vr < g.n_p ? vr
               : vr < g.n_p + g.n_c ? (int64_t)a.max_pages + (vr - g.n_p)
                                    : (int64_t)a.max_pages + a.c_cap + (vr - g.n_p - g.n_c);
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const int32_t qi = lg + 8 * j;
        x[r][j] = (ok && qi < Q) ? seq[row[r] * Q + qi] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float dot = 0.f, nr = 0.f;
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        dot = fmaf(x[r][j].x, av[j].x, dot);
        dot = fmaf(x[r][j].y, av[j].y, dot);
        dot = fmaf(x[r][j].z, av[j].z, dot);
        dot = fmaf(x[r][j].w, av[j].w, dot);
        nr = fmaf(x[r][j].x, x[r][j].x, nr);
        nr = fmaf(x[r][j].y, x[r][j].y, nr);
        nr = fmaf(x[r][j].z, x[r][j].z, nr);
        nr = fmaf(x[r][j].w, x[r][j].w, nr);
      }
      dot += __shfl_xor(dot, 1);
      nr += __shfl_xor(nr, 1);
      dot += __shfl_xor(dot, 2);
      nr += __shfl_xor(nr, 2);
      dot += __shfl_xor(dot, 4);
      nr += __shfl_xor(nr, 4);
      if (lg == 0 && v + 32 * r < v1) aff[row[r]] = affinity_of(dot, nr, sqrt_na, na);
    }
  }
}

template <int NQ>
hipError_t launch_nq(const ScoreArgs& a, hipStream_t st) {
  constexpr int R = NQ >= 16 ? 1 : 16 / NQ;
  const dim3 grid((unsigned)((int64_t)a.S * a.tiles_per_seq));
  hipLaunchKernelGGL((score_kernel<NQ, R>), grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)a.S), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// Rows per tile for a given head_dim: one pass of the 32 row-groups.
int32_t score_rows_per_tile(int32_t D) {
  const int32_t nq = (D / 4 + 7) / 8;
  int32_t NQ = 1;
  while (NQ < nq) NQ <<= 1;
  const int32_t R = NQ >= 16 ? 1 : 16 / NQ;
  return 32 * R;
}

hipError_t launch_score_topk(const ScoreArgs& a, hipStream_t st) {
  if (a.S <= 0) return hipSuccess;
  const int32_t nq = (a.D / 4 + 7) / 8;
  if (nq <= 1) return launch_nq<1>(a, st);
  if (nq <= 2) return launch_nq<2>(a, st);
  if (nq <= 4) return launch_nq<4>(a, st);
  if (nq <= 8) return launch_nq<8>(a, st);
  if (nq <= 16) return launch_nq<16>(a, st);
  return launch_nq<32>(a, st);
}

}  // namespace kka
