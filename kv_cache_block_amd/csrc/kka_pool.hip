// Pooling kernels: block vectors v_b and the query anchor.
//
// Page "Key-Key Semantic Affinity: Key vectors replace attention scores for
// KV-cache importance" (10100.com), section 2.2 steps 1-2 and section 5.2
// steps 1-2: a block is summarised by the mean of its keys over every token,
// KV head and layer; the anchor is the same mean over the last few tokens.
// Section 3.3 adds weighting of heads by their variance.
//
// The pool is streamed once.  Every thread owns one 16-byte chunk (8 bf16
// values of one head_dim row) of a token's H*D key row and walks tokens and
// layers, so a wavefront issues 1 KB-contiguous loads for the 7B shape
// (4 heads x 128 dims x 2 B) and keeps 8 independent 16-byte loads in
// flight per lane.  Partial sums stay in fp32 registers; a fixed-order LDS
// reduction finishes each group, so results do not depend on where blocks
// sit in the physical pool or on scheduling.
#include "kka_internal.h"

#ifndef KKA_NT_LOADS
#define KKA_NT_LOADS 1
#endif

namespace kka {
namespace {

constexpr int kUnroll = 8;
enum : int { kUniform = 0, kGiven = 2 };

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
#if KKA_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}

template <int MODE>
__device__ __forceinline__ void accum8(float (&acc)[8], u32x4 v, float w) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t x = v[c];
    if (MODE == kGiven) {
      acc[2 * c] = fmaf(w, bf16_lo(x), acc[2 * c]);
      acc[2 * c + 1] = fmaf(w, bf16_hi(x), acc[2 * c + 1]);
    } else {
      acc[2 * c] += bf16_lo(x);
      acc[2 * c + 1] += bf16_hi(x);
    }
  }
}

// One logical block of a pooling launch.
struct Item {
  int32_t b, s, i, n_b;
  int64_t p;
  int64_t row;  // output row, -1 when it cannot be written
};

// Resolves work item -> (block, sequence, valid tokens, physical block, row).
// Invalid device metadata zeroes n_b (the block then pools to zeros) and,
// when `report`, raises the matching flag bit.  Called by every thread of
// the work-group with the same item.  The metadata goes out in one round of
// loads: the block's table entry (a relaxed atomic load, which keeps its
// place ahead of the lookup; a plain load was issued after the lookup's
// branches, one more memory round trip), and, for fewer than 64 sequences
// on a whole wavefront, every offset and length, one per lane: the
// sequence is the number of offsets <= b less one (offsets are
// nondecreasing) and its values are read from the lanes that hold them.
// Otherwise a binary search over the offsets.  The table entry's atomic
// load is workgroup-scoped, so it may hit in the L2 (the table is written
// before the launch): an agent-scoped one goes past the L2 and, under a
// saturating read stream, queued for tens of microseconds.
__device__ Item locate(const PoolArgs& a, int32_t item, bool report) {
  Item it;
  it.b = a.subset ? a.subset[item] : item;
  it.n_b = 0;
  it.p = 0;
  it.row = -1;
  it.s = 0;
  it.i = 0;
  if (it.b < 0 || it.b >= a.total_blocks || a.S <= 0) {
    if (report) raise_err(a.err, KKA_DEVERR_OFFSETS);
    return it;
  }
  const int32_t p_raw = __hip_atomic_load(a.table + it.b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  int32_t o0, o1, len;
  if (a.S < 64 && __builtin_amdgcn_read_exec() == ~0ull) {
    const int lane = threadIdx.x & 63;
    const int32_t ov = lane <= a.S ? a.offs[lane] : 0;
    const int32_t lv = lane < a.S ? a.seq_len[lane] : 0;
    const uint64_t le = __ballot(lane < a.S && ov <= it.b);
    it.s = le ? (int32_t)__popcll(le) - 1 : 0;
    o0 = __builtin_amdgcn_readlane(ov, it.s);
    o1 = __builtin_amdgcn_readlane(ov, it.s + 1);
    len = __builtin_amdgcn_readlane(lv, it.s);
  } else {
    it.s = find_seq(a.offs, a.S, it.b);
    o0 = a.offs[it.s];
    o1 = a.offs[it.s + 1];
    len = a.seq_len[it.s];
  }
  it.i = it.b - o0;
  if (it.i < 0 || it.b >= o1) {
    if (report) raise_err(a.err, KKA_DEVERR_OFFSETS);
    return it;
  }
  if (a.vb_stride > 0) {
    if ((int64_t)it.i < a.vb_stride) it.row = (int64_t)it.s * a.vb_stride + it.i;
    else if (report) raise_err(a.err, KKA_DEVERR_ROW);
  } else {
    it.row = it.b;
  }
  int64_t nb = (int64_t)len - (int64_t)it.i * a.B;
  if (nb > a.B) nb = a.B;
  if (nb <= 0) {
    if (report) raise_err(a.err, KKA_DEVERR_SEQ_LEN);
    return it;
  }
  const int64_t p = __builtin_amdgcn_readfirstlane(p_raw);
  if (p < 0 || p >= a.P) {
    if (report) raise_err(a.err, KKA_DEVERR_BLOCK_TABLE);
    return it;
  }
  it.p = p;
  it.n_b = (int32_t)nb;
  return it;
}

// Fixed-order reduction of every thread's 8 partial sums into head_dim sums:
// the threads sharing a 16-byte column are tid = dg + r * (D/8).
__device__ __forceinline__ float column_sum(const float* red, int32_t D, int32_t nt, int32_t d) {
  const int32_t DG = D >> 3;
  const int32_t per = nt / DG;
  const int32_t base = ((d >> 3) << 3) + (d & 7);
  float sum = 0.f;
  for (int32_t r = 0; r < per; ++r) sum += red[base + r * DG * 8];
  return sum;
}

__device__ __forceinline__ void stash8(float* red, int tid, const float (&acc)[8]) {
  float4* r4 = reinterpret_cast<float4*>(red);
  r4[2 * tid] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  r4[2 * tid + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// Sum over the n shares of a layer split, in split order, of the partial at
// src + j * stride.  The loads are device-scope (they read past the L2, a
// memory round trip each), so up to 32 shares (every share of a layer
// split of up to 32 layers) are requested in one round before the first
// add; loads past the last share re-read it.
__device__ __forceinline__ float split_sum(const float* src, int32_t n, int32_t stride) {
  constexpr int kRound = 32;
  float sum = 0.f;
  for (int32_t j0 = 0; j0 < n; j0 += kRound) {
    float t[kRound];
#pragma unroll
    for (int u = 0; u < kRound; ++u) t[u] = load_agent(src + (int64_t)min(j0 + u, n - 1) * stride);
#pragma unroll
    for (int u = 0; u < kRound; ++u)
      if (j0 + u < n) sum += t[u];
  }
  return sum;
}

// ------------------------------------------------------------ v_b, one pass

template <int MODE, int MAXT>
__global__ __launch_bounds__(MAXT) void pool_kernel(PoolArgs a) {
  __shared__ float red[MAXT * 8];
  extern __shared__ float wsh[];  // [L*H] head weights (given-weight mode)
  const int tid = threadIdx.x;
  int32_t item = blockIdx.x / a.n_split;
  const int32_t j = blockIdx.x - item * a.n_split;
  if (a.xs.on) {  // one share per item: XCD blockIdx mod 8 takes its range
    const int32_t x = (int32_t)(blockIdx.x % kXcds), r = (int32_t)(blockIdx.x / kXcds);
    if (r >= a.xs.n[x]) return;
    item = a.xs.off[x] + r;
  }
  const Item it = locate(a, item, tid == 0 && j == 0);
  const int32_t LH = a.L * a.H;
  if (MODE == kGiven) {
    for (int x = tid; x < LH; x += a.ps.nt) wsh[x] = a.weights[(int64_t)it.s * LH + x];
    __syncthreads();
  }
  const int32_t DG = a.D >> 3;
  const int32_t q = tid % a.ps.rg;
  const int32_t h = q / DG;
  const int32_t dg = q - h * DG;
  const int32_t toff = tid / a.ps.rg;
  const int32_t l0 = j * a.lps;
  const int32_t nl = min(a.L, l0 + a.lps) - l0;
  const int32_t n_tok = it.n_b > toff ? (it.n_b - toff + a.ps.m - 1) / a.ps.m : 0;
  const int32_t total = n_tok * nl;
  const int64_t step_t = (int64_t)a.ps.m * a.sT;

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint16_t* tp = a.k + it.p * a.sB + (int64_t)h * a.sH + (int64_t)dg * 8 + (int64_t)toff * a.sT +
                       (int64_t)l0 * a.sL;
  const uint16_t* ptr = tp;
  int32_t li = 0;
  int32_t n = 0;
  // layer-inner walk over (token, layer): kUnroll independent loads per step
  for (; n + kUnroll <= total; n += kUnroll) {
    u32x4 v[kUnroll];
    float w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      v[u] = load16(ptr);
      w[u] = MODE == kGiven ? wsh[(l0 + li) * a.H + h] : 0.f;
      ++li;
      ptr += a.sL;
      if (li == nl) {
        li = 0;
        tp += step_t;
        ptr = tp;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) accum8<MODE>(acc, v[u], w[u]);
  }
  for (; n < total; ++n) {
    const u32x4 v = load16(ptr);
    const float w = MODE == kGiven ? wsh[(l0 + li) * a.H + h] : 0.f;
    accum8<MODE>(acc, v, w);
    ++li;
    ptr += a.sL;
    if (li == nl) {
      li = 0;
      tp += step_t;
      ptr = tp;
    }
  }

  stash8(red, tid, acc);
  __syncthreads();
  const float denom = MODE == kGiven ? (float)it.n_b : (float)((int64_t)it.n_b * LH);
  if (a.n_split == 1) {
    if (it.row >= 0)
      for (int32_t d = tid; d < a.D; d += a.ps.nt)
        a.out[it.row * a.D + d] = it.n_b > 0 ? column_sum(red, a.D, a.ps.nt, d) / denom : 0.f;
    return;
  }
  // layer split: shares' partial sums, added in split order by
  // pool_finish_kernel or (a.done set) by the work-group that finishes the
  // item's last share
  float* part = a.partial + (int64_t)item * a.n_split * a.D;
  if (!a.done) {
    for (int32_t d = tid; d < a.D; d += a.ps.nt) part[(int64_t)j * a.D + d] = column_sum(red, a.D, a.ps.nt, d);
    return;
  }
  for (int32_t d = tid; d < a.D; d += a.ps.nt) store_agent(part + (int64_t)j * a.D + d, column_sum(red, a.D, a.ps.nt, d));
  __shared__ uint32_t last;
  if (!arrive(a.done + item, (uint32_t)a.n_split, a.err, last) || it.row < 0) return;
  for (int32_t d = tid; d < a.D; d += a.ps.nt) {
    const float sum = split_sum(part + d, a.n_split, a.D);
    a.out[it.row * a.D + d] = it.n_b > 0 ? sum / denom : 0.f;
  }
}

// Sums the layer-split partials of each item in split order.
template <int MODE>
__global__ __launch_bounds__(256) void pool_finish_kernel(PoolArgs a) {
  const int32_t item = blockIdx.x;
  const Item it = locate(a, item, false);
  if (it.row < 0) return;
  const int32_t LH = a.L * a.H;
  for (int32_t d = threadIdx.x; d < a.D; d += blockDim.x) {
    const float* src = a.partial + (int64_t)item * a.n_split * a.D + d;
    float sum = 0.f;
    for (int32_t j0 = 0; j0 < a.n_split; j0 += 8) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = src[(int64_t)min(j0 + u, a.n_split - 1) * a.D];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < a.n_split) sum += t[u];
    }
    const float denom = MODE == kGiven ? (float)it.n_b : (float)((int64_t)it.n_b * LH);
    a.out[it.row * a.D + d] = it.n_b > 0 ? sum / denom : 0.f;
  }
}

// ------------------------------------------------- variance weights, 3 passes
//
// The weight of head (l, h) is the temporal variance of its keys, averaged
// over head_dim.  The statistics are taken about a shift c: the keys of the
// sequence's first token (shift_block), so that the sums hold x - c and
// (x - c)^2.  x - c of two bf16 values is exact in fp32 for any realistic
// spread of magnitudes and is of the order of the head's spread, not of its
// offset; the variance  sum (x - c)^2 / T - (sum (x - c) / T)^2  then loses
// nothing to cancellation, and a head whose keys never change (one token,
// or the same key at every token) has x - c = 0 everywhere and variance
// exactly 0, as the definition gives.

// Loads the shift of one thread's 16-byte column (8 dims) at layer l.
__device__ __forceinline__ void load_shift(const PoolArgs& a, int64_t p0, int32_t l, int32_t h, int32_t dg,
                                           float (&c)[8]) {
  if (p0 < 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = 0.f;
    return;
  }
  const u32x4 v = *reinterpret_cast<const u32x4*>(a.k + (int64_t)l * a.sL + p0 * a.sB + (int64_t)h * a.sH +
                                                  (int64_t)dg * 8);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    c[2 * e] = bf16_lo(v[e]);
    c[2 * e + 1] = bf16_hi(v[e]);
  }
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

// One 16-byte read of the pass-1 sums, which are read once per pass and
// never again from the cache: non-temporal.
__device__ __forceinline__ float4 load_sums(const float4* p) {
  const f32x4v t = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ void stats8(float (&s1)[8], float (&s2)[8], const float (&c)[8], u32x4 v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x0 = bf16_lo(v[e]) - c[2 * e];
    const float x1 = bf16_hi(v[e]) - c[2 * e + 1];
    s1[2 * e] += x0;
    s1[2 * e + 1] += x1;
    s2[2 * e] = fmaf(x0, x0, s2[2 * e]);
    s2[2 * e + 1] = fmaf(x1, x1, s2[2 * e + 1]);
  }
}

// Pass 1: per block and (layer, head): the token sums of x - c, s1[b][l][h][:],
// and the sum of (x - c)^2, q[b][l][h], one streaming pass over the keys.  A
// thread owns one 16-byte column (8 dims of one head) of one layer and walks
// all of the block's tokens, kUnroll loads in flight, in fp32 (one sum per
// dim, over at most block_size tokens); its 8 sums of x - c leave from
// registers.  The squares of a head's D/8 columns are added in fp64: with
// WAVE, inside the wavefront by a butterfly over the head's lanes (D/8 a
// power of two up to 64: a head's lanes then never straddle a wavefront), so
// the work-group has no barrier at all; otherwise through LDS, once per round
// of m layers.
template <int MAXT, bool WAVE>
__global__ __launch_bounds__(MAXT) void pool_stats_kernel(PoolArgs a) {
  __shared__ double redq[WAVE ? 1 : MAXT];
  const int tid = threadIdx.x;
  const int32_t item = blockIdx.x / a.n_split;
  const int32_t j = blockIdx.x - item * a.n_split;
  const Item it = locate(a, item, tid == 0 && j == 0);
  const int32_t DG = a.D >> 3;
  const int32_t q = tid % a.ps.rg;
  const int32_t h = q / DG;
  const int32_t dg = q - h * DG;
  const int32_t slot = tid / a.ps.rg;
  const int32_t l0 = j * a.lps;
  const int32_t l1 = min(a.L, l0 + a.lps);
  const int32_t n_tok = it.n_b;
  const int64_t p0 = n_tok > 0 ? shift_block(a.seq_len, a.offs, a.table, a.total_blocks, a.P, it.s) : -1;

  for (int32_t lr = l0; lr < l1; lr += a.ps.m) {
    const int32_t l = lr + slot;
    double sq = 0.0;
    if (l < l1) {
      float c[8];
      load_shift(a, p0, l, h, dg, c);
      float s1[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      float s2[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const uint16_t* tp = a.k + (int64_t)l * a.sL + it.p * a.sB + (int64_t)h * a.sH + (int64_t)dg * 8;
      int32_t ti = 0;
      for (; ti + kUnroll <= n_tok; ti += kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = load16(tp + (int64_t)(ti + u) * a.sT);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) stats8(s1, s2, c, v[u]);
      }
      for (; ti < n_tok; ++ti) stats8(s1, s2, c, load16(tp + (int64_t)ti * a.sT));
      // streamed out (non-temporal): read back once, by head_var_kernel and
      // pool_combine_kernel, long after this pass has moved on
      f32x4v* dst = reinterpret_cast<f32x4v*>(a.partial + (((int64_t)item * a.L + l) * a.H) * a.D + (int64_t)q * 8);
      __builtin_nontemporal_store(f32x4v{s1[0], s1[1], s1[2], s1[3]}, dst);
      __builtin_nontemporal_store(f32x4v{s1[4], s1[5], s1[6], s1[7]}, dst + 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) sq += (double)s2[e];
    }
    if constexpr (WAVE) {
      // a head's DG lanes are an aligned group inside one wavefront, all on
      // the same layer: every lane of the group takes part
      for (int32_t o = 1; o < DG; o <<= 1) sq += __shfl_xor(sq, o);
      if (l < l1 && dg == 0) a.stats_q[((int64_t)item * a.L + l) * a.H + h] = sq;
    } else {
      redq[tid] = sq;
      __syncthreads();
      // sum of squares per (layer, head) of this round, columns in order
      if (tid < a.ps.m * a.H) {
        const int32_t sl = tid / a.H, hh = tid - sl * a.H;
        const int32_t ll = lr + sl;
        if (ll < l1) {
          double t = 0.0;
          for (int32_t x = 0; x < DG; ++x) t += redq[sl * a.ps.rg + hh * DG + x];
          a.stats_q[((int64_t)item * a.L + ll) * a.H + hh] = t;
        }
      }
      __syncthreads();
    }
  }
}

// Pass 2: one group per (sequence, head): temporal variance of the head,
//   var = ( sum_tau |x_tau - c|^2 / T  -  sum_d (sum_tau (x_tau,d - c_d) / T)^2 ) / D,
// from the pass-1 sums, combined in fp64 (clamped at 0 against rounding).
// D / 4 lanes cover a head's row of sums with 16-byte loads; the 256
// threads form 256 / (D / 4) such lane groups, group g summing blocks g,
// g + ng, ... with kVarUnroll independent loads in flight.  The groups' sums
// are then added in group order (a fixed order, so the result is
// reproducible).
constexpr int kVarUnroll = 4;

__global__ __launch_bounds__(256) void head_var_kernel(WeightArgs w) {
  __shared__ double part[1024];  // [ng][D]: ng * D = 4 * 256 at most
  __shared__ double r1[256];
  __shared__ double r2[256];
  const int tid = threadIdx.x;
  const int32_t s = blockIdx.x / w.LH;
  const int32_t lh = blockIdx.x - s * w.LH;
  // offsets are device data: clamp to the sums the pass-1 launch wrote
  const int32_t b1 = min(max(w.offs[s + 1], 0), w.total_blocks);
  const int32_t b0 = min(max(w.offs[s], 0), b1);
  const int64_t T = w.seq_len[s] > 0 ? w.seq_len[s] : 0;
  const int32_t nl = w.D / 4;  // lanes per row (head_dim is a multiple of 8, at most 1024)
  const int32_t ng = 256 / nl;
  const int32_t g = tid / nl, c = tid - g * nl;
  const int64_t bstride = (int64_t)w.LH * nl;  // float4s from one block's sums to the next block's
  const float4* base = reinterpret_cast<const float4*>(w.s1 + (int64_t)lh * w.D) + c;
  if (g < ng) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    int32_t b = b0 + g;
    for (; b + (kVarUnroll - 1) * ng < b1; b += kVarUnroll * ng) {
      float4 x[kVarUnroll];
#pragma unroll
      for (int u = 0; u < kVarUnroll; ++u) x[u] = load_sums(base + (int64_t)(b + u * ng) * bstride);
#pragma unroll
      for (int u = 0; u < kVarUnroll; ++u) {
        acc[0] += (double)x[u].x;
        acc[1] += (double)x[u].y;
        acc[2] += (double)x[u].z;
        acc[3] += (double)x[u].w;
      }
    }
    for (; b < b1; b += ng) {
      const float4 x = load_sums(base + (int64_t)b * bstride);
      acc[0] += (double)x.x;
      acc[1] += (double)x.y;
      acc[2] += (double)x.z;
      acc[3] += (double)x.w;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) part[g * w.D + 4 * c + e] = acc[e];
  }
  __syncthreads();
  double m2 = 0.0;
  for (int32_t d = tid; d < w.D; d += 256) {
    double s1 = 0.0;
    for (int32_t q = 0; q < ng; ++q) s1 += part[q * w.D + d];
    const double mean = T > 0 ? s1 / (double)T : 0.0;
    m2 += mean * mean;
  }
  double qs = 0.0;
  for (int32_t b = b0 + tid; b < b1; b += 256) qs += w.q[(int64_t)b * w.LH + lh];
  r1[tid] = m2;
  r2[tid] = qs;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) {
      r1[tid] += r1[tid + off];
      r2[tid] += r2[tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double v = T > 0 ? (r2[0] / (double)T - r1[0]) / (double)w.D : 0.0;
    w.var[(int64_t)s * w.LH + lh] = v > 0.0 ? v : 0.0;
  }
}

// Pass 2b: weights = variance / sum of variances (uniform when the sum is
// 0), rounded to fp32; and the shift term of the block vectors,
//   csum[s][d] = sum_{l,h} w[l,h] * c[l,h][d]   (fp64),
// so that pass 3 adds it back: the weighted mean of a block's keys is the
// weighted mean of x - c plus this constant.
__global__ __launch_bounds__(256) void head_norm_kernel(WeightArgs w) {
  __shared__ double r[256];
  __shared__ float wf[4096];  // L*H <= 4096
  const int tid = threadIdx.x;
  const int32_t s = blockIdx.x;
  double v = 0.0;
  for (int32_t x = tid; x < w.LH; x += 256) v += w.var[(int64_t)s * w.LH + x];
  r[tid] = v;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) r[tid] += r[tid + off];
    __syncthreads();
  }
  const double total = r[0];
  for (int32_t x = tid; x < w.LH; x += 256) {
    const float wx = total > 0.0 ? (float)(w.var[(int64_t)s * w.LH + x] / total) : (float)(1.0 / (double)w.LH);
    w.head_weight[(int64_t)s * w.LH + x] = wx;
    wf[x] = wx;
  }
  __syncthreads();
  const int64_t p0 = shift_block(w.seq_len, w.offs, w.table, w.total_blocks, w.P, s);
  constexpr int kShiftLoads = 16;  // independent loads in flight per thread
  for (int32_t d = tid; d < w.D; d += 256) {
    double cs = 0.0;
    if (p0 >= 0) {
      const uint16_t* src = w.k + p0 * w.sB + d;
      for (int32_t lh0 = 0; lh0 < w.LH; lh0 += kShiftLoads) {
        float c[kShiftLoads];
#pragma unroll
        for (int u = 0; u < kShiftLoads; ++u) {
          const int32_t lh = min(lh0 + u, w.LH - 1);
          const int32_t l = lh / w.H, h = lh - l * w.H;
          c[u] = __uint_as_float((uint32_t)src[(int64_t)l * w.sL + (int64_t)h * w.sH] << 16);
        }
#pragma unroll
        for (int u = 0; u < kShiftLoads; ++u)
          if (lh0 + u < w.LH) cs = fma((double)wf[lh0 + u], (double)c[u], cs);
      }
    }
    w.csum[(int64_t)s * w.D + d] = cs;
  }
}

// Pass 3: v_b = sum_{l,h} w[s][l,h] * s1[b][l][h][:] / n_b + csum[s][:].  One
// group of head_dim threads per block: D / 4 lanes cover a row with 16-byte
// loads, and lane group g (of 4) accumulates heads lh = g, g + 4, ... in
// order; the four group sums are added as (g0 + g1) + (g2 + g3), a fixed
// order, divided by n_b and added to the shift term in fp64.
constexpr int kCombineUnroll = 4;

__global__ __launch_bounds__(1024) void pool_combine_kernel(PoolArgs a, const float* __restrict__ wts,
                                                            const double* __restrict__ csum) {
  extern __shared__ float4 gsum[];  // [3][D / 4]: the sums of groups 1..3
  const int32_t item = blockIdx.x;
  const Item it = locate(a, item, false);
  if (it.row < 0) return;  // the same for every thread of the group
  const int32_t LH = a.L * a.H;
  const int32_t nl = a.D / 4;
  const int32_t g = threadIdx.x / nl, c = threadIdx.x - g * nl;
  const float4* src = reinterpret_cast<const float4*>(a.partial + (int64_t)item * LH * a.D) + c;
  const float* wr = wts + (int64_t)it.s * LH;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  int32_t lh = g;
  for (; lh + 4 * (kCombineUnroll - 1) < LH; lh += 4 * kCombineUnroll) {
    float4 x[kCombineUnroll];
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) x[u] = load_sums(src + (int64_t)(lh + 4 * u) * nl);
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) {
      const float wv = wr[lh + 4 * u];
      acc.x = fmaf(wv, x[u].x, acc.x);
      acc.y = fmaf(wv, x[u].y, acc.y);
      acc.z = fmaf(wv, x[u].z, acc.z);
      acc.w = fmaf(wv, x[u].w, acc.w);
    }
  }
  for (; lh < LH; lh += 4) {
    const float wv = wr[lh];
    const float4 x = load_sums(src + (int64_t)lh * nl);
    acc.x = fmaf(wv, x.x, acc.x);
    acc.y = fmaf(wv, x.y, acc.y);
    acc.z = fmaf(wv, x.z, acc.z);
    acc.w = fmaf(wv, x.w, acc.w);
  }
  if (g > 0) gsum[(g - 1) * nl + c] = acc;
  __syncthreads();
  if (g == 0) {
    const float4 a1 = gsum[c], a2 = gsum[nl + c], a3 = gsum[2 * nl + c];
    const double nb = (double)it.n_b;
    const double* cs = csum + (int64_t)it.s * a.D + 4 * c;
    float4 v;
    v.x = it.n_b > 0 ? (float)((double)((acc.x + a1.x) + (a2.x + a3.x)) / nb + cs[0]) : 0.f;
    v.y = it.n_b > 0 ? (float)((double)((acc.y + a1.y) + (a2.y + a3.y)) / nb + cs[1]) : 0.f;
    v.z = it.n_b > 0 ? (float)((double)((acc.z + a1.z) + (a2.z + a3.z)) / nb + cs[2]) : 0.f;
    v.w = it.n_b > 0 ? (float)((double)((acc.w + a1.w) + (a2.w + a3.w)) / nb + cs[3]) : 0.f;
    reinterpret_cast<float4*>(a.out + it.row * a.D)[c] = v;
  }
}

// ------------------------------------------------------------------ anchor

// One group per (sequence, layer range): the last W_eff tokens of the
// sequence, gathered through the block table (the window may straddle
// blocks).  The window's block ids are read once into LDS; the (token,
// layer) pairs of a thread are then walked like the block pool, with
// kUnroll independent 16-byte loads in flight.
constexpr int kWindowBlocks = 1024;  // window block ids staged in LDS

template <int MODE, int MAXT>
__global__ __launch_bounds__(MAXT) void anchor_kernel(PoolArgs a) {
  __shared__ float red[MAXT * 8];
  __shared__ int64_t wblk[kWindowBlocks];
  extern __shared__ float wsh[];
  const int tid = threadIdx.x;
  const int32_t s = blockIdx.x / a.n_split;
  const int32_t j = blockIdx.x - s * a.n_split;
  const int32_t LH = a.L * a.H;
  const int32_t T = a.seq_len[s] > 0 ? a.seq_len[s] : 0;
  const int32_t W = a.window < T ? a.window : T;
  // offsets are device data: never index the table outside [0, total_blocks)
  const int32_t b1 = min(max(a.offs[s + 1], 0), a.total_blocks);
  const int32_t b0 = min(max(a.offs[s], 0), b1);
  const int32_t nb_s = b1 - b0;
  const int32_t i_first = W > 0 ? (T - W) / a.B : 0;
  const int32_t nbw = W > 0 ? (T - 1) / a.B - i_first + 1 : 0;
  const bool staged = nbw <= kWindowBlocks;
  if (MODE == kGiven)
    for (int x = tid; x < LH; x += a.ps.nt) wsh[x] = a.weights[(int64_t)s * LH + x];
  if (staged) {
    // -1: past the sequence's blocks; -2: physical id outside the pool
    for (int32_t x = tid; x < nbw; x += a.ps.nt) {
      const int32_t i = i_first + x;
      int64_t p = -1;
      if (i < nb_s) {
        p = a.table[b0 + i];
        if (p < 0 || p >= a.P) p = -2;
      }
      wblk[x] = p;
    }
  }
  __syncthreads();
  const int32_t DG = a.D >> 3;
  const int32_t q = tid % a.ps.rg;
  const int32_t h = q / DG;
  const int32_t dg = q - h * DG;
  const int32_t toff = tid / a.ps.rg;
  const int32_t l0 = j * a.lps;
  const int32_t nl = min(a.L, l0 + a.lps) - l0;
  const int32_t n_tok = W > toff ? (W - toff + a.ps.m - 1) / a.ps.m : 0;
  const int32_t total = n_tok * nl;
  const uint16_t* head = a.k + (int64_t)h * a.sH + (int64_t)dg * 8 + (int64_t)l0 * a.sL;
  bool bad_len = false, bad_tab = false;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // item n -> token tau = T - W + toff + (n / nl) * m, layer l0 + n % nl
  for (int32_t n0 = 0; n0 < total; n0 += kUnroll) {
    u32x4 v[kUnroll];
    float wv[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t n = n0 + u;
      const int32_t k = n / nl, li = n - k * nl;
      const int32_t tau = T - W + toff + k * a.ps.m;
      const int32_t i = tau / a.B;
      int64_t p;
      if (staged) {
        p = n < total ? wblk[i - i_first] : -1;
      } else {
        p = (n < total && i < nb_s) ? (int64_t)a.table[b0 + i] : -1;
        if (n < total && i < nb_s && (p < 0 || p >= a.P)) p = -2;
      }
      ok[u] = n < total && p >= 0;
      if (n < total && p == -1) bad_len = true;
      if (n < total && p == -2) bad_tab = true;
      const int64_t pc = ok[u] ? p : 0;
      const int32_t t = tau - i * a.B;
      v[u] = ok[u] ? load16(head + pc * a.sB + (int64_t)t * a.sT + (int64_t)li * a.sL) : u32x4{0u, 0u, 0u, 0u};
      wv[u] = MODE == kGiven ? wsh[(l0 + li) * a.H + h] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (ok[u]) accum8<MODE>(acc, v[u], wv[u]);
  }
  if (bad_len) raise_err(a.err, KKA_DEVERR_SEQ_LEN);
  if (bad_tab) raise_err(a.err, KKA_DEVERR_BLOCK_TABLE);
  stash8(red, tid, acc);
  __syncthreads();
  const float denom = MODE == kGiven ? (float)W : (float)((int64_t)W * LH);
  if (a.n_split == 1) {
    for (int32_t d = tid; d < a.D; d += a.ps.nt)
      a.out[(int64_t)s * a.D + d] = W > 0 ? column_sum(red, a.D, a.ps.nt, d) / denom : 0.f;
    return;
  }
  // layer split: shares' partial sums, added in split order by
  // anchor_finish_kernel or (a.done set) by the work-group that finishes
  // the sequence's last share
  float* part = a.partial + (int64_t)s * a.n_split * a.D;
  if (!a.done) {
    for (int32_t d = tid; d < a.D; d += a.ps.nt) part[(int64_t)j * a.D + d] = column_sum(red, a.D, a.ps.nt, d);
    return;
  }
  for (int32_t d = tid; d < a.D; d += a.ps.nt) store_agent(part + (int64_t)j * a.D + d, column_sum(red, a.D, a.ps.nt, d));
  __shared__ uint32_t last;
  if (!arrive(a.done + s, (uint32_t)a.n_split, a.err, last)) return;
  for (int32_t d = tid; d < a.D; d += a.ps.nt) {
    const float sum = split_sum(part + d, a.n_split, a.D);
    a.out[(int64_t)s * a.D + d] = W > 0 ? sum / denom : 0.f;
  }
}

// Sums each sequence's layer-split partials in split order (loads of a
// batch of 8 splits are issued before the first add).
template <int MODE>
__global__ __launch_bounds__(256) void anchor_finish_kernel(PoolArgs a) {
  const int32_t s = blockIdx.x;
  const int32_t T = a.seq_len[s] > 0 ? a.seq_len[s] : 0;
  const int32_t W = a.window < T ? a.window : T;
  const int32_t LH = a.L * a.H;
  for (int32_t d = threadIdx.x; d < a.D; d += blockDim.x) {
    const float* src = a.partial + (int64_t)s * a.n_split * a.D + d;
    float sum = 0.f;
    for (int32_t j0 = 0; j0 < a.n_split; j0 += 8) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = src[(int64_t)min(j0 + u, a.n_split - 1) * a.D];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < a.n_split) sum += t[u];
    }
    const float denom = MODE == kGiven ? (float)W : (float)((int64_t)W * LH);
    a.out[(int64_t)s * a.D + d] = W > 0 ? sum / denom : 0.f;
  }
}

inline int small_block(int32_t D) { return D >= 256 ? 256 : ((D + 63) / 64) * 64; }

}  // namespace

hipError_t launch_pool(const PoolArgs& a0, int mode, hipStream_t st) {
  PoolArgs a = a0;
  int64_t groups = (int64_t)a.n_items * a.n_split;
  double w[kXcds];
  if (a.n_split == 1 && a.n_items >= kXcdShareMinItems && xcd_weights(w)) {
    a.xs = xcd_shares(a.n_items, w);
    int32_t most = 0;
    for (int x = 0; x < kXcds; ++x) most = a.xs.n[x] > most ? a.xs.n[x] : most;
    groups = (int64_t)kXcds * most;
  }
  const dim3 grid((unsigned)groups);
  const dim3 block((unsigned)a.ps.nt);
  const size_t dyn = mode == kGiven ? sizeof(float) * (size_t)a.L * a.H : 0;
  if (a.n_items > 0) {
    if (a.ps.nt <= 256) {
      if (mode == kGiven) hipLaunchKernelGGL((pool_kernel<kGiven, 256>), grid, block, dyn, st, a);
      else hipLaunchKernelGGL((pool_kernel<kUniform, 256>), grid, block, dyn, st, a);
    } else {
      if (mode == kGiven) hipLaunchKernelGGL((pool_kernel<kGiven, 1024>), grid, block, dyn, st, a);
      else hipLaunchKernelGGL((pool_kernel<kUniform, 1024>), grid, block, dyn, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1 || a.done) return e;
    const dim3 fb((unsigned)small_block(a.D));
    if (mode == kGiven) hipLaunchKernelGGL((pool_finish_kernel<kGiven>), dim3(a.n_items), fb, 0, st, a);
    else hipLaunchKernelGGL((pool_finish_kernel<kUniform>), dim3(a.n_items), fb, 0, st, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_pool_stats(const PoolArgs& a, hipStream_t st) {
  if (a.n_items <= 0) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)a.n_items * a.n_split));
  const dim3 block((unsigned)a.ps.nt);
  // a head's columns reduce inside one wavefront when D/8 is a power of two up to 64
  const int32_t DG = a.D / 8;
  const bool wave = DG <= 64 && (DG & (DG - 1)) == 0;
  if (a.ps.nt <= 256) {
    if (wave) hipLaunchKernelGGL((pool_stats_kernel<256, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((pool_stats_kernel<256, false>), grid, block, 0, st, a);
  } else {
    if (wave) hipLaunchKernelGGL((pool_stats_kernel<1024, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((pool_stats_kernel<1024, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_head_weights(const WeightArgs& w, hipStream_t st) {
  if (w.S <= 0) return hipSuccess;
  hipLaunchKernelGGL(head_var_kernel, dim3((unsigned)((int64_t)w.S * w.LH)), dim3(256), 0, st, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(head_norm_kernel, dim3((unsigned)w.S), dim3(256), 0, st, w);
  return hipGetLastError();
}

hipError_t launch_pool_combine(const PoolArgs& a, const float* wts, const double* csum, hipStream_t st) {
  if (a.n_items <= 0) return hipSuccess;
  // head_dim threads (four lane groups of head_dim / 4), 3 * head_dim * 4 bytes of LDS
  hipLaunchKernelGGL(pool_combine_kernel, dim3((unsigned)a.n_items), dim3((unsigned)a.D),
                     (size_t)3 * a.D * sizeof(float), st, a, wts, csum);
  return hipGetLastError();
}

hipError_t launch_anchor(const PoolArgs& a, hipStream_t st) {
  if (a.S <= 0) return hipSuccess;
  const bool given = a.weights != nullptr;
  const dim3 grid((unsigned)((int64_t)a.S * a.n_split));
  const dim3 block((unsigned)a.ps.nt);
  const size_t dyn = given ? sizeof(float) * (size_t)a.L * a.H : 0;
  if (a.ps.nt <= 256) {
    if (given) hipLaunchKernelGGL((anchor_kernel<kGiven, 256>), grid, block, dyn, st, a);
    else hipLaunchKernelGGL((anchor_kernel<kUniform, 256>), grid, block, dyn, st, a);
  } else {
    if (given) hipLaunchKernelGGL((anchor_kernel<kGiven, 1024>), grid, block, dyn, st, a);
    else hipLaunchKernelGGL((anchor_kernel<kUniform, 1024>), grid, block, dyn, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1 || a.done) return e;
  const dim3 fb((unsigned)small_block(a.D));
  if (given) hipLaunchKernelGGL((anchor_finish_kernel<kGiven>), dim3((unsigned)a.S), fb, 0, st, a);
  else hipLaunchKernelGGL((anchor_finish_kernel<kUniform>), dim3((unsigned)a.S), fb, 0, st, a);
  return hipGetLastError();
}

}  // namespace kka
