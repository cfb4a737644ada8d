// Attention mass per block for one decode query per sequence, the
// reference the page compares its selection with.
//
// Page "Key-Key Semantic Affinity: Key vectors replace attention scores for
// KV-cache importance" (10100.com), section 3.3: the top-K blocks by real
// attention (QK^T averaged over every layer and head) against the top-K
// blocks by key-key affinity.  For query head hq of layer l (KV head
// h = hq / G, G = Hq / H) the attention is softmax over the sequence's
// tokens of scale * q . k; it is averaged over the L * Hq (layer, query
// head) pairs and summed over each block's tokens.
//
// The keys are streamed once.  A work-group takes one tile (TB logical
// blocks, about 64 tokens) of one sequence in one layer: each lane keeps the
// 8-dim piece of its KV head's G queries in registers (the lane's head and
// piece never change), loads 16 bytes of key per row and reduces the G dot
// products over the D/8 lanes of the row with a DPP butterfly that leaves
// every sum in every lane, so lane g stores logit g with one LDS write per
// row (head_dim and the query group are template parameters, so the
// unrolled loops carry no branches; row indices advance incrementally); the
// logits go to LDS rows padded by one word,
// and one wave per query head turns them into the tile maximum, the tile
// sum and each block's sum of exp(logit - tile max).  A second pass forms
// each (sequence, layer, query head) softmax maximum and normaliser from the
// tile partials and turns each tile maximum into the tile's scale factor; a
// third sums every block's normalised mass over head chunks, a fourth adds
// the chunks in order.  No float atomics: the result
// does not depend on scheduling.  Arithmetic is on the vector ALUs (about 7
// flop per key byte at G = 7, below the fp32 ridge), not on matrix cores.
#include <math.h>

#include "kka_internal.h"

namespace kka {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kChunkHeads = 32;  // (layer, query head) pairs per block-mass chunk
constexpr int kRowUnroll = 8;    // key rows in flight per lane (vector kernel)
constexpr int kMaxTB = 256;      // blocks per vector-kernel tile
#ifndef KKA_ATTN_BUFS
#define KKA_ATTN_BUFS 3
#endif
#ifndef KKA_ATTN_MFMA_TOKENS
#define KKA_ATTN_MFMA_TOKENS 512
#endif
constexpr int kMfmaBufs = KKA_ATTN_BUFS;           // key chunks in flight per wave
constexpr int kMfmaTileTokens = KKA_ATTN_MFMA_TOKENS;  // tokens per matrix-core tile (>= its blocks)

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v, float identity) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over lanes [lane, lane + N) of aligned groups of N lanes (N a power of
// two <= 64), exact in the lane that starts the group; fixed order.
template <int N>
__device__ __forceinline__ float group_sum_t(float v) {
  if constexpr (N >= 2) v += dpp_f<0x101>(v, 0.f);  // row_shl:1
  if constexpr (N >= 4) v += dpp_f<0x102>(v, 0.f);  // row_shl:2
  if constexpr (N >= 8) v += dpp_f<0x104>(v, 0.f);  // row_shl:4
  if constexpr (N >= 16) v += dpp_f<0x108>(v, 0.f);  // row_shl:8
  if constexpr (N >= 32) v += __shfl_down(v, 16);
  if constexpr (N >= 64) v += __shfl_down(v, 32);
  return v;
}

// Sum over aligned groups of N lanes (N a power of two <= 64) delivered to
// every lane of the group: a butterfly of pairwise adds (xor 1 and xor 2
// within quads, the half-row mirror, the row rotation by 8, then across
// rows).  Each step adds the same two values in both partner lanes, and
// float addition is commutative, so all lanes hold bit-identical totals.
template <int N>
__device__ __forceinline__ float group_allsum_t(float v) {
  if constexpr (N >= 2) v += dpp_f<0xB1>(v, 0.f);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v += dpp_f<0x4E>(v, 0.f);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v += dpp_f<0x141>(v, 0.f);  // row_half_mirror
  if constexpr (N >= 16) v += dpp_f<0x128>(v, 0.f);  // row_ror:8
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

// The same butterfly with the maximum.
template <int N>
__device__ __forceinline__ float group_allmax_t(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp_f<0xB1>(v, -INFINITY));
  if constexpr (N >= 4) v = fmaxf(v, dpp_f<0x4E>(v, -INFINITY));
  if constexpr (N >= 8) v = fmaxf(v, dpp_f<0x141>(v, -INFINITY));
  if constexpr (N >= 16) v = fmaxf(v, dpp_f<0x128>(v, -INFINITY));
  if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Group widths known only at run time (uniform; a power of two <= 64).
__device__ __forceinline__ float group_allsum_rt(float v, int32_t n) {
  switch (n) {
    case 1: return v;
    case 2: return group_allsum_t<2>(v);
    case 4: return group_allsum_t<4>(v);
    case 8: return group_allsum_t<8>(v);
    case 16: return group_allsum_t<16>(v);
    case 32: return group_allsum_t<32>(v);
    default: return group_allsum_t<64>(v);
  }
}

__device__ __forceinline__ float group_allmax_rt(float v, int32_t n) {
  switch (n) {
    case 1: return v;
    case 2: return group_allmax_t<2>(v);
    case 4: return group_allmax_t<4>(v);
    case 8: return group_allmax_t<8>(v);
    case 16: return group_allmax_t<16>(v);
    case 32: return group_allmax_t<32>(v);
    default: return group_allmax_t<64>(v);
  }
}

// Whole-wave sum and maximum, returned in every lane: DPP within each row
// of 16 lanes, then the four row results in lane order.
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum_t<16>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0x101>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x102>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x104>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x108>(v, -INFINITY));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// Offsets checked per sequence: 0 <= offs[s] <= offs[s+1] <= total_blocks.
__device__ __forceinline__ int32_t seq_blocks(const AttnArgs& a, int32_t s, bool report) {
  const int32_t o0 = a.offs[s], o1 = a.offs[s + 1];
  if (o0 < 0 || o1 < o0 || o1 > a.total_blocks) {
    if (report) raise_err(a.err, KKA_DEVERR_OFFSETS);
    return 0;
  }
  return o1 - o0;
}

// First tile of every sequence (tile counts capped so the total never
// exceeds the launch bound) and the blocks holding tokens.
__global__ __launch_bounds__(1024) void attn_tiles_kernel(AttnArgs a) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int32_t per = (a.S + 1023) / 1024;
  const int32_t s0 = min(a.S, tid * per), s1 = min(a.S, s0 + per);
  int32_t sum = 0;
  for (int32_t s = s0; s < s1; ++s) sum += (seq_blocks(a, s, false) + a.TB - 1) / a.TB;
  part[tid] = sum;
  __syncthreads();
  // inclusive scan (Hillis-Steele); tile counts are bounded by the block
  // count, so no sum overflows int32
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t add = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int32_t run = min(part[tid] - sum, a.max_tiles);
  if (tid == 1023) a.tile_offs[a.S] = min(part[1023], a.max_tiles);
  for (int32_t s = s0; s < s1; ++s) {
    const int32_t nb = seq_blocks(a, s, true);
    a.tile_offs[s] = run;
    run = min(run + (nb + a.TB - 1) / a.TB, a.max_tiles);
    int32_t T = a.seq_len[s];
    if (T < 0) {
      raise_err(a.err, KKA_DEVERR_SEQ_LEN);
      T = 0;
    }
    int32_t nv = (int32_t)(((int64_t)T + a.B - 1) / a.B);
    if (nv > nb) {
      raise_err(a.err, KKA_DEVERR_SEQ_LEN);
      nv = nb;
    }
    if (nv > a.out_stride) {
      raise_err(a.err, KKA_DEVERR_ROW);
      nv = (int32_t)a.out_stride;
    }
    a.n_blocks[s] = nv;
  }
}

// The tile a work-group of a logits kernel takes: its sequence, first
// block j0 (within the sequence), block count, the sequence's first global
// block o0 and its token count T clamped to its blocks.  valid is false
// for groups past the last tile (the grid is an upper bound) -- the same for
// every thread of the group.
struct Tile {
  bool valid;
  int32_t s, j0, o0, nblk;
  int64_t T;
};

__device__ __forceinline__ Tile find_tile(const AttnArgs& a, int32_t tile) {
  Tile t{};
  t.valid = false;
  if (tile >= a.tile_offs[a.S]) return t;
  int32_t lo = 0, hi = a.S - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (a.tile_offs[mid] <= tile) lo = mid;
    else hi = mid - 1;
  }
  t.s = lo;
  t.j0 = (tile - a.tile_offs[t.s]) * a.TB;
  t.o0 = a.offs[t.s];
  const int32_t nb_s = seq_blocks(a, t.s, false);
  t.nblk = min(a.TB, nb_s - t.j0);
  t.T = min((int64_t)max(a.seq_len[t.s], 0), (int64_t)nb_s * a.B);
  t.valid = t.nblk > 0;
  return t;
}

// Physical block of each of the tile's blocks into phys[] (-1 if invalid;
// raises the flag once, from the first layer).
__device__ __forceinline__ void load_tile_table(const AttnArgs& a, const Tile& t, int32_t l, int64_t* phys) {
  for (int32_t jb = threadIdx.x; jb < t.nblk; jb += kAttnThreads) {
    const int64_t p = a.table[t.o0 + t.j0 + jb];
    const bool ok = p >= 0 && p < a.P;
    if (!ok && l == 0) raise_err(a.err, KKA_DEVERR_BLOCK_TABLE);
    phys[jb] = ok ? p : -1;
  }
}

// Q8 = head_dim / 8 lanes per key row; GQ = query heads per KV head.
template <int Q8, int GQ>
__global__ __launch_bounds__(kAttnThreads) void attn_logits_kernel(AttnArgs a) {
  extern __shared__ float lg[];      // [Hq][TT + 1] logits of this tile (padded rows)
  __shared__ int64_t phys[kMaxTB];   // physical block of each tile block, -1 if invalid
  const int tid = threadIdx.x;
  const int32_t tile = blockIdx.x;
  const int32_t l = blockIdx.y;
  const Tile tt = find_tile(a, tile);
  if (!tt.valid) return;  // uniform over the group
  const int32_t s = tt.s, j0 = tt.j0, o0 = tt.o0, nblk = tt.nblk;
  const int64_t T = tt.T;

  constexpr int kSlots = kAttnThreads / Q8;
  const int32_t m = (kSlots / a.H) * a.H;  // rows in flight, a multiple of H
  const int32_t slot = tid / Q8;
  const int32_t dg = tid % Q8;
  const int32_t h = slot % a.H;  // fixed: rows advance by m
  const int32_t ldw = a.TT + 1;   // LDS row stride: the rows of one wave's heads fall in distinct banks
  // this lane's query pieces, loaded before the table wait so both overlap
  float qr[GQ][8];
  {
    const float* qb = a.q + (((int64_t)s * a.L + l) * a.Hq + (int64_t)h * a.G) * a.D + dg * 8;
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
      if (slot < m) {
        x0 = *reinterpret_cast<const float4*>(qb + (int64_t)g * a.D);
        x1 = *reinterpret_cast<const float4*>(qb + (int64_t)g * a.D + 4);
      }
      qr[g][0] = x0.x; qr[g][1] = x0.y; qr[g][2] = x0.z; qr[g][3] = x0.w;
      qr[g][4] = x1.x; qr[g][5] = x1.y; qr[g][6] = x1.z; qr[g][7] = x1.w;
    }
  }
  load_tile_table(a, tt, l, phys);
  __syncthreads();

  if (slot < m) {
    const uint16_t* kh = a.k + (int64_t)l * a.sL + (int64_t)h * a.sH + dg * 8;
    float* lrow = lg + h * GQ * ldw;
    const int32_t ntok = nblk * a.B;
    // row cursor: token tl (block jb, slot st) advances by dtl tokens a step
    const int32_t dtl = m / a.H;
    const int32_t dq = dtl / a.B, dr = dtl - (dtl / a.B) * a.B;
    int32_t tl = slot / a.H;
    int32_t jb = tl / a.B, st = tl - (tl / a.B) * a.B;
    const int32_t n_it = ((ntok + dtl - 1) / dtl + kRowUnroll - 1) / kRowUnroll;  // uniform

    u32x4 va[kRowUnroll];
    bool oka[kRowUnroll];
    int32_t ta[kRowUnroll];
    // Issues one batch of row loads.  A row outside the tile loads the
    // tile's first row (in bounds) and is never stored.
    auto issue = [&](u32x4 (&v)[kRowUnroll], bool (&ok)[kRowUnroll], int32_t (&t)[kRowUnroll]) {
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const bool in_tile = tl < ntok;
        const int32_t jbc = in_tile ? jb : 0, stc = in_tile ? st : 0;
        const int64_t p = phys[jbc];
        ok[u] = p >= 0 && (int64_t)(j0 + jbc) * a.B + stc < T;
        t[u] = in_tile ? tl : -1;
        v[u] = *reinterpret_cast<const u32x4*>(kh + (p >= 0 ? p : 0) * a.sB + (int64_t)stc * a.sT);
        tl += dtl;
        st += dr;
        jb += dq;
        if (st >= a.B) {
          st -= a.B;
          ++jb;
        }
      }
    };
    // Dot products of one batch with the G queries, reduced over the row's
    // lanes; the row's first lane stores the logits.
    auto compute = [&](const u32x4 (&v)[kRowUnroll], const bool (&ok)[kRowUnroll], const int32_t (&t)[kRowUnroll]) {
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        float x[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[2 * c] = bf16_lo(v[u][c]);
          x[2 * c + 1] = bf16_hi(v[u][c]);
        }
        float d[GQ];
#pragma unroll
        for (int g = 0; g < GQ; ++g) {
          d[g] = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) d[g] = fmaf(x[i], qr[g][i], d[g]);
        }
        // every lane of the row gets all G sums; lane dg stores logits
        // dg, dg + Q8, ... (one write per row when the row has >= G lanes)
#pragma unroll
        for (int g = 0; g < GQ; ++g) d[g] = group_allsum_t<Q8>(d[g]);
#pragma unroll
        for (int g0 = 0; g0 < GQ; g0 += Q8) {
          float mine = 0.f;
#pragma unroll
          for (int g = g0; g < GQ && g < g0 + Q8; ++g) mine = dg == g - g0 ? d[g] : mine;
          if (g0 + dg < GQ && t[u] >= 0) lrow[(g0 + dg) * ldw + t[u]] = ok[u] ? mine * a.scale : -INFINITY;
        }
      }
    };
    for (int32_t it = 0; it < n_it; ++it) {
      issue(va, oka, ta);
      compute(va, oka, ta);
    }
  }
  __syncthreads();

  // one wave per query head: each block's maximum logit and its sum of
  // exp(logit - maximum) (a unit is a block on this path)
  const int wave = tid >> 6, lane = tid & 63;
  const int32_t ntok = nblk * a.B;
  // tiles of whole 64-token segments whose blocks tile each segment: block
  // j of segment i = lanes [j*B, (j+1)*B) of token index 64 i + lane
  const bool aligned = a.TT % 64 == 0 && 64 % a.B == 0;
  const int32_t nseg = a.TT / 64;
  const int64_t nunits = (int64_t)a.total_blocks * a.UPB;
  for (int32_t hq = wave; hq < a.Hq; hq += kAttnThreads / 64) {
    const float* row = lg + hq * ldw;
    const int64_t base = ((int64_t)l * a.Hq + hq) * nunits + o0 + j0;
    if (aligned) {
      for (int32_t i = 0; i < nseg; ++i) {
        const int32_t t = 64 * i + lane;
        const float x = t < ntok ? row[t] : -INFINITY;
        const float gm = group_allmax_rt(x, a.B);
        const float ex = x == -INFINITY ? 0.f : expf(x - gm);
        const float gs = group_allsum_rt(ex, a.B);
        if (lane % a.B == 0 && t < ntok) {
          a.um[base + t / a.B] = gm;
          a.ue[base + t / a.B] = gs;
        }
      }
    } else {
      for (int32_t jb = 0; jb < nblk; ++jb) {
        float xm = -INFINITY;
        for (int32_t t = jb * a.B + lane; t < (jb + 1) * a.B; t += 64) xm = fmaxf(xm, row[t]);
        const float gm = wave_max(xm);
        float e = 0.f;
        for (int32_t t = jb * a.B + lane; t < (jb + 1) * a.B; t += 64) {
          const float x = row[t];
          e += x == -INFINITY ? 0.f : expf(x - gm);
        }
        e = wave_sum(e);
        if (lane == 0) {
          a.um[base + jb] = gm;
          a.ue[base + jb] = e;
        }
      }
    }
  }
}

// ------------------------------------------------------------ matrix-core logits

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Round to nearest even bf16 (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Eight fp32 values as three bf16 vectors whose sum equals them to about
// 2^-24 relative: each part is the bf16 rounding of what the earlier parts
// left (every remainder is exact in fp32).  A bf16 part times a bf16 key is
// exact in fp32, so the three products carry fp32 accuracy into the
// matrix cores' fp32 accumulation.
__device__ __forceinline__ void split3(const float (&x)[8], bf16x8& p1, bf16x8& p2, bf16x8& p3) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h1 = bf16_bits_rne(x[i]);
    const float r1 = x[i] - __uint_as_float(h1 << 16);
    const uint32_t h2 = bf16_bits_rne(r1);
    const float r2 = r1 - __uint_as_float(h2 << 16);
    const uint32_t h3 = bf16_bits_rne(r2);
    p1[i] = __builtin_bit_cast(__bf16, (uint16_t)h1);
    p2[i] = __builtin_bit_cast(__bf16, (uint16_t)h2);
    p3[i] = __builtin_bit_cast(__bf16, (uint16_t)h3);
  }
}

// KS = head_dim / 32.  A wave takes one KV head at a time and 16-token
// chunks of the tile: v_mfma_f32_16x16x32_bf16 with the head's (up to 16)
// queries as A (lane l: query l % 16, dims 8 (l / 16) + 32 ks) and the
// chunk's keys as B (lane l: token l % 16, the same dims), so each lane
// loads 16 bytes of key per k-step; the result gives lane l the logits of
// queries 4 (l / 16) + r for token l % 16.  Units of U <= 16 tokens are
// aligned lane groups of a 16-lane row, reduced with DPP butterflies.
template <int KS, int U>
__global__ __launch_bounds__(kAttnThreads) void attn_mfma_kernel(AttnArgs a) {
  __shared__ int64_t phys[kMfmaTileTokens];  // physical block of each tile block, -1 if invalid
  const int tid = threadIdx.x;
  const int32_t tile = blockIdx.x;
  const int32_t l = blockIdx.y;
  const Tile tt = find_tile(a, tile);
  if (!tt.valid) return;  // uniform over the group
  const int32_t s = tt.s, j0 = tt.j0, o0 = tt.o0, nblk = tt.nblk;
  const int64_t T = tt.T;
  load_tile_table(a, tt, l, phys);
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const int32_t n = lane & 15, quad = lane >> 4;
  const int32_t wph = a.H >= 4 ? 1 : 4 / a.H;  // waves per head
  const int32_t hstep = 4 / wph;
  const int32_t ntok = nblk * a.B;
  const int32_t nch = (ntok + 15) / 16;
  const int64_t nunits = (int64_t)a.total_blocks * a.UPB;
  const int64_t unit0 = ((int64_t)o0 + j0) * a.UPB;
  for (int32_t h = wave / wph; h < a.H; h += hstep) {
    bf16x8 q1[KS], q2[KS], q3[KS];
    {
      const bool qrow = n < a.G;
      const float* qb =
          a.q + (((int64_t)s * a.L + l) * a.Hq + (int64_t)h * a.G + (qrow ? n : 0)) * a.D + 8 * quad;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float x[8];
        float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
        if (qrow) {
          x0 = *reinterpret_cast<const float4*>(qb + 32 * ks);
          x1 = *reinterpret_cast<const float4*>(qb + 32 * ks + 4);
        }
        x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
        x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
        split3(x, q1[ks], q2[ks], q3[ks]);
      }
    }
    const uint16_t* kh = a.k + (int64_t)l * a.sL + (int64_t)h * a.sH + 8 * quad;
    // Issues the key loads of chunk c (all of them before any use).  A key
    // column outside the tile loads the tile's first row and is masked.
    auto load = [&](int32_t c, bf16x8 (&kv)[KS], bool& ok, int32_t& tl) {
      tl = 16 * c + n;
      const bool in_tile = tl < ntok;
      const int32_t jb = in_tile ? tl / a.B : 0;
      const int32_t st = in_tile ? tl - jb * a.B : 0;
      const int64_t p = phys[jb];
      ok = in_tile && p >= 0 && (int64_t)(j0 + jb) * a.B + st < T;
      if (!in_tile) tl = -1;
      const uint16_t* kr = kh + (p >= 0 ? p : 0) * a.sB + (int64_t)st * a.sT;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kv[ks] = *reinterpret_cast<const bf16x8*>(kr + 32 * ks);
    };
    // Logits of one chunk on the matrix cores, then each unit's maximum
    // and exp sum from the accumulator lanes.
    auto process = [&](const bf16x8 (&kv)[KS], bool ok, int32_t tl) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q1[ks], kv[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q2[ks], kv[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q3[ks], kv[ks], acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int32_t m = 4 * quad + r;  // query within the head's group
        const float x = ok && m < a.G ? acc[r] * a.scale : -INFINITY;
        const float gm = group_allmax_t<U>(x);
        const float ex = x == -INFINITY ? 0.f : expf(x - gm);
        const float gs = group_allsum_t<U>(ex);
        if (m < a.G && tl >= 0 && n % U == 0) {
          const int64_t at = ((int64_t)l * a.Hq + (int64_t)h * a.G + m) * nunits + unit0 + tl / U;
          a.um[at] = gm;
          a.ue[at] = gs;
        }
      }
    };
    // kMfmaBufs chunks in flight: while one computes, the next ones load
    bf16x8 kbuf[kMfmaBufs][KS];
    bool okb[kMfmaBufs];
    int32_t tlb[kMfmaBufs];
    const int32_t c0 = wave % wph;
#pragma unroll
    for (int b = 0; b < kMfmaBufs - 1; ++b) {
      okb[b] = false;
      tlb[b] = -1;
      if (c0 + b * wph < nch) load(c0 + b * wph, kbuf[b], okb[b], tlb[b]);
    }
    for (int32_t c = c0; c < nch; c += kMfmaBufs * wph) {
#pragma unroll
      for (int b = 0; b < kMfmaBufs; ++b) {
        const int32_t cc = c + b * wph;
        if (cc < nch) {
          const int32_t cn = cc + (kMfmaBufs - 1) * wph;
          const int bn = (b + kMfmaBufs - 1) % kMfmaBufs;
          if (cn < nch) load(cn, kbuf[bn], okb[bn], tlb[bn]);
          __builtin_amdgcn_sched_barrier(0);
          process(kbuf[b], okb[b], tlb[b]);
        }
      }
    }
  }
}

// Softmax maximum and normaliser of one (sequence, layer, query head) over
// its units: M = max of the unit maxima, Z = sum of unit sums rescaled to M.
__global__ __launch_bounds__(kAttnThreads) void attn_norm_kernel(AttnArgs a) {
  __shared__ float red[kAttnThreads / 64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int32_t LHq = a.L * a.Hq;
  const int64_t pair = blockIdx.x;
  const int32_t s = (int32_t)(pair / LHq);
  const int32_t lhq = (int32_t)(pair - (int64_t)s * LHq);
  const int64_t nu = (int64_t)seq_blocks(a, s, false) * a.UPB;
  const int64_t u0 = nu > 0 ? (int64_t)a.offs[s] * a.UPB : 0;
  const int64_t nunits = (int64_t)a.total_blocks * a.UPB;
  const float* um = a.um + (int64_t)lhq * nunits + u0;
  const float* ue = a.ue + (int64_t)lhq * nunits + u0;
  constexpr int U = 8;
  float mx = -INFINITY;
  for (int64_t i = tid; i < nu; i += (int64_t)U * kAttnThreads) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = i + u * kAttnThreads < nu ? um[i + u * kAttnThreads] : -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) mx = fmaxf(mx, v[u]);
  }
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float z = 0.f;
  if (mx != -INFINITY) {
    for (int64_t i = tid; i < nu; i += (int64_t)U * kAttnThreads) {
      float mv[U], ev[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool in = i + u * kAttnThreads < nu;
        const int64_t iu = in ? i + u * kAttnThreads : i;
        mv[u] = in ? um[iu] : -INFINITY;
        ev[u] = ue[iu];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) z += mv[u] == -INFINITY ? 0.f : ev[u] * expf(mv[u] - mx);
    }
  }
  z = wave_sum(z);
  if (lane == 0) red[wave] = z;
  __syncthreads();
  if (tid == 0) {
    a.M[pair] = mx;
    a.Z[pair] = (red[0] + red[1]) + (red[2] + red[3]);
  }
}

// Normalised mass of every block over one chunk of (layer, query head)
// pairs: the sum over its units of unit sum * exp(unit max - M) / Z.
__global__ __launch_bounds__(kAttnThreads) void attn_mass_kernel(AttnArgs a) {
  const int64_t b = (int64_t)blockIdx.x * kAttnThreads + threadIdx.x;
  const int32_t c = blockIdx.y;
  if (b >= a.total_blocks) return;
  const int32_t s = find_seq(a.offs, a.S, (int32_t)b);
  const int32_t j = (int32_t)b - a.offs[s];
  bool ok = j >= 0 && j < a.n_blocks[s];
  const int32_t tile = ok ? a.tile_offs[s] + j / a.TB : 0;
  ok = ok && tile < a.tile_offs[s + 1];  // the tile was computed
  float mass = 0.f;
  if (ok) {
    const int32_t LHq = a.L * a.Hq;
    const int32_t h0 = c * kChunkHeads;
    const int32_t nh = min(LHq, h0 + kChunkHeads) - h0;
    const int64_t nunits = (int64_t)a.total_blocks * a.UPB;
    constexpr int V = 8;  // (layer, query head) pairs whose loads are in flight together
    for (int32_t i = 0; i < nh; i += V) {
      float z[V], M[V];
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const int64_t at = (int64_t)s * LHq + h0 + min(i + u, nh - 1);
        z[u] = a.Z[at];
        M[u] = a.M[at];
      }
      for (int32_t v = 0; v < a.UPB; ++v) {
        float m[V], e[V];
#pragma unroll
        for (int u = 0; u < V; ++u) {
          const int64_t at = (int64_t)(h0 + min(i + u, nh - 1)) * nunits + b * a.UPB + v;
          m[u] = a.um[at];
          e[u] = a.ue[at];
        }
#pragma unroll
        for (int u = 0; u < V; ++u)
          if (i + u < nh && z[u] > 0.f && m[u] != -INFINITY) mass += e[u] * expf(m[u] - M[u]) / z[u];
      }
    }
  }
  a.partial[(int64_t)c * a.total_blocks + b] = mass;
}

// Block score = sum of the chunk masses in chunk order / (L * Hq).
__global__ __launch_bounds__(kAttnThreads) void attn_finish_kernel(AttnArgs a) {
  const int64_t b = (int64_t)blockIdx.x * kAttnThreads + threadIdx.x;
  if (b >= a.total_blocks) return;
  const int32_t s = find_seq(a.offs, a.S, (int32_t)b);
  const int32_t j = (int32_t)b - a.offs[s];
  if (j < 0 || j >= a.out_stride || (int64_t)a.offs[s] + j >= a.offs[s + 1]) return;
  float sum = 0.f;
  if (j < a.n_blocks[s]) {
    constexpr int V = 8;
    for (int32_t c = 0; c < a.n_chunks; c += V) {
      float pv[V];
#pragma unroll
      for (int u = 0; u < V; ++u) pv[u] = a.partial[(int64_t)min(c + u, a.n_chunks - 1) * a.total_blocks + b];
#pragma unroll
      for (int u = 0; u < V; ++u)
        if (c + u < a.n_chunks) sum += pv[u];
    }
  }
  a.out[(int64_t)s * a.out_stride + j] = sum / (float)(a.L * a.Hq);
}

template <int KS>
hipError_t launch_mfma_ks(const AttnArgs& a, dim3 grid, hipStream_t st) {
  switch (a.U) {
    case 1: hipLaunchKernelGGL((attn_mfma_kernel<KS, 1>), grid, dim3(kAttnThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((attn_mfma_kernel<KS, 2>), grid, dim3(kAttnThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL((attn_mfma_kernel<KS, 4>), grid, dim3(kAttnThreads), 0, st, a); break;
    case 8: hipLaunchKernelGGL((attn_mfma_kernel<KS, 8>), grid, dim3(kAttnThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((attn_mfma_kernel<KS, 16>), grid, dim3(kAttnThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

template <int Q8>
hipError_t launch_logits_q8(const AttnArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  switch (a.G) {
    case 1: hipLaunchKernelGGL((attn_logits_kernel<Q8, 1>), grid, dim3(kAttnThreads), lds, st, a); break;
    case 2: hipLaunchKernelGGL((attn_logits_kernel<Q8, 2>), grid, dim3(kAttnThreads), lds, st, a); break;
    case 3: hipLaunchKernelGGL((attn_logits_kernel<Q8, 3>), grid, dim3(kAttnThreads), lds, st, a); break;
    case 4: hipLaunchKernelGGL((attn_logits_kernel<Q8, 4>), grid, dim3(kAttnThreads), lds, st, a); break;
    case 5: hipLaunchKernelGGL((attn_logits_kernel<Q8, 5>), grid, dim3(kAttnThreads), lds, st, a); break;
    case 6: hipLaunchKernelGGL((attn_logits_kernel<Q8, 6>), grid, dim3(kAttnThreads), lds, st, a); break;
    case 7: hipLaunchKernelGGL((attn_logits_kernel<Q8, 7>), grid, dim3(kAttnThreads), lds, st, a); break;
    default: hipLaunchKernelGGL((attn_logits_kernel<Q8, 8>), grid, dim3(kAttnThreads), lds, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_blocks(const AttnArgs& a, hipStream_t st) {
  if (a.S <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_tiles_kernel, dim3(1), dim3(1024), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.total_blocks <= 0) return e;
  const dim3 grid((unsigned)a.max_tiles, (unsigned)a.L);
  if (a.mfma) {
    switch (a.D >> 5) {
      case 1: e = launch_mfma_ks<1>(a, grid, st); break;
      case 2: e = launch_mfma_ks<2>(a, grid, st); break;
      case 4: e = launch_mfma_ks<4>(a, grid, st); break;
      default: e = launch_mfma_ks<8>(a, grid, st); break;
    }
  } else {
  const size_t lds = sizeof(float) * (size_t)a.Hq * (a.TT + 1);
  switch (a.D >> 3) {
    case 1: e = launch_logits_q8<1>(a, grid, lds, st); break;
    case 2: e = launch_logits_q8<2>(a, grid, lds, st); break;
    case 4: e = launch_logits_q8<4>(a, grid, lds, st); break;
    case 8: e = launch_logits_q8<8>(a, grid, lds, st); break;
    case 16: e = launch_logits_q8<16>(a, grid, lds, st); break;
    case 32: e = launch_logits_q8<32>(a, grid, lds, st); break;
    default: e = launch_logits_q8<64>(a, grid, lds, st); break;
  }
  }
  if (e != hipSuccess) return e;
  const int64_t pairs = (int64_t)a.S * a.L * a.Hq;
  hipLaunchKernelGGL(attn_norm_kernel, dim3((unsigned)pairs), dim3(kAttnThreads), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned nbx = (unsigned)((a.total_blocks + kAttnThreads - 1) / kAttnThreads);
  hipLaunchKernelGGL(attn_mass_kernel, dim3(nbx, (unsigned)a.n_chunks), dim3(kAttnThreads), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(attn_finish_kernel, dim3(nbx), dim3(kAttnThreads), 0, st, a);
  return hipGetLastError();
}

int32_t attention_chunk_heads() { return kChunkHeads; }

bool attention_mfma_ok(int32_t D, int32_t G, int32_t B) {
  return (D == 32 || D == 64 || D == 128 || D == 256) && G >= 1 && G <= 16 && (16 % B == 0 || B % 16 == 0);
}

// Blocks per tile: about 256 tokens, whole 64-token segments when the block
// size divides 64, and the tile's logits (H * G rows of tokens + 1 floats)
// within 60 KB of LDS.  0 when even one block does not fit.
int32_t attention_tile_blocks(int32_t B, int32_t H, int32_t G, bool mfma) {
  if (mfma) return B >= kMfmaTileTokens ? 1 : kMfmaTileTokens / B;  // logits stay in registers
  const int64_t cap = 15360 / ((int64_t)H * G) - 1;  // tokens
  if (64 % B == 0) {
    int64_t tt = 256;
    while (tt > 64 && tt > cap) tt >>= 1;
    if (tt <= cap) return (int32_t)(tt / B);
  }
  int64_t tb = B >= 256 ? 1 : 256 / B;
  while (tb > 1 && tb * B > cap) --tb;
  return tb * B <= cap ? (int32_t)tb : 0;
}

}  // namespace kka
