// Grid -> Chunk -> Page representations.
//
// Page "Key-Key Semantic Affinity: Key vectors replace attention scores for
// KV-cache importance" (10100.com), section 5.1: a grid's vector is the mean
// of its chunk vectors; chunks are built the same way from their pages.
//
// One work-group per (sequence, grid): it averages the page rows of each of
// the grid's chunks (32 lanes x float4 per 128-wide row, so a row is one
// coalesced 512-byte read; 32 chunks in parallel with 16 row loads in flight
// each), writes the chunk rows, keeps them in LDS and averages them into the
// grid row.  Sums run in fp32 in child order and are divided once by the
// number of present children.  The first rows of each lane's first chunk are
// requested together with the page count: they are that chunk's pages
// whatever the count turns out to be (rows past it are loaded, clamped, and
// not added), so the rows need not wait for the count.
#include "kka_internal.h"

namespace kka {
namespace {

constexpr int kLevelThreads = 1024;

__global__ __launch_bounds__(kLevelThreads) void levels_kernel(LevelArgs a) {
  extern __shared__ float4 cbuf[];  // [cpg][D/4] chunk rows of this grid
  constexpr int kBatch = 16;        // row loads in flight per lane
  const int tid = threadIdx.x;
  const int32_t s = blockIdx.x / a.g_cap;
  const int32_t g = blockIdx.x - s * a.g_cap;
  const int32_t Q = a.D >> 2;  // float4 per row (<= 256)
  const int32_t slots = kLevelThreads / Q;
  const int32_t rs = tid / Q;
  const int32_t x = tid - rs * Q;
  const int32_t c0 = g * a.cpg;
  float4* seq = reinterpret_cast<float4*>(a.lvl + (int64_t)s * a.rows_per_seq * a.D);
  // the page count (a relaxed atomic load keeps its place ahead of the rows)
  // and, in lanes whose first chunk (c0 + rs) belongs to this grid, that
  // chunk's first batch of rows, clamped into the level buffer's pages (the
  // other lanes would read the next grid's pages for nothing)
  const int32_t n_p_v = __hip_atomic_load(a.n_pages + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  float4 v[kBatch];
  if (rs < a.cpg) {
    const int64_t pf = (int64_t)(c0 + rs) * a.ppc;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t r = pf + min(u, a.ppc - 1);
      v[u] = seq[(r < a.max_pages ? r : a.max_pages - 1) * Q + x];
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // the count is read after the rows have gone out
  int32_t n_p = __builtin_amdgcn_readfirstlane(n_p_v);
  if (n_p < 0 || n_p > a.max_pages) {
    if (tid == 0 && g == 0) raise_err(a.err, KKA_DEVERR_PAGES);
    n_p = n_p < 0 ? 0 : a.max_pages;
  }
  const int32_t n_c = (n_p + a.ppc - 1) / a.ppc;
  const int32_t n_g = (n_c + a.cpg - 1) / a.cpg;
  if (g >= n_g) return;
  if (a.first_dirty) {
    int32_t fd = a.first_dirty[s];
    if (fd < 0) fd = 0;
    if (g < (fd / a.ppc) / a.cpg) return;
  }
  const int32_t nch = min(n_c, c0 + a.cpg) - c0;
  // threads past the last whole slot (when D / 4 does not divide the group) take no chunk
  for (int32_t ci = rs; rs < slots && ci < nch; ci += slots) {
    const int32_t c = c0 + ci;
    const int32_t p0 = c * a.ppc;
    const int32_t np_ = min(n_p, p0 + a.ppc) - p0;
    const float4* src = seq + (int64_t)p0 * Q + x;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // pages in order, kBatch row loads in flight (rows past the chunk are
    // loaded, clamped, and not added); the first chunk's first batch is in v
    for (int32_t r0 = 0; r0 < np_; r0 += kBatch) {
      if (ci != rs || r0 != 0) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) v[u] = src[(int64_t)min(r0 + u, np_ - 1) * Q];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (r0 + u < np_) {
          acc.x += v[u].x;
          acc.y += v[u].y;
          acc.z += v[u].z;
          acc.w += v[u].w;
        }
      }
    }
    const float n = (float)np_;
    const float4 m = make_float4(acc.x / n, acc.y / n, acc.z / n, acc.w / n);
    seq[((int64_t)a.max_pages + c) * Q + x] = m;
    cbuf[ci * Q + x] = m;
  }
  __syncthreads();
  for (int32_t y = tid; y < Q; y += kLevelThreads) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int32_t ci = 0; ci < nch; ++ci) {
      const float4 v = cbuf[ci * Q + y];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const float n = (float)nch;
    seq[((int64_t)a.max_pages + a.c_cap + g) * Q + y] = make_float4(acc.x / n, acc.y / n, acc.z / n, acc.w / n);
  }
}

}  // namespace

hipError_t launch_levels(const LevelArgs& a, hipStream_t st) {
  if (a.S <= 0 || a.g_cap <= 0) return hipSuccess;
  const size_t dyn = sizeof(float) * (size_t)a.cpg * a.D;
  hipLaunchKernelGGL(levels_kernel, dim3((unsigned)((int64_t)a.S * a.g_cap)), dim3(kLevelThreads), dyn, st, a);
  return hipGetLastError();
}

}  // namespace kka
