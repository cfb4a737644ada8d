// Grid -> Chunk -> Page representations.
//
// Page "Key-Key Semantic Affinity: Key vectors replace attention scores for
// KV-cache importance" (10100.com), section 5.1: a grid's vector is the mean
// of its chunk vectors; chunks are built the same way from their pages.
//
// One work-group per (sequence, grid): it averages the page rows of each of
// the grid's chunks (32 lanes x float4 per 128-wide row, so a row is one
// coalesced 512-byte read), writes the chunk rows, keeps them in LDS and
// averages them into the grid row.  Sums run in fp32 in child order and are
// divided once by the number of present children.
#include "kka_internal.h"

namespace kka {
namespace {

__global__ __launch_bounds__(256) void levels_kernel(LevelArgs a) {
  extern __shared__ float4 cbuf[];  // [cpg][D/4] chunk rows of this grid
  const int tid = threadIdx.x;
  const int32_t s = blockIdx.x / a.g_cap;
  const int32_t g = blockIdx.x - s * a.g_cap;
  int32_t n_p = a.n_pages[s];
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
  const int32_t Q = a.D >> 2;  // float4 per row
  const int32_t slots = 256 / Q > 0 ? 256 / Q : 1;
  const int32_t rs = tid / Q;
  const int32_t x = tid - rs * Q;
  const int32_t c0 = g * a.cpg;
  const int32_t nch = min(n_c, c0 + a.cpg) - c0;
  float4* seq = reinterpret_cast<float4*>(a.lvl + (int64_t)s * a.rows_per_seq * a.D);
  if (rs < slots && x < Q) {
    for (int32_t ci = rs; ci < nch; ci += slots) {
      const int32_t c = c0 + ci;
      const int32_t p0 = c * a.ppc;
      const int32_t np_ = min(n_p, p0 + a.ppc) - p0;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      const float4* src = seq + (int64_t)p0 * Q + x;
      int32_t r = 0;
      for (; r + 4 <= np_; r += 4) {
        const float4 v0 = src[(int64_t)(r + 0) * Q], v1 = src[(int64_t)(r + 1) * Q];
        const float4 v2 = src[(int64_t)(r + 2) * Q], v3 = src[(int64_t)(r + 3) * Q];
        acc.x += v0.x; acc.y += v0.y; acc.z += v0.z; acc.w += v0.w;
        acc.x += v1.x; acc.y += v1.y; acc.z += v1.z; acc.w += v1.w;
        acc.x += v2.x; acc.y += v2.y; acc.z += v2.z; acc.w += v2.w;
        acc.x += v3.x; acc.y += v3.y; acc.z += v3.z; acc.w += v3.w;
      }
      for (; r < np_; ++r) {
        const float4 v = src[(int64_t)r * Q];
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      const float n = (float)np_;
      const float4 m = make_float4(acc.x / n, acc.y / n, acc.z / n, acc.w / n);
      seq[((int64_t)a.max_pages + c) * Q + x] = m;
      cbuf[ci * Q + x] = m;
    }
  }
  __syncthreads();
  for (int32_t y = tid; y < Q; y += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int32_t ci = 0; ci < nch; ++ci) {
      const float4 v = cbuf[ci * Q + y];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    const float n = (float)nch;
    seq[((int64_t)a.max_pages + a.c_cap + g) * Q + y] = make_float4(acc.x / n, acc.y / n, acc.z / n, acc.w / n);
  }
}

}  // namespace

hipError_t launch_levels(const LevelArgs& a, hipStream_t st) {
  if (a.S <= 0 || a.g_cap <= 0) return hipSuccess;
  const size_t dyn = sizeof(float) * (size_t)a.cpg * a.D;
  hipLaunchKernelGGL(levels_kernel, dim3((unsigned)((int64_t)a.S * a.g_cap)), dim3(256), dyn, st, a);
  return hipGetLastError();
}

}  // namespace kka
