// Pool-on-write: block vectors kept current while keys are written.
//
// Page "Key-Key Semantic Affinity: Key vectors replace attention scores for
// KV-cache importance" (10100.com), section 2.2 step 1 and section 5.2
// step 2: v_b is taken from the keys as they leave k_proj and is stored, not
// recomputed each step.  Here a decode step appends one token per sequence:
// one work-group per sequence stores the token's keys (every layer and KV
// head) into its slot of the paged pool, adds their (weighted) sum to the
// open block's running sum and writes the open block's vector, so a step
// touches one token's keys instead of re-reading the whole block.
//
// Threads: q8 = D/8 lanes cover one head_dim row in 16-byte pieces, m rows
// (one row = one (token, layer, head)) are in flight, nt = q8 * m <= 256.
// Rows are walked token-major, then layer, then head; each lane keeps 8
// fp32 partial sums and a fixed-order LDS reduction finishes the group.
#include "kka_internal.h"

namespace kka {
namespace {

constexpr int kWriteThreads = 256;
constexpr int kWriteUnroll = 8;
constexpr int kMaxLH = 4096;
constexpr int kMaxD = 1024;

template <bool GIVEN>
__global__ __launch_bounds__(kWriteThreads) void write_pool_kernel(WriteArgs a) {
  __shared__ float red[kWriteThreads * 8];
  __shared__ float wsh[GIVEN ? kMaxLH : 1];
  const int tid = threadIdx.x;
  const int32_t s = blockIdx.x;
  const int32_t LH = a.L * a.H;
  const int32_t dg = tid % a.q8;
  const int32_t r0 = tid / a.q8;
  const bool active = tid < a.nt;
  // Loads whose addresses depend only on the sequence go first, so they
  // overlap the metadata reads below: the first rows of the new token's
  // keys (a step without seeding reads nothing else) and the running sums.
  const uint16_t* knew = a.k_new ? a.k_new + (int64_t)s * LH * a.D + dg * 8 : nullptr;
  const bool pre_ok = knew && !a.seed && active;
  u32x4 pre[kWriteUnroll];
#pragma unroll
  for (int u = 0; u < kWriteUnroll; ++u) {
    const int32_t rr = r0 + u * a.m < LH ? r0 + u * a.m : min(r0, LH - 1);
    pre[u] = pre_ok ? *reinterpret_cast<const u32x4*>(knew + (int64_t)rr * a.D) : u32x4{0u, 0u, 0u, 0u};
  }
  float rp[kMaxD / kWriteThreads];
#pragma unroll
  for (int i = 0; i < kMaxD / kWriteThreads; ++i) {
    const int32_t d = tid + i * kWriteThreads;
    rp[i] = !a.seed && d < a.D ? a.running[(int64_t)s * a.D + d] : 0.f;
  }
  const int32_t T = a.seq_len[s];
  // every thread takes the same exits, so the barriers below stay uniform
  if (T <= 0) {
    if (T < 0 && tid == 0) raise_err(a.err, KKA_DEVERR_SEQ_LEN);
    return;
  }
  const int32_t t = T - 1;
  const int32_t j = t / a.B;
  const int32_t slot = t - j * a.B;
  const int32_t o0 = a.offs[s];
  if (j >= a.offs[s + 1] - o0) {
    if (tid == 0) raise_err(a.err, KKA_DEVERR_SEQ_LEN);
    return;
  }
  const int64_t b = (int64_t)o0 + j;
  const int64_t p = a.table[b];
  if (p < 0 || p >= a.P) {
    if (tid == 0) raise_err(a.err, KKA_DEVERR_BLOCK_TABLE);
    return;
  }
  int64_t row_out = b;
  if (a.vb_stride > 0) {
    if (j >= a.vb_stride) {
      if (tid == 0) raise_err(a.err, KKA_DEVERR_ROW);
      return;
    }
    row_out = (int64_t)s * a.vb_stride + j;
  }
  if (GIVEN) {
    for (int32_t x = tid; x < LH; x += kWriteThreads) wsh[x] = a.weights[(int64_t)s * LH + x];
    __syncthreads();
  }

  const int32_t t0 = a.seed ? 0 : slot;
  const int32_t n_rows = (slot - t0 + 1) * LH;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (active) {
    uint16_t* kp = a.k + p * a.sB + dg * 8;
    for (int32_t r = r0; r < n_rows; r += kWriteUnroll * a.m) {
      u32x4 v[kWriteUnroll];
      float w[kWriteUnroll];
#pragma unroll
      for (int u = 0; u < kWriteUnroll; ++u) {
        // rows past the end are replaced by this lane's first row (loaded, not added)
        const int32_t rr = r + u * a.m < n_rows ? r + u * a.m : r0;
        const int32_t ti = t0 + rr / LH;
        const int32_t lh = rr - (ti - t0) * LH;
        const int32_t l = lh / a.H;
        const int32_t h = lh - l * a.H;
        uint16_t* dst = kp + (int64_t)l * a.sL + (int64_t)ti * a.sT + (int64_t)h * a.sH;
        if (knew && ti == slot) {
          // the first batch of a step without seeding was loaded at entry
          v[u] = pre_ok && r == r0 ? pre[u] : *reinterpret_cast<const u32x4*>(knew + (int64_t)lh * a.D);
          *reinterpret_cast<u32x4*>(dst) = v[u];  // the cache write (idempotent for repeats)
        } else {
          v[u] = *reinterpret_cast<const u32x4*>(dst);
        }
        w[u] = GIVEN ? wsh[lh] : 1.f;
      }
#pragma unroll
      for (int u = 0; u < kWriteUnroll; ++u) {
        if (r + u * a.m < n_rows) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t x = v[u][c];
            if (GIVEN) {
              acc[2 * c] = fmaf(w[u], bf16_lo(x), acc[2 * c]);
              acc[2 * c + 1] = fmaf(w[u], bf16_hi(x), acc[2 * c + 1]);
            } else {
              acc[2 * c] += bf16_lo(x);
              acc[2 * c + 1] += bf16_hi(x);
            }
          }
        }
      }
    }
    float4* r4 = reinterpret_cast<float4*>(red);
    r4[2 * tid] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    r4[2 * tid + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  __syncthreads();
  const float denom = GIVEN ? (float)(slot + 1) : (float)((int64_t)(slot + 1) * LH);
#pragma unroll
  for (int i = 0; i < kMaxD / kWriteThreads; ++i) {
    const int32_t d = tid + i * kWriteThreads;
    if (d < a.D) {
      // lanes sharing the 16-byte column of d are dg + r * q8, r < m
      const int32_t base = ((d >> 3) << 3) + (d & 7);
      float sum = 0.f;
      for (int32_t r = 0; r < a.m; ++r) sum += red[base + r * a.q8 * 8];
      const float total = (a.seed || slot == 0) ? sum : rp[i] + sum;
      a.running[(int64_t)s * a.D + d] = total;
      a.out[row_out * a.D + d] = total / denom;
    }
  }
}

}  // namespace

hipError_t launch_pool_on_write(const WriteArgs& a, hipStream_t st) {
  if (a.S <= 0) return hipSuccess;
  if (a.weights)
    hipLaunchKernelGGL(write_pool_kernel<true>, dim3((unsigned)a.S), dim3(kWriteThreads), 0, st, a);
  else
    hipLaunchKernelGGL(write_pool_kernel<false>, dim3((unsigned)a.S), dim3(kWriteThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace kka
