// C ABI of libkka: argument validation, workspace sizing, launch set-up.
// Every check here runs on the host before anything is enqueued, so a
// rejected call has no effect on the device.
#include <mutex>

#include <cmath>
#include <cstdlib>
#include <cstring>

#include "kka_internal.h"

namespace kka {

bool handoff_disabled() {
  const char* v = std::getenv("KKA_NO_HANDOFF");
  return v && v[0] == '1';
}

bool xcd_weights(double (&w)[kXcds]) {
  const char* v = std::getenv("KKA_XCD_WEIGHTS");
  if (v && v[0] != '\0') {
    if (std::strcmp(v, "off") == 0) return false;
    const char* p = v;
    int x = 0;
    for (; x < kXcds; ++x) {
      char* end = nullptr;
      const double d = std::strtod(p, &end);
      if (end == p || !(d > 0.0) || !(d < 1e6)) break;
      w[x] = d;
      p = end;
      if (x + 1 < kXcds) {
        if (*p != ',') break;
        ++p;
      }
    }
    if (x == kXcds && *p == '\0') return true;
    // anything else is not a list of eight weights: the default below
  }
  if (device_cus() != 256) return false;
  for (int x = 0; x < kXcds; ++x) w[x] = x % 2 == 0 ? 1.1 : 1.0;
  return true;
}

// Per-device flag word for errors that only device-resident data reveals.
__device__ uint32_t g_device_error;

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_err_mu;
uint32_t* g_err_ptr[kMaxDevices] = {};

uint32_t* device_error_word() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_err_mu);
  if (!g_err_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_device_error)) != hipSuccess) return nullptr;
    g_err_ptr[dev] = static_cast<uint32_t*>(p);
  }
  return g_err_ptr[dev];
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Scoring workspace head: one tile counter per sequence.
inline size_t score_counter_bytes(int32_t S) { return S > 0 ? align256((size_t)S * sizeof(uint32_t)) : 0; }

kka_status check_kpool(const kka_kpool* kp) {
  if (!kp || !kp->k) return KKA_ERR_NULL;
  if (kp->num_layers < 1 || kp->num_kv_heads < 1 || kp->block_size < 1 || kp->num_phys_blocks < 1)
    return KKA_ERR_SHAPE;
  const int32_t D = kp->head_dim;
  if (D < 8 || D > 1024 || D % 8 != 0) return KKA_ERR_SHAPE;
  if ((int64_t)kp->num_kv_heads * (D / 8) > kMaxPoolThreads) return KKA_ERR_SHAPE;
  if ((int64_t)kp->num_layers * kp->num_kv_heads > 4096) return KKA_ERR_SHAPE;
  if (kp->stride_layer < 0 || kp->stride_block < 0 || kp->stride_token < 0 || kp->stride_head < 0)
    return KKA_ERR_SHAPE;
  if (kp->stride_layer % 8 || kp->stride_block % 8 || kp->stride_token % 8 || kp->stride_head % 8)
    return KKA_ERR_ALIGN;
  if (!aligned16(kp->k)) return KKA_ERR_ALIGN;
  return KKA_OK;
}

kka_status check_seqs(const kka_seqs* sq) {
  if (!sq) return KKA_ERR_NULL;
  if (sq->num_seqs < 0 || sq->total_blocks < 0) return KKA_ERR_SHAPE;
  if (sq->num_seqs > 0 && (!sq->seq_len || !sq->block_offsets)) return KKA_ERR_NULL;
  if (sq->total_blocks > 0 && !sq->block_table) return KKA_ERR_NULL;
  if (sq->num_seqs == 0 && sq->total_blocks > 0) return KKA_ERR_SHAPE;
  return KKA_OK;
}

// Key bytes of one layer of one pooled block (full block): what one layer
// of a split share reads.
inline int64_t pool_layer_bytes(const kka_kpool* kp) {
  return (int64_t)kp->block_size * kp->num_kv_heads * kp->head_dim * 2;
}

// Byte layout of the pooling workspace: layer-split pooling keeps one
// arrival counter per item, then each (item, split)'s partial sums; variance
// pooling keeps per-(block, layer, head) sums, sums of squares and fp64
// per-(sequence, head) variances.
struct PoolWs {
  size_t counters = 0, partial = 0, q = 0, var = 0, csum = 0, total = 0;
};

PoolWs pool_ws(const kka_kpool* kp, const kka_seqs* sq, int64_t items, int32_t mode) {
  PoolWs w;
  const size_t D = (size_t)kp->head_dim, LH = (size_t)kp->num_layers * kp->num_kv_heads;
  if (mode == KKA_WEIGHT_VARIANCE) {
    const size_t tb = (size_t)sq->total_blocks;
    w.partial = align256(tb * LH * D * sizeof(float));
    w.q = align256(tb * LH * sizeof(double));
    w.var = align256((size_t)sq->num_seqs * LH * sizeof(double));
    w.csum = align256((size_t)sq->num_seqs * D * sizeof(double));
  } else {
    const LayerSplit ls = layer_split(items, kp->num_layers, pool_layer_bytes(kp));
    if (ls.n_split > 1) {
      w.counters = align256((size_t)items * sizeof(uint32_t));
      w.partial = align256((size_t)items * ls.n_split * D * sizeof(float));
    }
  }
  w.total = w.counters + w.partial + w.q + w.var + w.csum;
  return w;
}

void fill_pool_args(PoolArgs& a, const kka_kpool* kp, const kka_seqs* sq) {
  a.k = kp->k;
  a.sL = kp->stride_layer;
  a.sB = kp->stride_block;
  a.sT = kp->stride_token;
  a.sH = kp->stride_head;
  a.L = kp->num_layers;
  a.H = kp->num_kv_heads;
  a.D = kp->head_dim;
  a.B = kp->block_size;
  a.P = kp->num_phys_blocks;
  a.S = sq->num_seqs;
  a.total_blocks = sq->total_blocks;
  a.seq_len = sq->seq_len;
  a.offs = sq->block_offsets;
  a.table = sq->block_table;
  a.ps = pool_shape(a.H, a.D);
}

struct LevelGeom {
  int64_t rows;
  int32_t c_cap, g_cap;
};

bool level_geom(const kka_level_layout* lay, LevelGeom& g) {
  if (!lay) return false;
  // at most 2^30 page rows per sequence, also once rounded up to whole
  // chunks, so row and candidate counters stay far from int32 overflow
  if (lay->num_seqs < 0 || lay->max_pages < 0 || lay->max_pages > kMaxPagesPerSeq) return false;
  const int32_t D = lay->head_dim;
  if (D < 8 || D > 1024 || D % 8 != 0) return false;
  g.c_cap = g.g_cap = 0;
  if (lay->hierarchical) {
    if (lay->pages_per_chunk < 1 || lay->chunks_per_grid < 1) return false;
    const int64_t c = ((int64_t)lay->max_pages + lay->pages_per_chunk - 1) / lay->pages_per_chunk;
    if (c > kMaxParents || c * lay->pages_per_chunk > kMaxPagesPerSeq) return false;
    if ((int64_t)lay->chunks_per_grid * D > kMaxGridFloats) return false;
    g.c_cap = (int32_t)c;
    g.g_cap = (int32_t)((c + lay->chunks_per_grid - 1) / lay->chunks_per_grid);
  }
  g.rows = (int64_t)lay->max_pages + g.c_cap + g.g_cap;
  return true;
}

inline kka_status launched(hipError_t e) { return e == hipSuccess ? KKA_OK : KKA_ERR_DEVICE; }

// KKA_SCORE_TWO_LAUNCH=1 in the environment sends every scoring call to the
// two-launch path (scoring launch, then selection launch; same results).
inline bool two_launch_forced() {
  const char* force = std::getenv("KKA_SCORE_TWO_LAUNCH");
  return force && force[0] == '1';
}

// Whether the levels of this layout and these k fit the small selector of
// the one-launch path for large batches.
inline bool small_levels(const kka_level_layout* lay, const LevelGeom& g, const kka_select* sel) {
  const bool h = lay->hierarchical != 0;
  return small_select_fits(h, lay->max_pages, g.c_cap, g.g_cap, h ? lay->pages_per_chunk : 1,
                           h ? lay->chunks_per_grid : 1, h ? sel->k_grid : 0, h ? sel->k_chunk : 0, sel->k_page);
}

}  // namespace
}  // namespace kka

using namespace kka;

extern "C" {

size_t kka_pool_blocks_workspace(const kka_kpool* kp, const kka_seqs* seqs, const int32_t* blocks,
                                 int32_t num_blocks, int32_t mode) {
  if (check_kpool(kp) != KKA_OK || check_seqs(seqs) != KKA_OK) return 0;
  const int64_t items = blocks ? (num_blocks > 0 ? num_blocks : 0) : seqs->total_blocks;
  return pool_ws(kp, seqs, items, mode).total;
}

kka_status kka_pool_blocks(const kka_kpool* kp, const kka_seqs* seqs, const int32_t* blocks, int32_t num_blocks,
                           int32_t mode, float* head_weight, float* vb_out, int64_t vb_seq_stride, void* workspace,
                           size_t workspace_bytes, void* stream) {
  kka_status st = check_kpool(kp);
  if (st != KKA_OK) return st;
  if ((st = check_seqs(seqs)) != KKA_OK) return st;
  if (mode != KKA_WEIGHT_UNIFORM && mode != KKA_WEIGHT_VARIANCE && mode != KKA_WEIGHT_GIVEN) return KKA_ERR_SHAPE;
  if (blocks && num_blocks < 0) return KKA_ERR_SHAPE;
  if (blocks && num_blocks > 0 && seqs->total_blocks == 0) return KKA_ERR_SHAPE;
  if (mode == KKA_WEIGHT_VARIANCE && blocks) return KKA_ERR_SHAPE;
  if (mode != KKA_WEIGHT_UNIFORM && seqs->num_seqs > 0 && !head_weight) return KKA_ERR_NULL;
  if (vb_seq_stride < 0) return KKA_ERR_SHAPE;
  const int64_t items = blocks ? num_blocks : seqs->total_blocks;
  if (items > 0 && !vb_out) return KKA_ERR_NULL;
  if (vb_out && !aligned16(vb_out)) return KKA_ERR_ALIGN;
  const PoolWs ws = pool_ws(kp, seqs, items, mode);
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total)) return KKA_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return KKA_ERR_ALIGN;
  uint32_t* err = device_error_word();
  if (!err) return KKA_ERR_DEVICE;
  (void)hipGetLastError();

  hipStream_t s = static_cast<hipStream_t>(stream);
  PoolArgs a = {};
  fill_pool_args(a, kp, seqs);
  a.subset = blocks;
  a.n_items = (int32_t)items;
  a.out = vb_out;
  a.vb_stride = vb_seq_stride;
  a.err = err;
  char* wsb = static_cast<char*>(workspace);
  if (mode == KKA_WEIGHT_VARIANCE) {
    if (seqs->num_seqs == 0) return KKA_OK;
    // At most one round of layers per work-group (a.ps.m layers at a time):
    // each round ends in stores of its sums, and a later round's loads,
    // counted in order with those stores, would wait for them to complete
    // (the ragged batch: 6.32 -> 6.12 ms, the same bits).
    const LayerSplit ls = layer_split(items, a.L);
    a.lps = ls.lps < a.ps.m ? ls.lps : a.ps.m;
    a.n_split = (a.L + a.lps - 1) / a.lps;
    a.partial = reinterpret_cast<float*>(wsb);
    a.stats_q = reinterpret_cast<double*>(wsb + ws.partial);
    hipError_t e = launch_pool_stats(a, s);
    if (e != hipSuccess) return KKA_ERR_DEVICE;
    WeightArgs w = {};
    w.s1 = a.partial;
    w.q = a.stats_q;
    w.var = reinterpret_cast<double*>(wsb + ws.partial + ws.q);
    w.csum = reinterpret_cast<double*>(wsb + ws.partial + ws.q + ws.var);
    w.head_weight = head_weight;
    w.seq_len = seqs->seq_len;
    w.offs = seqs->block_offsets;
    w.table = seqs->block_table;
    w.k = kp->k;
    w.sL = kp->stride_layer;
    w.sB = kp->stride_block;
    w.sH = kp->stride_head;
    w.P = kp->num_phys_blocks;
    w.S = seqs->num_seqs;
    w.L = a.L;
    w.H = a.H;
    w.LH = a.L * a.H;
    w.D = a.D;
    w.B = a.B;
    w.total_blocks = seqs->total_blocks;
    w.err = err;
    if ((e = launch_head_weights(w, s)) != hipSuccess) return KKA_ERR_DEVICE;
    return launched(launch_pool_combine(a, head_weight, w.csum, s));
  }
  if (items == 0) return KKA_OK;
  const LayerSplit ls = layer_split(items, a.L, pool_layer_bytes(kp));
  a.n_split = ls.n_split;
  a.lps = ls.lps;
  // upper bound of the launch's key bytes: full blocks
  const double key_bytes = (double)items * kp->block_size * a.L * a.H * a.D * 2.0;
  a.done = split_in_one_launch(items, ls.n_split, key_bytes) ? reinterpret_cast<uint32_t*>(wsb) : nullptr;
  a.partial = ls.n_split > 1 ? reinterpret_cast<float*>(wsb + ws.counters) : nullptr;
  a.weights = mode == KKA_WEIGHT_GIVEN ? head_weight : nullptr;
  return launched(launch_pool(a, mode, s));
}

kka_status kka_pool_on_write(const kka_kpool* kp, const kka_seqs* seqs, const uint16_t* new_k, int32_t mode,
                             const float* head_weight, float* running, int32_t seed, float* vb_out,
                             int64_t vb_seq_stride, void* stream) {
  kka_status st = check_kpool(kp);
  if (st != KKA_OK) return st;
  if ((st = check_seqs(seqs)) != KKA_OK) return st;
  if (mode != KKA_WEIGHT_UNIFORM && mode != KKA_WEIGHT_GIVEN) return KKA_ERR_SHAPE;
  if (vb_seq_stride < 0) return KKA_ERR_SHAPE;
  if ((int64_t)kp->block_size * kp->num_layers * kp->num_kv_heads >= ((int64_t)1 << 30)) return KKA_ERR_SHAPE;
  if (seqs->num_seqs == 0) return KKA_OK;
  if (!running || !vb_out || (mode == KKA_WEIGHT_GIVEN && !head_weight)) return KKA_ERR_NULL;
  if ((new_k && !aligned16(new_k)) || !aligned16(vb_out)) return KKA_ERR_ALIGN;
  uint32_t* err = device_error_word();
  if (!err) return KKA_ERR_DEVICE;
  (void)hipGetLastError();
  WriteArgs a{};
  a.k_new = new_k;
  a.k = const_cast<uint16_t*>(kp->k);  // written only when new_k is given (documented)
  a.sL = kp->stride_layer;
  a.sB = kp->stride_block;
  a.sT = kp->stride_token;
  a.sH = kp->stride_head;
  a.L = kp->num_layers;
  a.H = kp->num_kv_heads;
  a.D = kp->head_dim;
  a.B = kp->block_size;
  a.P = kp->num_phys_blocks;
  a.S = seqs->num_seqs;
  a.seq_len = seqs->seq_len;
  a.offs = seqs->block_offsets;
  a.table = seqs->block_table;
  a.weights = mode == KKA_WEIGHT_GIVEN ? head_weight : nullptr;
  a.running = running;
  a.out = vb_out;
  a.vb_stride = vb_seq_stride;
  a.seed = seed ? 1 : 0;
  a.q8 = kp->head_dim / 8;
  a.m = a.q8 >= 256 ? 1 : 256 / a.q8;
  a.nt = a.q8 * a.m;
  a.err = err;
  return launched(launch_pool_on_write(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Geometry and workspace layout of the attention reference.
struct AttnPlan {
  int32_t G = 0, TB = 0, TT = 0, max_tiles = 0, n_chunks = 0, U = 0, UPB = 0;
  bool mfma = false;
  size_t tile_offs = 0, n_blocks = 0, um = 0, ue = 0, M = 0, Z = 0, partial = 0, total = 0;
};

kka_status attn_plan(const kka_kpool* kp, const kka_seqs* sq, int32_t Hq, AttnPlan& p) {
  kka_status st = check_kpool(kp);
  if (st != KKA_OK) return st;
  if ((st = check_seqs(sq)) != KKA_OK) return st;
  const int32_t H = kp->num_kv_heads, D = kp->head_dim, B = kp->block_size, L = kp->num_layers;
  if (Hq < H || Hq % H != 0) return KKA_ERR_SHAPE;
  p.G = Hq / H;
  p.mfma = attention_mfma_ok(D, p.G, B);
  if (!p.mfma) {  // vector kernel: query group in registers, D/8 lanes per key row
    const int32_t q8 = D / 8;
    if (p.G > 8 || D > 512 || (q8 & (q8 - 1)) != 0 || (int64_t)q8 * H > 256) return KKA_ERR_SHAPE;
  }
  p.TB = attention_tile_blocks(B, H, p.G, p.mfma);
  if (p.TB < 1) return KKA_ERR_SHAPE;  // one block's logits do not fit in LDS
  p.TT = p.TB * B;
  p.U = p.mfma && B > 16 ? 16 : B;
  p.UPB = B / p.U;
  const int64_t tiles = ((int64_t)sq->total_blocks + p.TB - 1) / p.TB + sq->num_seqs;
  const int64_t LHq = (int64_t)L * Hq;
  const int64_t units = (int64_t)sq->total_blocks * p.UPB;
  if (tiles > 0x7fffffffLL || units > 0x7fffffffLL || LHq * units > ((int64_t)1 << 40)) return KKA_ERR_SHAPE;
  p.max_tiles = (int32_t)tiles;
  p.n_chunks = (int32_t)((LHq + attention_chunk_heads() - 1) / attention_chunk_heads());
  const size_t S = (size_t)sq->num_seqs, tb = (size_t)sq->total_blocks;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  p.tile_offs = take((S + 1) * sizeof(int32_t));
  p.n_blocks = take(S * sizeof(int32_t));
  p.um = take((size_t)LHq * units * sizeof(float));
  p.ue = take((size_t)LHq * units * sizeof(float));
  p.M = take(S * LHq * sizeof(float));
  p.Z = take(S * LHq * sizeof(float));
  p.partial = take((size_t)p.n_chunks * tb * sizeof(float));
  p.total = off;
  return KKA_OK;
}

}  // namespace

extern "C" {

size_t kka_attention_topk_workspace(const kka_kpool* kp, const kka_seqs* seqs, int32_t num_q_heads) {
  AttnPlan p;
  if (attn_plan(kp, seqs, num_q_heads, p) != KKA_OK) return 0;
  return p.total;
}

kka_status kka_attention_topk(const kka_kpool* kp, const kka_seqs* seqs, const float* queries, int32_t num_q_heads,
                              float scale, int32_t k, float* block_score_out, int64_t out_seq_stride,
                              int32_t* idx_out, float* score_out, int32_t* n_selected_out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  AttnPlan p;
  kka_status st = attn_plan(kp, seqs, num_q_heads, p);
  if (st != KKA_OK) return st;
  if (!std::isfinite(scale) || k < 0 || k > kMaxK || out_seq_stride < 1 || out_seq_stride > 0x7fffffffLL)
    return KKA_ERR_SHAPE;
  if (seqs->num_seqs == 0) return KKA_OK;
  if (!queries || !block_score_out || (k > 0 && !idx_out)) return KKA_ERR_NULL;
  if (!aligned16(queries) || !aligned16(block_score_out)) return KKA_ERR_ALIGN;
  if (!workspace || workspace_bytes < p.total) return KKA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KKA_ERR_ALIGN;
  uint32_t* err = device_error_word();
  if (!err) return KKA_ERR_DEVICE;
  (void)hipGetLastError();
  char* ws = static_cast<char*>(workspace);
  AttnArgs a{};
  a.k = kp->k;
  a.sL = kp->stride_layer;
  a.sB = kp->stride_block;
  a.sT = kp->stride_token;
  a.sH = kp->stride_head;
  a.L = kp->num_layers;
  a.H = kp->num_kv_heads;
  a.D = kp->head_dim;
  a.B = kp->block_size;
  a.P = kp->num_phys_blocks;
  a.S = seqs->num_seqs;
  a.total_blocks = seqs->total_blocks;
  a.seq_len = seqs->seq_len;
  a.offs = seqs->block_offsets;
  a.table = seqs->block_table;
  a.q = queries;
  a.Hq = num_q_heads;
  a.G = p.G;
  a.scale = scale;
  a.TB = p.TB;
  a.TT = p.TT;
  a.max_tiles = p.max_tiles;
  a.n_chunks = p.n_chunks;
  a.U = p.U;
  a.UPB = p.UPB;
  a.mfma = p.mfma ? 1 : 0;
  a.tile_offs = reinterpret_cast<int32_t*>(ws + p.tile_offs);
  a.n_blocks = reinterpret_cast<int32_t*>(ws + p.n_blocks);
  a.um = reinterpret_cast<float*>(ws + p.um);
  a.ue = reinterpret_cast<float*>(ws + p.ue);
  a.M = reinterpret_cast<float*>(ws + p.M);
  a.Z = reinterpret_cast<float*>(ws + p.Z);
  a.partial = reinterpret_cast<float*>(ws + p.partial);
  a.out = block_score_out;
  a.out_stride = out_seq_stride;
  a.err = err;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  hipError_t e = launch_attention_blocks(a, strm);
  if (e != hipSuccess || k == 0) return launched(e);
  // flat top-k over the block scores (non-negative by construction)
  ScoreArgs sa{};
  sa.aff = block_score_out;
  sa.rows_per_seq = out_seq_stride;
  sa.S = a.S;
  sa.max_pages = (int32_t)out_seq_stride;
  sa.D = a.D;
  sa.hier = 0;
  sa.ppc = sa.cpg = 1;
  sa.n_pages = a.n_blocks;
  sa.k_p = k;
  sa.idx_out = idx_out;
  sa.score_out = score_out;
  sa.cnt_out = n_selected_out;
  sa.err = err;
  return launched(launch_select(sa, strm));
}

// Anchor workspace of a layer split: one arrival counter per sequence, then
// each (sequence, split)'s partial sums.
static size_t anchor_counter_bytes(int32_t S) { return align256((size_t)S * sizeof(uint32_t)); }

size_t kka_pool_anchor_workspace(const kka_kpool* kp, const kka_seqs* seqs, int32_t window) {
  (void)window;
  if (check_kpool(kp) != KKA_OK || check_seqs(seqs) != KKA_OK) return 0;
  const LayerSplit ls = anchor_split(seqs->num_seqs, kp->num_layers);
  if (ls.n_split <= 1) return 0;
  return anchor_counter_bytes(seqs->num_seqs) +
         align256((size_t)seqs->num_seqs * ls.n_split * kp->head_dim * sizeof(float));
}

kka_status kka_pool_anchor(const kka_kpool* kp, const kka_seqs* seqs, int32_t window, const float* head_weight,
                           float* anchor_out, void* workspace, size_t workspace_bytes, void* stream) {
  kka_status st = check_kpool(kp);
  if (st != KKA_OK) return st;
  if ((st = check_seqs(seqs)) != KKA_OK) return st;
  if (window < 0) return KKA_ERR_SHAPE;
  if (seqs->num_seqs > 0 && !anchor_out) return KKA_ERR_NULL;
  if (anchor_out && !aligned16(anchor_out)) return KKA_ERR_ALIGN;
  const size_t need = kka_pool_anchor_workspace(kp, seqs, window);
  if (need > 0 && (!workspace || workspace_bytes < need)) return KKA_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return KKA_ERR_ALIGN;
  if (seqs->num_seqs == 0) return KKA_OK;
  uint32_t* err = device_error_word();
  if (!err) return KKA_ERR_DEVICE;
  (void)hipGetLastError();
  PoolArgs a = {};
  fill_pool_args(a, kp, seqs);
  const LayerSplit ls = anchor_split(seqs->num_seqs, a.L);
  a.n_split = ls.n_split;
  a.lps = ls.lps;
  a.n_items = seqs->num_seqs;
  a.weights = head_weight;
  a.out = anchor_out;
  // upper bound of the launch's key bytes: full windows
  const double key_bytes = (double)seqs->num_seqs * window * a.L * a.H * a.D * 2.0;
  a.done = split_in_one_launch(seqs->num_seqs, ls.n_split, key_bytes) ? static_cast<uint32_t*>(workspace) : nullptr;
  a.partial = ls.n_split > 1
                  ? reinterpret_cast<float*>(static_cast<char*>(workspace) + anchor_counter_bytes(seqs->num_seqs))
                  : nullptr;
  a.window = window;
  a.err = err;
  return launched(launch_anchor(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Fixed device scratch of kka_pool_anchor_noalloc: the layer-split partial
// sums of one call, one copy per device for the life of the process.  Host
// code reaches it only through the device address hipGetSymbolAddress
// returns for the current device (the array's name is a host-side stand-in).
constexpr size_t kAnchorScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kAnchorScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up once per
// device (with that device current); nullptr if the lookup failed.
void* anchor_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t kka_pool_anchor_noalloc_scratch(const kka_kpool* kp, const kka_seqs* seqs) {
  if (check_kpool(kp) != KKA_OK || check_seqs(seqs) != KKA_OK) return 0;
  const LayerSplit ls = anchor_split(seqs->num_seqs, kp->num_layers);
  if (ls.n_split <= 1) return 0;
  return (size_t)seqs->num_seqs * ls.n_split * kp->head_dim * sizeof(float);
}

kka_status kka_pool_anchor_noalloc(const kka_kpool* kp, const kka_seqs* seqs, int32_t window,
                                   const float* head_weight, float* anchor_out, void* stream) {
  kka_status st = check_kpool(kp);
  if (st != KKA_OK) return st;
  if ((st = check_seqs(seqs)) != KKA_OK) return st;
  if (window < 0) return KKA_ERR_SHAPE;
  if (seqs->num_seqs > 0 && !anchor_out) return KKA_ERR_NULL;
  if (anchor_out && !aligned16(anchor_out)) return KKA_ERR_ALIGN;
  const size_t need = kka_pool_anchor_noalloc_scratch(kp, seqs);
  if (need > kAnchorScratchBytes) return KKA_ERR_SCRATCH;
  if (seqs->num_seqs == 0) return KKA_OK;
  uint32_t* err = device_error_word();
  if (!err) return KKA_ERR_DEVICE;
  void* scr = need > 0 ? anchor_scratch() : nullptr;
  if (need > 0 && !scr) return KKA_ERR_DEVICE;
  (void)hipGetLastError();
  PoolArgs a = {};
  fill_pool_args(a, kp, seqs);
  const LayerSplit ls = anchor_split(seqs->num_seqs, a.L);
  a.n_split = ls.n_split;
  a.lps = ls.lps;
  a.n_items = seqs->num_seqs;
  a.weights = head_weight;
  a.out = anchor_out;
  // shares always added by the second kernel: no arrival counters, so no
  // part of the scratch has to hold a known value between calls
  a.done = nullptr;
  a.partial = ls.n_split > 1 ? static_cast<float*>(scr) : nullptr;
  a.window = window;
  a.err = err;
  return launched(launch_anchor(a, static_cast<hipStream_t>(stream)));
}

int64_t kka_level_rows(const kka_level_layout* lay) {
  LevelGeom g;
  if (!level_geom(lay, g)) return -1;
  return g.rows;
}

kka_status kka_build_levels(const kka_level_layout* lay, float* level_buf, const int32_t* n_pages,
                            const int32_t* first_dirty_page, void* stream) {
  if (!lay) return KKA_ERR_NULL;
  LevelGeom g;
  if (!level_geom(lay, g)) return KKA_ERR_SHAPE;
  if (!lay->hierarchical || lay->num_seqs == 0 || g.g_cap == 0) return KKA_OK;
  if (!level_buf || !n_pages) return KKA_ERR_NULL;
  if (!aligned16(level_buf)) return KKA_ERR_ALIGN;
  uint32_t* err = device_error_word();
  if (!err) return KKA_ERR_DEVICE;
  (void)hipGetLastError();
  LevelArgs a = {};
  a.lvl = level_buf;
  a.rows_per_seq = g.rows;
  a.S = lay->num_seqs;
  a.max_pages = lay->max_pages;
  a.D = lay->head_dim;
  a.ppc = lay->pages_per_chunk;
  a.cpg = lay->chunks_per_grid;
  a.c_cap = g.c_cap;
  a.g_cap = g.g_cap;
  a.n_pages = n_pages;
  a.first_dirty = first_dirty_page;
  a.err = err;
  return launched(launch_levels(a, static_cast<hipStream_t>(stream)));
}

size_t kka_score_topk_workspace(const kka_level_layout* lay, const kka_select* sel, int32_t with_affinity_out) {
  (void)sel;
  LevelGeom g;
  if (!level_geom(lay, g)) return 0;
  return score_counter_bytes(lay->num_seqs) +
         (with_affinity_out ? 0 : align256((size_t)lay->num_seqs * (size_t)g.rows * sizeof(float)));
}

}  // extern "C"

namespace {

// Validates a scoring call and fills the launch arguments.
kka_status prepare_score(const kka_level_layout* lay, const float* level_buf, const int32_t* n_pages,
                         const float* anchors, const kka_select* sel, float* affinity_out, int32_t* page_idx_out,
                         float* page_score_out, int32_t* n_selected_out, void* workspace, size_t workspace_bytes,
                         size_t need, ScoreArgs& a) {
  if (!lay || !sel) return KKA_ERR_NULL;
  LevelGeom g;
  if (!level_geom(lay, g)) return KKA_ERR_SHAPE;
  if (sel->k_page < 0 || sel->k_page > kMaxK) return KKA_ERR_SHAPE;
  if (lay->hierarchical &&
      (sel->k_grid < 0 || sel->k_grid > kMaxK || sel->k_chunk < 0 || sel->k_chunk > kMaxK))
    return KKA_ERR_SHAPE;
  if (lay->num_seqs == 0) return KKA_OK;
  if (!level_buf || !n_pages || !anchors) return KKA_ERR_NULL;
  if (sel->k_page > 0 && !page_idx_out) return KKA_ERR_NULL;
  if (!aligned16(level_buf) || !aligned16(anchors)) return KKA_ERR_ALIGN;
  if (need > 0 && (!workspace || workspace_bytes < need)) return KKA_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return KKA_ERR_ALIGN;
  if (affinity_out && !aligned16(affinity_out)) return KKA_ERR_ALIGN;
  uint32_t* err = device_error_word();
  if (!err) return KKA_ERR_DEVICE;
  (void)hipGetLastError();
  a = ScoreArgs{};
  a.lvl = level_buf;
  a.rows_per_seq = g.rows;
  a.S = lay->num_seqs;
  a.max_pages = lay->max_pages;
  a.D = lay->head_dim;
  a.hier = lay->hierarchical ? 1 : 0;
  a.ppc = lay->hierarchical ? lay->pages_per_chunk : 1;
  a.cpg = lay->hierarchical ? lay->chunks_per_grid : 1;
  a.c_cap = g.c_cap;
  a.g_cap = g.g_cap;
  a.n_pages = n_pages;
  a.anchors = anchors;
  // workspace: per-sequence tile counters, then scratch affinities
  const bool forced = two_launch_forced();
  a.small = !forced && small_levels(lay, g, sel) ? 1 : 0;
  a.done = forced || handoff_disabled() ? nullptr : static_cast<uint32_t*>(workspace);
  a.aff = affinity_out ? affinity_out
                       : reinterpret_cast<float*>(static_cast<char*>(workspace) + score_counter_bytes(lay->num_seqs));
  a.k_g = lay->hierarchical ? sel->k_grid : 0;
  a.k_c = lay->hierarchical ? sel->k_chunk : 0;
  a.k_p = sel->k_page;
  a.idx_out = page_idx_out;
  a.score_out = page_score_out;
  a.cnt_out = n_selected_out;
  a.rows_per_tile = score_rows_per_tile(a.D);
  const int64_t tiles = (g.rows + a.rows_per_tile - 1) / a.rows_per_tile;
  a.tiles_per_seq = (int32_t)(tiles > 0 ? tiles : 1);
  // the grid of any path fits: tiles of at least 16 rows, plus one selecting group per sequence
  if ((int64_t)a.S * ((g.rows + 15) / 16 + 1) > 0x7fffffffLL) return KKA_ERR_SHAPE;
  a.err = err;
  return KKA_OK;
}

}  // namespace

extern "C" {

kka_status kka_score_topk(const kka_level_layout* lay, const float* level_buf, const int32_t* n_pages,
                          const float* anchors, const kka_select* sel, float* affinity_out, int32_t* page_idx_out,
                          float* page_score_out, int32_t* n_selected_out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  ScoreArgs a;
  const size_t need = kka_score_topk_workspace(lay, sel, affinity_out != nullptr);
  const kka_status st = prepare_score(lay, level_buf, n_pages, anchors, sel, affinity_out, page_idx_out,
                                      page_score_out, n_selected_out, workspace, workspace_bytes, need, a);
  if (st != KKA_OK || lay->num_seqs == 0) return st;
  return launched(launch_score_topk(a, static_cast<hipStream_t>(stream)));
}

kka_status kka_score_topk_stable(const kka_level_layout* lay, const float* level_buf, const int32_t* n_pages,
                                 const float* anchors, const kka_select* sel, const kka_stability* stab,
                                 float* affinity_out, int32_t* page_idx_out, float* page_score_out,
                                 int32_t* n_selected_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!stab || !lay) return KKA_ERR_NULL;
  if (stab->window < 1 || stab->window > 32 || !std::isfinite(stab->theta)) return KKA_ERR_SHAPE;
  const bool words = lay->num_seqs > 0 && lay->max_pages > 0;
  if (words && !stab->history) return KKA_ERR_NULL;
  if (words &&
      ((reinterpret_cast<uintptr_t>(stab->history) & 3u) || (reinterpret_cast<uintptr_t>(stab->score_out) & 3u)))
    return KKA_ERR_ALIGN;
  ScoreArgs a;
  const size_t need = kka_score_topk_workspace(lay, sel, affinity_out != nullptr);
  const kka_status st = prepare_score(lay, level_buf, n_pages, anchors, sel, affinity_out, page_idx_out,
                                      page_score_out, n_selected_out, workspace, workspace_bytes, need, a);
  if (st != KKA_OK || lay->num_seqs == 0) return st;
  if (words) {
    a.hist = stab->history;
    a.stab_out = stab->score_out;
    a.stab_w = stab->window;
    a.stab_mask = stab->window == 32 ? 0xFFFFFFFFu : ((1u << stab->window) - 1u);
    a.theta = stab->theta;
  }
  return launched(launch_score_topk(a, static_cast<hipStream_t>(stream)));
}

kka_status kka_score_topk_lazy(const kka_level_layout* lay, const float* level_buf, const int32_t* n_pages,
                               const float* anchors, const kka_select* sel, float* affinity_out,
                               int32_t* page_idx_out, float* page_score_out, int32_t* n_selected_out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (lay && !lay->hierarchical)  // flat: every page is a candidate, the single pass is the lazy pass
    return kka_score_topk(lay, level_buf, n_pages, anchors, sel, affinity_out, page_idx_out, page_score_out,
                          n_selected_out, workspace, workspace_bytes, stream);
  ScoreArgs a;
  const size_t need = kka_score_topk_workspace(lay, sel, affinity_out != nullptr);
  const kka_status st = prepare_score(lay, level_buf, n_pages, anchors, sel, affinity_out, page_idx_out,
                                      page_score_out, n_selected_out, workspace, workspace_bytes, need, a);
  if (st != KKA_OK || lay->num_seqs == 0) return st;
  // long sequences keep scored rows in a.aff (affinity_out or workspace);
  // short ones keep them in LDS and copy to affinity_out when it is given
  float* lazy_out = a.rows_per_seq <= kSelectLdsRows ? affinity_out : nullptr;
  return launched(launch_score_topk_lazy(a, lazy_out, static_cast<hipStream_t>(stream)));
}

int32_t kka_device_error(void* stream) {
  uint32_t* p = device_error_word();
  if (!p) return -1;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return -1;
  uint32_t v = 0;
  if (hipMemcpy(&v, p, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return -1;
  const uint32_t zero = 0;
  if (v != 0 && hipMemcpy(p, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return -1;
  return (int32_t)v;
}

const char* kka_status_string(kka_status s) {
  switch (s) {
    case KKA_OK: return "ok";
    case KKA_ERR_NULL: return "a required pointer is NULL";
    case KKA_ERR_SHAPE: return "a size, count or mode is out of range";
    case KKA_ERR_ALIGN: return "a pointer or stride breaks its alignment rule";
    case KKA_ERR_WORKSPACE: return "workspace missing or too small";
    case KKA_ERR_DEVICE: return "HIP runtime error";
    case KKA_ERR_SCRATCH: return "the call needs more than the library's fixed scratch array holds";
  }
  return "unknown status";
}

int32_t kka_version(void) { return KKA_VERSION; }

}  // extern "C"
