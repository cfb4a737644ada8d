/*
 * kka.h -- Key-Key Semantic Affinity block selection for paged KV caches,
 * C ABI of libkka.so (AMD Instinct MI355X, gfx950).
 *
 * The method is the one described on the page "Key-Key Semantic Affinity:
 * Key vectors replace attention scores for KV-cache importance"
 * (10100.com): every KV-cache block is summarised once by the mean of its
 * keys (section 2.2 step 1, section 5.2 step 2); at every decode step the
 * keys of the last few tokens are pooled the same way into an anchor
 * (section 2.2 step 2, section 5.2 step 1); blocks are scored by the
 * cosine of anchor and block vector mapped to [0, 1] (section 2.2 step 3,
 * section 3.2) and the top-K are kept (section 5.2 step 4), optionally
 * through the Grid -> Chunk -> Page hierarchy scored in one pass with
 * parent masks (section 5.1).  Further entry points: the same selection
 * scored coarse to fine (kka_score_topk_lazy, section 5.1), the stability
 * filter fused into the scoring pass (kka_score_topk_stable, section 5.3),
 * block vectors kept current as keys are written (kka_pool_on_write,
 * section 5.2 step 2), and the attention-mass reference the page compares
 * its selection with (kka_attention_topk, section 3.3).
 *
 * Conventions shared by every entry point
 *  - Pointers named "device" are HIP device pointers; structs and scalars
 *    are read on the host during the call and may be freed afterwards.
 *  - Every buffer is caller-owned.  The library never allocates, frees or
 *    keeps device memory; scratch space is the caller's `workspace`.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only
 *    enqueue work and return; nothing is synchronised except by
 *    kka_device_error().
 *  - Arguments are validated on the host before anything is enqueued.  A
 *    non-zero kka_status means nothing was enqueued and no output written.
 *    Errors that depend on device-resident values (block-table entries,
 *    sequence lengths, page counts) cannot be seen on the host: kernels
 *    skip the offending item, write zeros for it where an output exists,
 *    and raise a bit in a per-device flag word read by kka_device_error().
 *  - Results are deterministic: no floating-point atomics; the same inputs
 *    give the same bits, wherever blocks sit in the physical pool.
 *  - bf16 keys are widened exactly and accumulated in fp32.
 *  - A few small launches (a layer-split pooling or anchor launch of at most
 *    one work-group per compute unit; a scoring batch whose tiles all fit on
 *    the chip) hand values from one work-group to another inside the launch
 *    through device-scope stores, an arrival counter and device-scope
 *    loads.  KKA_NO_HANDOFF=1 in the environment makes every call use a
 *    second launch instead; the results are the same bits.
 *  - A pooling launch of at least 2048 blocks, one work-group each, gives
 *    every XCD (work-group i runs on XCD i mod 8) a contiguous share of the
 *    blocks sized by a weight per XCD: by default 1.1 for even and 1.0 for
 *    odd XCDs on a 256-compute-unit device, whose odd XCDs stream slower;
 *    KKA_XCD_WEIGHTS="w0,...,w7" (eight positive numbers) sets others and
 *    KKA_XCD_WEIGHTS=off gives one block per work-group in order.  Every
 *    block is pooled once by the same arithmetic: the same bits either way.
 */
#ifndef KKA_H_
#define KKA_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define KKA_API __attribute__((visibility("default")))
#else
#define KKA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kka_status {
  KKA_OK = 0,
  KKA_ERR_NULL = 1,      /* a required pointer is NULL                          */
  KKA_ERR_SHAPE = 2,     /* a size, count or mode is outside its documented range */
  KKA_ERR_ALIGN = 3,     /* a pointer or stride breaks its alignment rule        */
  KKA_ERR_WORKSPACE = 4, /* workspace NULL or smaller than the *_workspace() size */
  KKA_ERR_DEVICE = 5,    /* the HIP runtime refused a launch                      */
  KKA_ERR_SCRATCH = 6    /* an allocation-free call needs more than its fixed     */
                         /* scratch array holds (kka_pool_anchor_noalloc)         */
} kka_status;

/* Bits of the device flag word returned by kka_device_error(). */
#define KKA_DEVERR_BLOCK_TABLE 1u /* a block-table entry outside [0, num_phys_blocks)      */
#define KKA_DEVERR_SEQ_LEN 2u     /* a logical block holds no valid token, or a window     */
                                  /* reaches past the sequence's blocks                    */
#define KKA_DEVERR_ROW 4u         /* a block's index in its sequence >= vb_seq_stride      */
#define KKA_DEVERR_PAGES 8u       /* n_pages[s] < 0 or > max_pages                         */
#define KKA_DEVERR_OFFSETS 16u    /* block_offsets not nondecreasing / total mismatch      */
#define KKA_DEVERR_WORKSPACE 32u  /* a workspace's arrival counter was not zero when a     */
                                  /* call used it (kka_score_topk, kka_pool_blocks,         */
                                  /* kka_pool_anchor: see their workspace)                  */

/*
 * Paged key pool.  Element (layer l, physical block p, token slot t,
 * KV head h, dimension d) is k[l*stride_layer + p*stride_block +
 * t*stride_token + h*stride_head + d]: one head_dim row is contiguous.
 * A single-tensor [L][P][B][H][D] pool has strides (P*B*H*D, B*H*D, H*D, D);
 * per-layer [P][B][H][D] caches placed at a fixed distance fit too.
 * Rules: k 16-byte aligned; head_dim a multiple of 8 in [8, 1024];
 * num_kv_heads * head_dim / 8 <= 1024; num_layers * num_kv_heads <= 4096;
 * strides >= 0 and multiples of 8 elements.
 */
typedef struct kka_kpool {
  const uint16_t* k; /* device, bf16 bit patterns */
  int32_t num_layers;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int64_t num_phys_blocks;
  int64_t stride_layer;
  int64_t stride_block;
  int64_t stride_token;
  int64_t stride_head;
} kka_kpool;

/*
 * A batch of sequences in CSR form.  Sequence s has seq_len[s] tokens in
 * logical blocks block_offsets[s] .. block_offsets[s+1]-1 (global logical
 * block ids), token tau in logical block tau / block_size, slot
 * tau % block_size; logical block b lives in physical block block_table[b].
 * A sequence normally owns ceil(seq_len / block_size) blocks; extra blocks
 * hold no valid token and raise KKA_DEVERR_SEQ_LEN when pooled.
 * total_blocks is the host's copy of block_offsets[num_seqs].
 */
typedef struct kka_seqs {
  int32_t num_seqs;
  int32_t total_blocks;
  const int32_t* seq_len;       /* device [num_seqs]       */
  const int32_t* block_offsets; /* device [num_seqs + 1]   */
  const int32_t* block_table;   /* device [total_blocks]   */
} kka_seqs;

typedef enum kka_weight_mode {
  KKA_WEIGHT_UNIFORM = 0,  /* plain mean over tokens, layers and heads                */
  KKA_WEIGHT_VARIANCE = 1, /* compute per-head variance weights, write them, use them */
  KKA_WEIGHT_GIVEN = 2     /* read frozen per-head weights                            */
} kka_weight_mode;

/*
 * kka_pool_blocks -- block key representation v_b (page section 2.2 step 1,
 * section 3.3, section 5.2 step 2).
 *
 * For each selected logical block b of sequence s, with n_b = min(B,
 * seq_len[s] - i*B) valid tokens (i = b - block_offsets[s]):
 *   UNIFORM:  v_b = 1/(n_b*L*H) * sum_{l,h,t<n_b} K[l][p][t][h][:]
 *   GIVEN / VARIANCE:
 *             v_b = sum_{l,h} w[s][l*H+h] * (1/n_b) sum_{t<n_b} K[l][p][t][h][:]
 * where p = block_table[b].  In VARIANCE mode the weights are first
 * computed from all seq_len[s] tokens of each sequence: w[s][l*H+h] is the
 * temporal variance of that (layer, KV head)'s keys -- per-dimension
 * population variance over the tokens, averaged over head_dim --
 * normalised to sum 1 over the L*H heads (uniform when all are 0), rounded
 * to fp32 and written to head_weight.  (The page names variance weighting
 * but prints no formula; this is the reading used here.)
 *
 * blocks      device [num_blocks] global logical block ids to pool, or NULL
 *             for all total_blocks blocks (num_blocks is then ignored).
 *             VARIANCE mode requires NULL.
 * head_weight device [num_seqs][L*H] fp32: written in VARIANCE mode, read in
 *             GIVEN mode, ignored (may be NULL) in UNIFORM mode.
 * vb_out      device fp32, 16-byte aligned; v_b of block b goes to row
 *             s*vb_seq_stride + i (vb_seq_stride > 0: one row range per
 *             sequence, e.g. the page rows of a level buffer) or to row b
 *             (vb_seq_stride == 0); a row is head_dim floats.
 * workspace   device, 16-byte aligned, >= kka_pool_blocks_workspace() bytes
 *             (may be NULL when that size is 0).  With fewer blocks than fill
 *             the chip, a block's layers are split over several work-groups
 *             (shares of at least 128 KiB of keys, full blocks counted):
 *             the workspace then starts with one uint32 arrival counter per
 *             block (4 * blocks bytes, rounded up to 256), followed by the
 *             shares' partial sums, which are added in split order.  A call
 *             of at most one work-group per compute unit (blocks times
 *             splits) that reads at most 32 MiB of keys (full blocks counted)
 *             adds them in the same launch, in the work-group that finishes a
 *             block's last share, which it finds through the counters; other
 *             calls add them in a second launch.  The counters must be zero before
 *             the first call that uses the workspace (allocate it
 *             zero-filled); every call leaves them zero.  A counter found at
 *             or above the split count raises KKA_DEVERR_WORKSPACE and that
 *             block's v_b is not written (re-zero the counters).  In VARIANCE
 *             mode the workspace holds instead the statistics pass's sums:
 *             per block and (layer, KV head) the head_dim token sums of the
 *             shifted keys (fp32) and their sum of squares (fp64), then per
 *             sequence the L*H head variances and the head_dim shift terms
 *             (fp64); nothing has to be zeroed.  Calls that run concurrently
 *             must not share a workspace.
 */
KKA_API kka_status kka_pool_blocks(const kka_kpool* kp, const kka_seqs* seqs, const int32_t* blocks, int32_t num_blocks,
                           int32_t mode, float* head_weight, float* vb_out, int64_t vb_seq_stride, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Workspace bytes kka_pool_blocks needs for these shapes (0 when none). */
KKA_API size_t kka_pool_blocks_workspace(const kka_kpool* kp, const kka_seqs* seqs, const int32_t* blocks,
                                 int32_t num_blocks, int32_t mode);

/*
 * kka_pool_anchor -- query anchor v_anchor (page section 2.2 step 2,
 * section 5.2 step 1): the same pooling over the last W_eff = min(window,
 * seq_len[s]) tokens of each sequence, which may span several blocks.
 * head_weight device [num_seqs][L*H] or NULL for uniform pooling.
 * anchor_out  device [num_seqs][head_dim] fp32, 16-byte aligned; an empty
 *             window gives the zero vector.
 * workspace   >= kka_pool_anchor_workspace() bytes, 16-byte aligned (NULL
 *             allowed when that size is 0); with a layer split, one uint32
 *             arrival counter per sequence then the shares' partial sums,
 *             with the same rules as kka_pool_blocks' workspace
 *             (sequences times splits work-groups, full windows counted).
 * Rules: window >= 0.
 */
KKA_API kka_status kka_pool_anchor(const kka_kpool* kp, const kka_seqs* seqs, int32_t window, const float* head_weight,
                           float* anchor_out, void* workspace, size_t workspace_bytes, void* stream);

KKA_API size_t kka_pool_anchor_workspace(const kka_kpool* kp, const kka_seqs* seqs, int32_t window);

/*
 * kka_pool_anchor_noalloc -- kka_pool_anchor for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, rules and results as
 * kka_pool_anchor (bit for bit), without a workspace: the layer-split
 * partial sums go to a scratch array of 4 MiB that the library holds in
 * every device's memory from its first use until the process ends, and are
 * always added by a second kernel (no arrival counters, so nothing in the
 * array has to be cleared between calls).  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).
 * Limit: kka_pool_anchor_noalloc_scratch() bytes (num_seqs * shares *
 * head_dim * 4, shares <= num_layers; 0 when the sequences are many enough
 * that each work-group takes all layers) must be at most 4 MiB, else
 * KKA_ERR_SCRATCH and nothing is enqueued.  Every call on a device shares
 * that device's array: calls that overlap on one device (two streams, two
 * host threads) race on it and must be serialised by the caller.
 */
KKA_API kka_status kka_pool_anchor_noalloc(const kka_kpool* kp, const kka_seqs* seqs, int32_t window,
                                           const float* head_weight, float* anchor_out, void* stream);

/* Scratch bytes a kka_pool_anchor_noalloc call with these shapes uses. */
KKA_API size_t kka_pool_anchor_noalloc_scratch(const kka_kpool* kp, const kka_seqs* seqs);

/*
 * kka_pool_on_write -- keep block vectors current as keys are written (page
 * section 2.2 step 1 and section 5.2 step 2: v_b is taken from the keys as
 * k_proj produces them and stored).  One call per decode step in which
 * every sequence gained one token: sequence s now holds seq_len[s] tokens
 * and its newest token t = seq_len[s] - 1 sits in logical block
 * j = t / block_size at slot t % block_size (the block table must already
 * list that block).
 *
 * new_k          device [num_seqs][num_layers][num_kv_heads][head_dim] bf16
 *                bits, 16-byte aligned: the new token's keys; they are
 *                stored into the pool at (layer, block_table[j], slot, head),
 *                so kp->k must then be writable memory (the const in
 *                kka_kpool says only that the other entry points never
 *                write it).  NULL: the keys are already in the pool and are
 *                only read.
 * mode           KKA_WEIGHT_UNIFORM (mean over tokens, layers and heads) or
 *                KKA_WEIGHT_GIVEN (head_weight [num_seqs][L*H], frozen).
 * running        device [num_seqs][head_dim] fp32, caller-owned state: the
 *                open block's key sum (uniform) or weighted key sum (given).
 * seed           0: `running` holds the open block's earlier tokens (a token
 *                at slot 0 starts a new sum); 1: rebuild it from the pool's
 *                tokens 0..slot-1 of the open block (e.g. after a prefill,
 *                or when the state is not known).
 * vb_out         receives the open block's vector, at row
 *                s * vb_seq_stride + j (vb_seq_stride > 0) or at the global
 *                logical block id (vb_seq_stride == 0); 16-byte aligned.
 * The vector equals the block's mean over its tokens so far, as
 * kka_pool_blocks computes it, up to fp32 summation order.  Sequences with
 * seq_len 0 are skipped; a seq_len beyond the sequence's blocks, a bad
 * physical block or a row past vb_seq_stride raises the device flag.
 * Errors: KKA_ERR_NULL (kp, seqs, running, vb_out, head_weight in given
 * mode), KKA_ERR_SHAPE (mode VARIANCE or unknown, vb_seq_stride < 0,
 * block_size * L * H >= 2^30), KKA_ERR_ALIGN (new_k, vb_out).  One launch.
 */
KKA_API kka_status kka_pool_on_write(const kka_kpool* kp, const kka_seqs* seqs, const uint16_t* new_k, int32_t mode,
                                     const float* head_weight, float* running, int32_t seed, float* vb_out,
                                     int64_t vb_seq_stride, void* stream);

/*
 * kka_attention_topk -- the reference selection the page compares with
 * (section 3.3): for one decode query per sequence, the attention mass of
 * every block, QK^T softmax averaged over every layer and query head, and
 * the top-k blocks by that mass.  Query head hq of layer l uses KV head
 * hq / (num_q_heads / num_kv_heads); its attention is softmax over the
 * sequence's seq_len[s] tokens of scale * (q . k); a block's score is the
 * sum over its tokens, averaged over the L * num_q_heads (layer, query head)
 * pairs, so a sequence's scores sum to 1.
 *
 * queries          device [num_seqs][L][num_q_heads][head_dim] fp32,
 *                  16-byte aligned.
 * block_score_out  device [num_seqs][out_seq_stride] fp32, 16-byte aligned:
 *                  block j of sequence s (j < its listed blocks) at
 *                  s * out_seq_stride + j; blocks without tokens score 0.
 * k, idx_out, score_out, n_selected_out
 *                  top-k logical block indices per sequence by (score
 *                  descending, index ascending) over the blocks holding
 *                  tokens, as in kka_score_topk's flat mode ([num_seqs][k];
 *                  k = 0 skips the selection).
 * workspace        >= kka_attention_topk_workspace() bytes, 16-byte aligned.
 * Rules: num_q_heads a multiple of num_kv_heads (G = num_q_heads /
 * num_kv_heads).  Matrix-core path: head_dim in {32, 64, 128, 256},
 * G <= 16 and block_size dividing 16 or a multiple of 16.  Otherwise the
 * vector path: G <= 8, head_dim a power of two <= 512 with
 * (head_dim / 8) * num_kv_heads <= 256 and num_q_heads * (block_size + 1)
 * <= 15360 (one block's logits must fit in LDS).  Both: scale finite, the
 * queries finite; k in 0..1024;
 * out_seq_stride >= 1.  Device-side problems (offsets, block table,
 * seq_len beyond the listed blocks, blocks past out_seq_stride) raise the
 * device flag and are skipped.  Several launches on `stream`.
 */
KKA_API kka_status kka_attention_topk(const kka_kpool* kp, const kka_seqs* seqs, const float* queries,
                                      int32_t num_q_heads, float scale, int32_t k, float* block_score_out,
                                      int64_t out_seq_stride, int32_t* idx_out, float* score_out,
                                      int32_t* n_selected_out, void* workspace, size_t workspace_bytes,
                                      void* stream);

KKA_API size_t kka_attention_topk_workspace(const kka_kpool* kp, const kka_seqs* seqs, int32_t num_q_heads);

/*
 * Level buffer geometry (page section 5.1).  Each sequence owns
 * rows_per_seq = kka_level_rows() consecutive rows of head_dim fp32:
 *   pages  rows [0, n_p)                   -- the block vectors v_b
 *   chunks rows [max_pages, max_pages + n_c)
 *   grids  rows [max_pages + C, max_pages + C + n_g)
 * with C = ceil(max_pages / pages_per_chunk), n_c = ceil(n_p /
 * pages_per_chunk), n_g = ceil(n_c / chunks_per_grid) and n_p the
 * sequence's page count.  Flat layouts (hierarchical == 0) hold pages only.
 * Sequence s starts at row s * rows_per_seq.
 * Rules: num_seqs >= 0; 0 <= max_pages <= 2^30; head_dim a multiple of 8
 * in [8, 1024]; hierarchical layouts need pages_per_chunk >= 1,
 * chunks_per_grid >= 1, C <= 16384, C * pages_per_chunk <= 2^30 and
 * chunks_per_grid * head_dim <= 16384.
 */
typedef struct kka_level_layout {
  int32_t num_seqs;
  int32_t max_pages;
  int32_t head_dim;
  int32_t hierarchical;
  int32_t pages_per_chunk;
  int32_t chunks_per_grid;
} kka_level_layout;

/* Rows per sequence of a level buffer, or -1 if the layout breaks a rule. */
KKA_API int64_t kka_level_rows(const kka_level_layout* lay);

/*
 * kka_build_levels -- chunk and grid vectors (page section 5.1: a grid's
 * vector is the mean of its chunk vectors; a chunk's is, by the same rule,
 * the mean of its page vectors).  Only the present children of a ragged
 * last chunk or grid are averaged.
 * level_buf        device, 16-byte aligned, [num_seqs][rows_per_seq][head_dim]
 * n_pages          device [num_seqs] pages per sequence (0..max_pages)
 * first_dirty_page device [num_seqs] or NULL: only chunks and grids that
 *                  can contain pages >= first_dirty_page[s] are rebuilt
 *                  (the whole grid holding that page and every later one).
 * A flat layout is accepted and does nothing.
 */
KKA_API kka_status kka_build_levels(const kka_level_layout* lay, float* level_buf, const int32_t* n_pages,
                            const int32_t* first_dirty_page, void* stream);

/* How many rows to keep at each level; each in [0, 1024]. */
typedef struct kka_select {
  int32_t k_grid;
  int32_t k_chunk;
  int32_t k_page;
} kka_select;

/*
 * kka_score_topk -- affinity of every row and top-K selection (page
 * section 2.2 step 3, section 5.1, section 5.2 steps 3-4).
 * Every present row r of sequence s (pages, chunks and grids alike, in one
 * pass) gets aff = clamp((1 + cos(r, anchor_s)) / 2, 0, 1), with cos = 0
 * when either vector has zero norm and -0 written as +0.  (The page's
 * affinity formula did not survive; this is the reading used here.)
 * Flat layout: the result is the top k_page pages by (aff desc, index asc).
 * Hierarchical layout: the top k_grid grids are kept; a chunk scores its
 * affinity if its grid was kept and +0 otherwise; the top k_chunk chunks
 * are kept; a page scores its affinity if its chunk was kept and +0
 * otherwise; the result is the top k_page pages by (score desc, index asc).
 * At each level min(k, rows present) rows are kept.  Selection compares
 * exactly the fp32 values the affinity pass produced.
 *
 * anchors        device [num_seqs][head_dim] fp32, 16-byte aligned
 * affinity_out   device [num_seqs][rows_per_seq] fp32, 16-byte aligned, or
 *                NULL; rows that are not present are left untouched
 * page_idx_out   device [num_seqs][k_page] int32 page index in its sequence,
 *                best first; slots past the kept count hold -1
 * page_score_out device [num_seqs][k_page] fp32 masked score, or NULL; slots
 *                past the kept count hold 0
 * n_selected_out device [num_seqs] int32 kept count, or NULL
 * workspace      device, 16-byte aligned, >= kka_score_topk_workspace()
 *                bytes (0, and NULL allowed, only when num_seqs is 0): one
 *                uint32 tile counter per sequence (the first 4 * num_seqs
 *                bytes, rounded up to 256), then scratch affinities when
 *                affinity_out is NULL.  The counters must be zero before the
 *                first call that uses the workspace (allocate it
 *                zero-filled); every call leaves them zero.  A counter found
 *                at or above the sequence's tile count raises
 *                KKA_DEVERR_WORKSPACE, and that sequence's selection is then
 *                not valid (re-zero the counters).  Calls that run
 *                concurrently must not share a workspace.
 * Work-groups score tiles of rows spread over the chip.  When every tile
 * of the batch fits on the chip at once, the call is one launch on
 * `stream`: the work-group that completes a sequence's last tile selects
 * that sequence (affinities pass between work-groups through device-scope
 * stores and loads).  Larger batches whose levels are small -- every level
 * offers at most 256 candidates (all grids; the chunks of the kept grids;
 * the pages of the kept chunks; all pages of a flat layout) and every k is
 * at most 256 -- are one launch too: a work-group per sequence selects
 * coarse to fine on its own, re-scoring its candidate rows with the
 * scoring tiles' code, and no work-group reads what another writes.  Other
 * batches run as two launches: the scoring pass, then one selecting
 * work-group per sequence.  KKA_SCORE_TWO_LAUNCH=1 in the environment sends
 * every call to the two-launch path.  Results are the same, bit for bit,
 * on every path.
 */
KKA_API kka_status kka_score_topk(const kka_level_layout* lay, const float* level_buf, const int32_t* n_pages,
                          const float* anchors, const kka_select* sel, float* affinity_out, int32_t* page_idx_out,
                          float* page_score_out, int32_t* n_selected_out, void* workspace, size_t workspace_bytes,
                          void* stream);

KKA_API size_t kka_score_topk_workspace(const kka_level_layout* lay, const kka_select* sel, int32_t with_affinity_out);

/*
 * Stability filter state (page section 5.3): per page, a word holding the
 * last `window` steps, bit i set when the page's affinity i steps before the
 * newest was above `theta`.  stability score = set bits / window.
 *
 * history    device [num_seqs][max_pages] uint32, caller-owned, in/out;
 *            word of page p of sequence s at s * max_pages + p.  Zero-fill
 *            it for a new sequence or a new page (no steps seen yet).
 *            Only words of present pages (p < n_pages[s]) are touched.
 * score_out  device [num_seqs][max_pages] fp32, same indexing, or NULL.
 * window     number of steps, 1..32 (the page uses 20).
 * theta      per-step threshold, finite (the page uses 0.5); a step counts
 *            when the affinity is strictly above it.
 * Readings where the page is silent: the strict comparison; steps before
 * the first (or before the page existed) count as not high, so the score
 * is set bits / window from the first step on; the affinity is the page's
 * own, before any hierarchical masking.
 */
typedef struct kka_stability {
  uint32_t* history;
  float* score_out;
  int32_t window;
  float theta;
} kka_stability;

/*
 * kka_score_topk_stable -- kka_score_topk with the stability filter fused
 * into the scoring pass: every present page's window word shifts by one
 * step and takes this step's bit (one 4-byte read and write per page, plus
 * the 4-byte score when score_out is set).  Selection is unchanged (the
 * page leaves the trigger threshold on the score to the caller, who reads
 * score_out).  Other arguments, rules and workspace as kka_score_topk.
 * Errors: stab NULL or history NULL (with num_seqs > 0 and max_pages > 0)
 * -> KKA_ERR_NULL; window outside 1..32 or theta not finite -> KKA_ERR_SHAPE;
 * history or score_out not 4-byte aligned -> KKA_ERR_ALIGN.
 */
KKA_API kka_status kka_score_topk_stable(const kka_level_layout* lay, const float* level_buf, const int32_t* n_pages,
                                         const float* anchors, const kka_select* sel, const kka_stability* stab,
                                         float* affinity_out, int32_t* page_idx_out, float* page_score_out,
                                         int32_t* n_selected_out, void* workspace, size_t workspace_bytes,
                                         void* stream);

/*
 * kka_score_topk_lazy -- the same selection, scored coarse to fine (page
 * section 5.1: chunks are scored only inside kept grids, pages only inside
 * surviving chunks).  One work-group per sequence scores the grids, keeps
 * the top k_grid, scores only the chunks of kept grids, keeps the top
 * k_chunk, scores only the pages of kept chunks and keeps the top k_page.
 * Rows under unkept parents are never read; their score is +0 by
 * definition, so page_idx_out, page_score_out and n_selected_out are bit
 * for bit those of kka_score_topk on the same inputs.  affinity_out (if
 * given) receives only the rows actually scored, bit-identical to
 * kka_score_topk's values for those rows; other rows are left untouched.
 * Arguments, rules and workspace are those of kka_score_topk (the same
 * kka_score_topk_workspace() size suffices; the tile counters are not
 * touched).  A flat layout has no parents: the call is then
 * kka_score_topk.  One launch on `stream`.
 */
KKA_API kka_status kka_score_topk_lazy(const kka_level_layout* lay, const float* level_buf, const int32_t* n_pages,
                                       const float* anchors, const kka_select* sel, float* affinity_out,
                                       int32_t* page_idx_out, float* page_score_out, int32_t* n_selected_out,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * kka_device_error -- waits for `stream`, returns the KKA_DEVERR_* bits
 * raised on the current device since the last call, and clears them.
 * Returns -1 if the wait or the read failed (HIP error).
 */
KKA_API int32_t kka_device_error(void* stream);

/* Static description of a kka_status value. */
KKA_API const char* kka_status_string(kka_status s);

/* Version of this header as major*10000 + minor*100 + patch.  0.2.0: the
 * kka_score_topk workspace holds per-sequence tile counters that must be
 * zero at first use.  0.3.0: so do the kka_pool_blocks and kka_pool_anchor
 * workspaces of layer-split launches (per-block / per-sequence arrival
 * counters; the smallest launches combine the split shares in the same
 * launch).  0.4.0: kka_pool_anchor_noalloc and KKA_ERR_SCRATCH. */
#define KKA_VERSION 400

/* Version of the loaded library, same encoding (equals KKA_VERSION when the
 * header and the library match). */
KKA_API int32_t kka_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KKA_H_ */
