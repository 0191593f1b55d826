/*
 * csa2.h — C ABI of libcsa2.so: CSA2 compressed-KV sparse decode on MI355X (gfx950).
 *
 * Sources (web pages on DeepSeek-V4.1 Flash and its CSA2 attention):
 *   [P1] "DeepSeek-v4.1 Flash: KVキャッシュ圧縮の限界を押し広げる" (hackernews.jp
 *        translation of zartbot's walk-through of the tech report)
 *   [P2] ai.freelance-job.com news summary of that walk-through
 *   [P3] "DeepSeek V4.1 Flash architecture: making a giant AI faster through reuse"
 *        (yasmorita.com)
 *
 * Conventions for every entry point
 *   - Pointers marked (device) point to GPU memory; everything else is host memory.
 *     The caller allocates and frees all memory: cache pages, tables, inputs, outputs
 *     and workspace.  The library allocates nothing and keeps no mutable global state.
 *   - bf16 values travel as uint16_t bit patterns.
 *   - Alignment: every device array starts on a 16-byte boundary (the kernels load
 *     rows with 16-byte vector loads); torch and hipMalloc allocations satisfy this.
 *   - Graph capture: the launches can be recorded into a HIP graph.  A function's
 *     first call in a process raises its kernels' dynamic-LDS limit (a runtime call
 *     that a stream capture may refuse), so make that first call outside a capture;
 *     csa2_schedule_create does this itself.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = default
 *     stream).  A return of CSA2_OK means the launch was accepted; results are ready
 *     once the stream is synchronised.
 *   - Return codes: CSA2_OK (0) or a negative CSA2_E* code.  Only host-visible
 *     arguments are validated, and nothing is enqueued when validation fails.  Device
 *     arrays are read defensively: an entry index outside [0, visible entries), a page
 *     id outside [0, n_pages) or a context beyond the cache table is treated as an
 *     absent row, never dereferenced.
 *   - Token positions: a decode query for a context of L tokens sits at position
 *     t = L - 1; entry j merges tokens 2j and 2j+1 and is visible to t iff 2j+1 <= t
 *     ([P3], causal-mask section), so floor(L/2) entries are visible.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fixed shapes.  512-d shared latent ([P1] §1.1, [P2] spec table); 64-d indexer
 * key and 4 indexer heads (the pages leave them blank); e2m1 codes with one e8m0
 * scale byte per 32 channels (the pages only say FP4 plus magnitude data, [P3]);
 * 64 entries per page ([P3], memory is taken in fixed blocks). */
#define CSA2_D_LATENT 512
#define CSA2_D_INDEX 64
#define CSA2_H_INDEX 4
#define CSA2_MX_BLOCK 32
#define CSA2_PAGE 64
#define CSA2_LAT_CODE_BYTES 256   /* per entry */
#define CSA2_LAT_SCALE_BYTES 16
#define CSA2_IDX_CODE_BYTES 32
#define CSA2_IDX_SCALE_BYTES 2
#define CSA2_MAX_TOPK 2048
#define CSA2_MAX_WINDOW 1024

enum {
  CSA2_OK = 0,
  CSA2_EINVAL = -1,       /* null pointer, bad size, odd token count, ... */
  CSA2_EWORKSPACE = -2,   /* workspace missing or smaller than csa2_workspace_size() */
  CSA2_EUNSUPPORTED = -3, /* a valid request this library does not implement */
  CSA2_EHIP = -4,         /* the HIP runtime refused a launch */
  CSA2_ESCRATCH = -5      /* csa2_index_full_noalloc: workspace above the fixed array */
};

/* Size of the per-GPU array that csa2_index_full_noalloc uses as its workspace. */
#define CSA2_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Workspace-sized functions (argument `fn` of csa2_workspace_size). */
enum {
  CSA2_FN_INDEX_FULL = 1,
  CSA2_FN_REINDEX = 2,
  CSA2_FN_SPARSE_DECODE = 3,
  CSA2_FN_PREFILL_CHUNK = 4
};

/* Paged cache of entries.  Entry j of sequence b lives in slot j % 64 of
 * page block_table[b * max_pages + j / 64].  ratio ([P1] §2.3.1) is the number of
 * tokens per entry: 2 for the encoder's cache (entry j merges tokens 2j, 2j+1) and
 * 1 for the decoder's (entry j is token j, uncompressed in the sequence dimension);
 * 0 means 2.  A query at token t sees floor((t+1)/ratio) entries, so a context of
 * L tokens has floor(L/ratio).  Per entry:
 *   lat_codes  [n_pages][64][256]  512 e2m1 codes, channel 2i in the low nibble
 *   lat_scales [n_pages][64][16]   e8m0 scale byte of channels 32k..32k+31
 *   idx_codes  [n_pages][64][32]   64 e2m1 indexer-key codes
 *   idx_scales [n_pages][64][2]
 * A code c stands for (-1)^(c>>3) * {0, .5, 1, 1.5, 2, 3, 4, 6}[c & 7] and a scale
 * byte u for 2^(u-127).  All pointers (device); the struct itself is host memory. */
typedef struct csa2_cache_t {
  uint8_t *lat_codes;
  uint8_t *lat_scales;
  uint8_t *idx_codes;
  uint8_t *idx_scales;
  int32_t n_pages;
  const int32_t *block_table; /* [B][max_pages] int32 (device) */
  int32_t max_pages;
  int32_t ratio;              /* tokens per entry: 2 (or 0) or 1 */
} csa2_cache_t;

/* Bytes one merged entry occupies: 272 latent + 34 indexer = 306. */
int csa2_bytes_per_entry(void);

/* Static description of a return code. */
const char *csa2_strerror(int code);

/* Workspace bytes `fn` needs for these sizes (0 if none).  max_ctx bounds every
 * ctx_len / prior_len + C (tokens); pool_blocks is the Full layer's pool quota;
 * ratio is the cache's (2, or 0 meaning 2, or 1). */
size_t csa2_workspace_size(int fn, int B, int H, int64_t max_ctx, int topk, int pool_blocks, int C,
                           int ratio);

/* csa2_write_kv — write path ([P1] §1.1 sequence dimension, §2.3.1 compressor).
 *   ratio must equal the cache's.  Ratio 2 (encoder): merge token pairs with
 *   per-channel weights, quantise to FP4, store.  Ratio 1 (decoder): entry
 *   j = start_tok[b] + i is token i quantised as it is (y = x[b][i]; w unused, may
 *   be NULL); k_idx: [B][T_new][64]; any start_tok >= 0 and T_new >= 1.
 *   Ratio 2: for each sequence b and i < T_new/2, entry j = start_tok[b]/2 + i is
 *     y_c = fp32_rne(w[b][2i][c] * x[b][2i][c] + w[b][2i+1][c] * x[b][2i+1][c])
 *   (exact products and sum, one rounding; no normalisation), then every block of
 *   32 channels is quantised: scale exponent e = clamp(floor(log2 max|y|) - 2,
 *   -127, 127), code = nearest e2m1 value of |y|/2^e with ties to the even code,
 *   saturating at 6, sign bit = sign of y; an all-zero block stores scale 0 and +0
 *   codes.  The indexer key k_idx[b][i] (64 bf16; its projection from the entry is a
 *   trained weight the caller applies, [P1] §2.3.1) is quantised the same way.
 *   x, w: [B][T_new][512] bf16 (device); k_idx: [B][T_new/2][64] bf16 (device);
 *   start_tok: [B] int32 (device), even.  T_new must be even (> 0); an unpaired last
 *   token is the caller's to resubmit with the next one.  The table must already
 *   hold pages for every written entry.  The rule above covers finite y; the codes of
 *   a block holding an Inf or NaN are unspecified.  More than 2^31 - 1 entries in one
 *   call return CSA2_EUNSUPPORTED. */
int csa2_write_kv(const csa2_cache_t *cache, int B, const int32_t *start_tok, int T_new,
                  const uint16_t *x, const uint16_t *w, const uint16_t *k_idx, int ratio,
                  void *stream);

/* csa2_write_kv_proj — the write path with the indexer key projected from the entry
 *   ([P1] §2.3.1: the indexer key is a projection of the compressed main entry).
 *   Same arguments, layout and latent as csa2_write_kv, but instead of k_idx the
 *   caller passes the projection weights w_proj: [64][512] bf16 (device, row o =
 *   output channel o).  With y the entry's fp32 latent before quantisation (the
 *   merge above at ratio 2, the token at ratio 1), key channel o is
 *     k_o = fp32_rne(s_512),  s_0 = 0,  s_{d+1} = fp64_rne(s_d + w_proj[o][d] * y[d])
 *   accumulated over d = 0..511 in that order (each product is exact in fp64), then
 *   quantised like any indexer key.  The pages give no precision for the projection;
 *   this one fixes every rounding, so the stored codes are reproducible bit for bit.
 *   Returns CSA2_EINVAL for a null w_proj or the csa2_write_kv conditions; allocates
 *   nothing (75 KB of LDS per workgroup). */
int csa2_write_kv_proj(const csa2_cache_t *cache, int B, const int32_t *start_tok, int T_new,
                       const uint16_t *x, const uint16_t *w, const uint16_t *w_proj, int ratio,
                       void *stream);

/* csa2_block_keys — HISA block summaries ([P1] §2.3.4, the HISA scheme it builds on:
 *   each block of positions keeps the mean of its indexer keys; during decoding only
 *   the current block changes).  Block k of sequence b covers entries k*cand_block ..
 *   k*cand_block + cand_block - 1 of `cache`; its summary is the mean of the
 *   dequantised keys of those entries that are visible (j < ctx_len[b] >> (ratio-1))
 *   and present, summed in float32 in entry order and divided once by their count (the
 *   zero key for a block with none), quantised like an indexer key and stored in slot k
 *   of `blocks` (its idx_codes / idx_scales through its own block table, 64 blocks per
 *   page; its latent arrays are not touched; blocks->ratio must be 1).
 *   Blocks written: per sequence blk_first[b] .. min(blk_first[b] + n_span, nb) - 1
 *   with nb = ceil(visible entries / cand_block) (decode: blk_first = the newest block,
 *   n_span = 1), or every block when blk_first is NULL (n_span ignored).  n_blocks
 *   ([B] int32, device, optional) receives nb, the context to give csa2_index_full on
 *   `blocks`.  The HISA selection is then csa2_index_full(blocks, B, n_blocks, ...,
 *   topk = the number of blocks to keep, pool_blocks = 0), whose ascending block ids
 *   are the pool of csa2_reindex(cache, ..., that pool, cand_block, K).
 *   cand_block: a power of two in [1, 32].  Returns CSA2_EINVAL for bad arguments;
 *   allocates nothing. */
int csa2_block_keys(const csa2_cache_t *cache, const csa2_cache_t *blocks, int B, const int32_t *ctx_len,
                    int64_t max_ctx, int cand_block, const int32_t *blk_first, int n_span, int32_t *n_blocks,
                    void *stream);

/* csa2_index_full — Full-mode indexer ([P1] §2.3.2 Full mode, §2.3.4 HSI).
 *   For every sequence b with n = floor(ctx_len[b]/ratio) visible entries:
 *     s_j = sum_{h<4} w_idx[b][h] * max(0, q_idx[b][h] . k_j)   (k_j dequantised)
 *   topk_idx[b] = the min(topk, n) entries with the largest s (ties: lower j), in
 *   ascending j order, padded with -1.  If pool_blocks > 0: block maxima over blocks
 *   of cand_block entries (last block padded with -inf), the block holding entry n-1
 *   forced to +inf, the best min(pool_blocks, #blocks) blocks (ties: lower block id)
 *   written to pool[b] in ascending order, padded with -1.
 *   ctx_len: [B] int32 tokens (device), each <= max_ctx; q_idx: [B][4][64] bf16;
 *   w_idx: [B][4] bf16; topk_idx: [B][topk] int32; pool: [B][pool_blocks] int32 or
 *   NULL when pool_blocks == 0 (all device).  1 <= topk <= 2048; cand_block in
 *   {1,2,4,8,16,32}; max_ctx/ratio <= 64 * max_pages.  ws: csa2_workspace_size(
 *   CSA2_FN_INDEX_FULL, B, 0, max_ctx, topk, pool_blocks, 0, ratio) bytes (device).
 *   Capacity, with n = max_ctx / ratio: ceil(n / 16384) * topk <= 32768 (1,048,576
 *   entries at topk 512), and with pool_blocks > 0 also ceil(n / cand_block) <= 32768
 *   (262,144 entries at cand_block 8, 1,048,576 at 32).  Past these the call returns
 *   CSA2_EUNSUPPORTED.  The workspace size does not depend on cand_block; the size
 *   query returns 0 only when no cand_block fits (it checks with cand_block 32). */
int csa2_index_full(const csa2_cache_t *cache, int B, const int32_t *ctx_len, int64_t max_ctx,
                    const uint16_t *q_idx, const uint16_t *w_idx, int topk, int pool_blocks,
                    int cand_block, int32_t *topk_idx, int32_t *pool, void *ws, size_t ws_bytes,
                    void *stream);

/* csa2_write_index_full — the step's write followed by the Full selection, in one
 *   launch sequence ([P1] §2.3.1: a decode step appends the new entry, then the
 *   indexer scores every visible entry, the new one included; §2.3.2 Full mode).
 *   Results, outputs and workspace are exactly those of csa2_write_kv(cache, B,
 *   start_tok, T_new, x, w, k_idx, ratio) followed on the same stream by
 *   csa2_index_full(cache, B, ctx_len, max_ctx, q_idx, w_idx, topk, pool_blocks,
 *   cand_block, topk_idx, pool, ws, ws_bytes): the same cache bytes and the same
 *   selections, bit for bit.  The write is done by the scan itself (each written entry
 *   that a chunk streams is stored by the wave that reads it, just before it reads it),
 *   which saves the write's launch.  That holds for writes of up to 2 entries per
 *   sequence (a decode step); a larger write runs as the two launches, since a wave
 *   stores its entries one after another.  Arguments, layouts, ownership and error
 *   codes are those of the two calls; any argument either call rejects is rejected here
 *   before anything runs. */
int csa2_write_index_full(const csa2_cache_t *cache, int B, const int32_t *start_tok, int T_new,
                          const uint16_t *x, const uint16_t *w, const uint16_t *k_idx, int ratio,
                          const int32_t *ctx_len, int64_t max_ctx, const uint16_t *q_idx, const uint16_t *w_idx,
                          int topk, int pool_blocks, int cand_block, int32_t *topk_idx, int32_t *pool, void *ws,
                          size_t ws_bytes, void *stream);

/* csa2_index_full_noalloc — csa2_index_full for callers that cannot allocate device
 *   memory: code under HIP graph capture, tight serving loops, and harnesses that
 *   forbid hipMalloc.  Same arguments, results and checks as csa2_index_full, without
 *   ws / ws_bytes: the workspace is a library-owned array of
 *   CSA2_NOALLOC_SCRATCH_BYTES (32 MiB) in device memory, one per GPU, resident from
 *   the first call on that GPU until the process ends.  A request whose workspace
 *   (csa2_workspace_size(CSA2_FN_INDEX_FULL, ...)) is larger returns CSA2_ESCRATCH
 *   before any launch; 32 MiB covers batch 32 at 32,768 entries with a 4096-entry
 *   pool, and batch 8 at 524,288 entries without a pool.  The call allocates nothing
 *   (no hipMalloc, no allocating library routine); on its first call on a GPU it looks
 *   up the array's device address (CSA2_EHIP if that fails).  Every call on one GPU
 *   shares that GPU's array: calls that overlap in time on one GPU (two streams, or
 *   two host threads) race and give undefined results; calls ordered on one stream
 *   are safe.  The array needs no clearing between calls. */
int csa2_index_full_noalloc(const csa2_cache_t *cache, int B, const int32_t *ctx_len, int64_t max_ctx,
                            const uint16_t *q_idx, const uint16_t *w_idx, int topk, int pool_blocks,
                            int cand_block, int32_t *topk_idx, int32_t *pool, void *stream);

/* csa2_reindex — Reindex mode ([P1] §2.3.2 Reindex mode, §2.3.4: later indexers
 *   score only the candidate pool).  Scores, with this layer's q_idx / w_idx, the
 *   visible entries j < floor(ctx_len[b]/ratio) of the blocks listed in pool[b] (block
 *   ids, -1 entries ignored, each block covering cand_block entries), and writes the
 *   min(topk, pool size) best (ties: lower j) to topk_idx[b] in ascending order,
 *   padded with -1.  Shapes as in csa2_index_full; pool_blocks * cand_block <= 16384.
 *   ws: optional.  With ws_bytes >= csa2_workspace_size(CSA2_FN_REINDEX, B, 0, 0, topk,
 *   pool_blocks, 0, ratio) (device memory) the pool is scored by many workgroups per
 *   sequence and selected by a second pass; with ws == NULL by one workgroup per
 *   sequence.  Results are the same. */
int csa2_reindex(const csa2_cache_t *cache, int B, const int32_t *ctx_len, const uint16_t *q_idx,
                 const uint16_t *w_idx, const int32_t *pool, int pool_blocks, int cand_block,
                 int topk, int32_t *topk_idx, void *ws, size_t ws_bytes, void *stream);

/* csa2_sparse_decode — one CSA2 attention for one decode query per sequence
 *   ([P1] §2.3.1: each query attends to the selected entries and the layer's window
 *   KV together; [P3]: scores -> weights summing to 1 -> weighted sum of values).
 *   Rows R = dequantised latent of every valid topk_idx[b][i] (valid: 0 <= j <
 *   floor(ctx_len[b]/ratio)) followed by the window rows of positions max(0, t-W+1)..t,
 *   t = ctx_len[b]-1, taken from swa[b][pos % W].  For every head h:
 *     z_r = sm_scale * q[b][h] . R_r,  p = softmax(z),  out[b][h] = sum_r p_r R_r
 *   (K = V = the 512-d latent), rounded to bf16; lse[b][h] = log sum_r exp(z_r).
 *   Reuse mode ([P1] §2.3.2) is this call with an earlier layer's topk_idx.
 *   q: [B][H][512] bf16; topk_idx: [B][topk] int32; swa: [B][W][512] bf16;
 *   out: [B][H][512] bf16; lse: [B][H] float or NULL (all device).  H a multiple of
 *   16; 1 <= W <= 1024; 0 <= topk <= 2048.  ws, ws_bytes: kept for callers of the
 *   workspace-sized interface; the call needs no workspace (csa2_workspace_size(
 *   CSA2_FN_SPARSE_DECODE, ...) returns 0) and ignores them, except that ws_bytes > 0
 *   with ws NULL is CSA2_EWORKSPACE.  No state goes through memory between kernels:
 *   small batches split each (sequence, 16-head group)'s output dims over several
 *   workgroups, not its rows. */
int csa2_sparse_decode(const csa2_cache_t *cache, int B, int H, const int32_t *ctx_len,
                       const uint16_t *q, const int32_t *topk_idx, int topk, const uint16_t *swa,
                       int W, float sm_scale, uint16_t *out, float *lse, void *ws, size_t ws_bytes,
                       void *stream);

/* csa2_prefill_chunk — chunked prefill after csa2_write_kv stored the chunk
 *   ([P1] §2.3.1: every query runs the indexer over the entries its causal mask
 *   lets it see, keeps the top K and attends to them plus its window; [P3] causal
 *   mask).  For sequence b and chunk query i (position t = prior_len[b] + i):
 *   Full-mode indexer over the floor((t+1)/2) entries visible to t, top-K as in
 *   csa2_index_full (no pool), then the attention of csa2_sparse_decode with window
 *   rows for positions max(0, t-W+1)..t taken from local[b][pos - prior_len[b] + W - 1].
 *   q: [B][C][H][512]; q_idx: [B][C][4][64]; w_idx: [B][C][4]; local: [B][W-1+C][512]
 *   (bf16, device); out: [B][C][H][512] bf16; topk_idx: [B][C][topk] int32 or NULL
 *   (then the lists live in the workspace).  prior_len: [B] int32 (device),
 *   prior_len[b] + C <= max_ctx.  H a multiple of 16; 1 <= W <= 1024; 1 <= topk <= 2048.
 *   Chunked prefill is the encoder's path: a ratio-1 cache gives CSA2_EUNSUPPORTED.
 *   ws: csa2_workspace_size(CSA2_FN_PREFILL_CHUNK, B, H, max_ctx, topk, 0, C, 2) bytes
 *   (device): per-query candidate lists, and the top-K lists when topk_idx is NULL. */
int csa2_prefill_chunk(const csa2_cache_t *cache, int B, int H, const int32_t *prior_len,
                       int64_t max_ctx, int C, const uint16_t *q, const uint16_t *q_idx,
                       const uint16_t *w_idx, const uint16_t *local, int W, int topk,
                       float sm_scale, uint16_t *out, int32_t *topk_idx, void *ws,
                       size_t ws_bytes, void *stream);

/* Layer schedules ([P1] §2.3.2 modes, §2.3.3 schedules: an encoder block is one
 * Full layer then five Reuse layers; the decoder runs [Full + 3 Reuse] then four
 * blocks of [Reindex + 3 Reuse]). */
enum { CSA2_LAYER_FULL = 0, CSA2_LAYER_REINDEX = 1, CSA2_LAYER_REUSE = 2 };

/* One layer of a schedule.  All pointers device memory. */
typedef struct csa2_layer_t {
  int32_t mode;             /* CSA2_LAYER_* */
  int32_t pool_blocks;      /* Full: candidate blocks kept for later Reindex layers (0: none) */
  const uint16_t *q;        /* [B][H][512] bf16 */
  const uint16_t *q_idx;    /* [B][4][64] bf16 (Full and Reindex layers) */
  const uint16_t *w_idx;    /* [B][4] bf16 (Full and Reindex layers) */
  const uint16_t *swa;      /* [B][W][512] bf16, ring slot pos % W */
  uint16_t *out;            /* [B][H][512] bf16 */
  float *lse;               /* [B][H] or NULL */
} csa2_layer_t;

typedef struct csa2_schedule csa2_schedule_t;   /* opaque: a captured HIP graph */

/* Workspace bytes of csa2_schedule_create for these sizes and layers (0 if the
 *   schedule is invalid).  ratio: the cache's. */
size_t csa2_schedule_workspace_size(int B, int H, int64_t max_ctx, int topk, int n_layers,
                                    const csa2_layer_t *layers, int ratio);

/* csa2_schedule_create — capture one decode step of a layer schedule into a HIP
 *   graph: the step's write (csa2_write_kv of T_new tokens at start_tok; skipped when
 *   x is NULL), then per layer its selection (Full: csa2_index_full with the layer's
 *   pool_blocks; Reindex: csa2_reindex over the pool of the latest Full layer that
 *   kept one; Reuse: none) and csa2_sparse_decode with the latest selection.  The
 *   graph runs exactly those calls on the buffers given here, so its results equal
 *   theirs; every pointer and the workspace must stay valid while the schedule
 *   exists, and their contents are read when the graph runs.  The first layer must
 *   be Full; a Reindex layer needs an earlier Full layer with pool_blocks > 0.
 *   Other arguments as in the single calls.  ws: csa2_schedule_workspace_size(...)
 *   bytes (device; no initialisation needed: every byte a launch reads was written
 *   earlier in the same launch); schedules that run at the same time need separate
 *   workspaces.  On success *out receives the schedule; on failure *out is NULL. */
int csa2_schedule_create(const csa2_cache_t *cache, int B, int H, const int32_t *ctx_len, int64_t max_ctx,
                         int topk, int cand_block, int W, float sm_scale, const int32_t *start_tok, int T_new,
                         const uint16_t *x, const uint16_t *w, const uint16_t *k_idx, int n_layers,
                         const csa2_layer_t *layers, void *ws, size_t ws_bytes, csa2_schedule_t **out);

/* Run the captured step on `stream` (asynchronous). */
int csa2_schedule_launch(csa2_schedule_t *schedule, void *stream);

/* Free the graph (host objects of the HIP runtime).  NULL is a no-op. */
void csa2_schedule_destroy(csa2_schedule_t *schedule);

/* csa2_debug_gather — test hook: dequantise entries through the page table with the
 *   same FP4 decode the kernels use.  idx: [B][n] int32 entry ids (device);
 *   out_lat: [B][n][512] float, out_idx: [B][n][64] float (device; either may be
 *   NULL).  An id < 0 or a page id outside [0, n_pages) yields NaN rows. */
int csa2_debug_gather(const csa2_cache_t *cache, int B, const int32_t *idx, int n, float *out_lat,
                      float *out_idx, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
