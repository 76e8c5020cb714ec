/*
 * csa.h -- C ABI of the CSA / HCA hybrid long-context attention library
 * (libcsa.so, gfx950).
 *
 * The operators follow the DeepSeek-V4 pages:
 *   - CSA: compress every m = 4 tokens' KV into one entry, score entries with
 *     the Lightning Indexer, keep the top-k, attend to those (llm-tech
 *     overview, "Compressed Sparse Attention"; kenelite analysis 5.1-5.3).
 *   - HCA: compress every m' = 128 tokens, attend densely (llm-tech overview,
 *     "Heavily Compressed Attention"; kenelite analysis section 6).
 *   - both add a 128-token sliding window of raw tokens and a per-head
 *     attention-sink logit (llm-tech overview, HCA section and "other
 *     architecture details"; kenelite analysis section 7).
 *   - KV rows keep RoPE dims in BF16 and the rest in FP8; the indexer runs in
 *     FP8 or MXFP4 (llm-tech overview, "other architecture details" and
 *     "FP4 Quantization-Aware Training"; kenelite analysis 8.2, 8.3).
 * Where the pages leave an operator open the library fixes it as stated at
 * each entry point.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless said otherwise; the caller owns all
 *     memory.  The library allocates nothing, keeps no state between calls
 *     and only enqueues work on `stream` (no synchronisation, no host copies).
 *   - Arguments are validated on the host before anything is enqueued.  An
 *     invalid call returns CSA_EINVAL / CSA_EUNSUPPORTED / CSA_EWORKSPACE and
 *     writes nothing; a failed launch returns CSA_EHIP.  csa_last_error()
 *     gives a message for the last failure on the calling thread.
 *   - A call with no rows to process (B == 0, or T / Tq / n == 0 where the
 *     entry point takes one) enqueues nothing and returns CSA_OK as soon as
 *     its sizes are checked to be >= 0; no other argument is looked at, so
 *     its pointers may be NULL.
 *   - Results are deterministic: fixed reduction orders, no float atomics.
 *   - Query, output and partial-result arrays of the attention entry points
 *     (q, out, part_out) must be 16-byte aligned; lse arrays 4-byte aligned.
 *   - Positions: a prefill query row t has position t.  A query at position
 *     t sees compressed entry j iff (j+1)*m - 1 <= t, i.e. the first
 *     n_t = min(n_entries, floor((t+1)/m)) entries, and the window positions
 *     max(0, t-W+1) .. t.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_EINVAL = 1,        /* bad argument (null, size, alignment, range)        */
  CSA_EUNSUPPORTED = 2,  /* valid but not implemented (format / shape combo)   */
  CSA_EWORKSPACE = 3,    /* workspace missing or too small                     */
  CSA_EHIP = 4           /* a HIP call or kernel launch failed                 */
} csa_status;

typedef enum {
  CSA_F32 = 0,           /* IEEE binary32                                     */
  CSA_BF16 = 1,          /* bfloat16                                          */
  CSA_FP8_E4M3 = 2,      /* OCP E4M3FN, per-row power-of-two fp32 scale        */
  CSA_MXFP4 = 3          /* OCP MX: E2M1 elements, one E8M0 per 32 elements    */
} csa_fmt;

/*
 * An entry store: rows of `dim` values for each of B batch elements.
 * Row r of batch element b starts at rows + (b*cap + r) * row_bytes.
 *   fmt CSA_F32      : dim float32; scales NULL; row_bytes = 4*dim.
 *   fmt CSA_FP8_E4M3 : dims [0, dim-rope_dim) as E4M3 codes of x/s, then
 *                      rope_dim BF16; s = scales[b*cap + r] (float32, a power
 *                      of two, the smallest with max|x| <= 448 s);
 *                      row_bytes = (dim - rope_dim) + 2*rope_dim.
 *   fmt CSA_MXFP4    : dim/2 bytes, element 2i in the low nibble of byte i;
 *                      scales = uint8 E8M0 [B][cap][dim/32]; rope_dim 0;
 *                      row_bytes = dim/2.
 * rows must be 16-byte aligned and row_bytes a multiple of 16 (4 for MXFP4
 * rows of 32 values).
 */
typedef struct {
  void* rows;
  void* scales;
  int64_t cap;
  int32_t dim;
  int32_t rope_dim;
  int32_t fmt;
  int32_t row_bytes;
} csa_store;

/*
 * Optional post-processing of stored KV rows (csa_compress_kv,
 * csa_decode_append) and of queries (attention entry points): RMSNorm, then
 * partial RoPE (10100 analysis, section 3 item 1, auxiliary optimisations:
 * RMSNorm on query / KV entries against logit blow-up, partial rotary
 * embedding for relative position; llm-tech overview, other architecture
 * details: the RoPE dims are the BF16 ones).  A NULL pointer to this struct
 * means none of it.
 *   norm_gain  DEVICE float [dim], 16-byte aligned, or NULL for no RMSNorm:
 *              y = x / sqrt(mean(x^2) + norm_eps) * norm_gain over the row
 *              (a query row is one head's dim values);
 *   rope_dims  trailing dims rotated: even, 0 <= rope_dims <= dim (0: none);
 *   rope_theta DEVICE float [rope_dims / 2]: pair i = dims (dim - rope_dims
 *              + 2 i, dim - rope_dims + 2 i + 1) of a row at position p turns
 *              by a = fl32(fl32(p) * rope_theta[i]):
 *              (x, y) -> (x cos a - y sin a, x sin a + y cos a);
 *   pos0       csa_compress_kv only: position of token row 0.  Compressed
 *              entry j is at pos0 + (j + 1) m - 1, the last token of its
 *              block (where it becomes visible); m = 1 rows at pos0 + j.
 * Decode appends use the new token's position for its window row and for
 * the entry it closes; queries use their own positions (row t, or q_pos).
 * The processed query is rounded to the query format before it is used
 * (BF16 queries stay BF16).
 */
typedef struct {
  const float* norm_gain;
  float norm_eps;
  int32_t rope_dims;
  const float* rope_theta;
  int64_t pos0;
} csa_norm_rope;

/* flags of the attention entry points */
#define CSA_ATTN_PARTIAL 1  /* attend to the compressed entries only: no window,
                               no sink; `out` is float32, normalised over those
                               entries, lse = ln sum_e exp(l_e) (-inf if none)  */
#define CSA_WIN_RING 2      /* the window store is a ring of W slots per batch
                               element; position p lives in slot p mod W      */
#define CSA_BATCH_INVARIANT 4  /* a row's result bits depend on its own inputs
                               only, whatever else is in the batch (the
                               default splits few-query calls to fill the
                               chip, and the split count follows B).  Calls
                               with Tq = 1 and a workspace split every list
                               at a fixed 512 entries and merge the splits in
                               a fixed order; other calls run one workgroup
                               per (query row, 64 heads) over the whole list */

/* diagnostic event counters (csa_diag_counters) */
#define CSA_DIAG_INDEXER_GIVEUPS 0      /* one-pass long-list indexer workgroups that
                                           stopped waiting for their query's other
                                           chunks and kept every key as a candidate   */
#define CSA_DIAG_INDEXER_WIDE_SELECT 1  /* final selections over more candidates than
                                           fit in LDS (heavy ties, or the above)      */
#define CSA_DIAG_COUNT 4

const char* csa_version(void);
const char* csa_status_string(int status);
const char* csa_last_error(void);   /* host string, per calling thread */

/*
 * csa_compress_kv -- learned block compression (kenelite analysis 5.2: each
 * token's contribution weight is learned, not average pooling; section 6 for
 * m' = 128), then quantisation into `out`.
 *
 * tok: [B] x [T][dim] token K/V (or indexer keys / queries), element type
 *   tok_fmt (CSA_F32 or CSA_BF16), batch element b at tok + b*tok_bstride
 *   elements, rows contiguous.
 * For block j < floor(T/m) (an incomplete tail block is not compressed):
 *   a_i = <x_{jm+i}, gate> + bias_i (i < m), alpha = softmax(a),
 *   c_j = sum_i alpha_i x_{jm+i}  (float32),
 * stored as row out_row0 + j of `out` in out.fmt.  m = 1 stores the tokens
 * themselves (alpha = 1 exactly): the raw-token window store and the
 * quantisation of indexer queries.
 * gate: [dim] float32; bias: [m] float32.  1 <= m <= 1024; dim in
 * {32, 64, 128, 256, 512}; MXFP4 output needs dim in {32, 64}.
 * Writes floor(T/m) rows per batch element; out_row0 + floor(T/m) <= out.cap.
 * post (nullable): RMSNorm and partial RoPE of each entry before it is
 * quantised (see csa_norm_rope).
 */
csa_status csa_compress_kv(const void* tok, int tok_fmt, int B, int64_t T, int64_t tok_bstride,
                           int m, const float* gate, const float* bias,
                           csa_store out, int64_t out_row0, const csa_norm_rope* post,
                           hipStream_t stream);

/*
 * csa_decode_append -- cache maintenance for one decoded token per sequence
 * (the window keeps the latest raw tokens: llm-tech overview, HCA section;
 * only whole compression blocks enter the compressed cache, the incomplete
 * tail block stays raw: kenelite analysis 16, inference infrastructure).
 *
 * For each b < B with position p = pos[b] (device int64; p < 0: nothing):
 *   1. tail[b][p mod tail_rows] = tok[b]  (raw copy; tail is the caller's
 *      [B][tail_rows][dim] ring of tok_fmt, tail_rows a positive multiple of
 *      m, so a block's m rows are contiguous in it);
 *   2. if win.rows != NULL: row p mod W of win for b = tok[b] quantised to
 *      win.fmt (the bytes csa_compress_kv stores with m = 1);
 *   3. if (p + 1) mod m == 0: entry j = (p + 1)/m - 1 of out for b = the
 *      compression of tail rows for positions p+1-m .. p, with the gate,
 *      bias and arithmetic of csa_compress_kv (its bytes are identical to
 *      what csa_compress_kv stores for block j of the same tokens).  An entry
 *      at or past out.cap is not written (pos is only known on the device).
 * A decode step calls this once per cache: CSA KV (m = 4, with the window
 * store), CSA indexer keys (m = 4, win.rows = NULL), HCA KV (m' = 128).
 * Positions advance by one per call; the tail must hold the sequence's raw
 * tokens of its current block (from prefill, or earlier calls).
 * tok: [B][dim] (CSA_F32 or CSA_BF16), 16-byte aligned, as is tail.
 * dim, formats and rope_dim as for csa_compress_kv; win.dim == out.dim,
 * 1 <= W <= win.cap.  post (nullable) as for csa_compress_kv, at position p
 * for both the window row and the entry (pos0 is not used).
 */
csa_status csa_decode_append(const void* tok, int tok_fmt, int B, const int64_t* pos, void* tail, int tail_rows,
                             int m, const float* gate, const float* bias, csa_store out, csa_store win, int W,
                             const csa_norm_rope* post, hipStream_t stream);

/*
 * csa_decode_rebuild -- a sequence's decode state recomputed from raw tokens
 * (kenelite analysis, section 十六: compressed CSA / HCA caches restored for
 * a shared prefix need the tail of the incomplete compression block
 * recomputed, and with zero SWA caching the recent window is rebuilt rather
 * than stored).  After the caller restores the entries of the complete
 * blocks into `out`, this call recomputes the rest from the raw tokens of
 * the prefix's last positions.
 * For each b, rows tok[b][0 .. nb) (row i at tok + b * bstride + i * dim
 * elements; nb = min(n, n_valid[b]) with n_valid a DEVICE int32 [B], or n
 * when n_valid is NULL) are the raw tokens at positions p0[b] .. p0[b] +
 * nb - 1, where p0[b] (DEVICE int64 [B]) is a multiple of m; a sequence with
 * p0[b] < 0 or not a multiple of m is skipped (nothing written).  The stores
 * then hold, byte for byte, what nb calls of csa_decode_append at those
 * positions leave:
 *   - tail slot q mod tail_rows: the last min(nb, tail_rows) rows;
 *   - win (when win.rows != NULL) slot q mod W: the last min(nb, W) rows,
 *     quantised (and processed by post at position q);
 *   - out entry (q + 1)/m - 1 for every row q that ends a block (entries at
 *     or past out.cap are skipped); entries of earlier blocks are untouched.
 * To continue decoding at position P after restoring the entries of the
 * complete blocks below P, pass the raw tokens of positions p0 .. P - 1 with
 * p0 = the largest multiple of m at or below max(0, min(P - W, P)): the
 * window and the incomplete block are then rebuilt, and the blocks in
 * between recomputed with the bytes they were restored with.
 * tok: CSA_F32 or CSA_BF16, 16-byte aligned (bstride in elements keeps rows
 * aligned); tail, m, gate, bias, out, win, W and post as for
 * csa_decode_append.  Returns CSA_EINVAL on NULL or misaligned pointers,
 * n < 0, or bad store / window sizes.
 */
csa_status csa_decode_rebuild(const void* tok, int tok_fmt, int B, int n, int64_t bstride, const int64_t* p0,
                              const int32_t* n_valid, void* tail, int tail_rows, int m, const float* gate, const float* bias, csa_store out,
                              csa_store win, int W, const csa_norm_rope* post, hipStream_t stream);

/*
 * csa_indexer_topk -- Lightning Indexer scores and top-k selection
 * (llm-tech overview, CSA section: the indexer picks the top-k compressed
 * entries; kenelite analysis 5.3: top-512 Flash, top-1024 Pro).
 *
 * For query row q of batch element b at position t (q_pos[b*Tq + q], or
 * t = q when q_pos is NULL) and every visible entry j < n_t:
 *   I(t, j) = sum_h w[b][q][h] * ReLU(<qI[b][q][h], K[b][j]>)   (float32)
 * sel[b][q][0..k) receives the min(k, n_t) entries of largest I, ties to the
 * smaller j, in ascending j, padded with -1.
 *
 * q_idx: store of indexer queries, row (q*H_I + h) of batch element b, dim
 *   d_I, same format as `keys` (CSA_F32, CSA_FP8_E4M3 with rope_dim 0, or
 *   CSA_MXFP4).  head_w: float32 [B][Tq][H_I].  keys: the compressed indexer
 *   key store (dim d_I), first n_entries rows valid.
 * Limits: d_I in {32, 64}; 1 <= H_I <= 16; 1 <= k <= 2048;
 *   n_entries * k <= 32768 * 32768.
 * sel_score: float32 [B][Tq][k] or NULL.  When given, slot i receives the
 *   score I(t, sel[b][q][i]) exactly as the selection compared it (the
 *   float32 value behind its order key; -0 reads as +0) and padded slots
 *   -inf, so that the (score, index) pairs of several selections (of entry
 *   ranges held by different devices) can be merged into the same top-k.
 *   Queries that see at most k entries are then scored too (without it they
 *   are selected whole, unscored).  The selection itself is the same either way.
 * ws: device workspace of at least csa_indexer_topk_workspace(...) bytes
 *   (may be 0 bytes, then ws may be NULL).
 */
size_t csa_indexer_topk_workspace(int B, int Tq, int64_t n_entries, int k);
csa_status csa_indexer_topk(csa_store q_idx, const float* head_w, csa_store keys,
                            int64_t n_entries, const int64_t* q_pos, int B, int Tq, int H_I,
                            int m, int k, int32_t* sel, float* sel_score, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * csa_sparse_attn_prefill -- CSA core attention for T prefill queries
 * (kenelite analysis 5.1 "top-k compressed blocks -> core attention",
 * section 7 sliding window; llm-tech overview, attention sink).
 *
 * q: [B][T][H][dim] in q_fmt (CSA_F32 or CSA_BF16).  For query t, head h:
 *   entries E_t = {ckv[b][j] : j in sel[b][t][0..k), 0 <= j < n_entries}
 *               + {win[b][u] : max(0, t-W+1) <= u <= t}   (win has >= T rows),
 *   l_e = sm_scale * <q_{t,h}, e>,  M = max(sink_h, max_e l_e),
 *   o = sum_e exp(l_e - M) e / (exp(sink_h - M) + sum_e exp(l_e - M)),
 *   lse = M + ln(denominator).  K = V = the stored entry (all dim dims).
 * sink: float32 [H] or NULL (= -inf).  out: [B][T][H][dim] in q_fmt (float32
 * with CSA_ATTN_PARTIAL).  lse: float32 [B][T][H] or NULL.
 * Indices outside [0, n_entries) in sel are skipped.
 * q_post (nullable): RMSNorm and partial RoPE of each query head row at its
 * position before it is used (see csa_norm_rope; pos0 is not used).
 */
csa_status csa_sparse_attn_prefill(const void* q, int q_fmt, int B, int T, int H,
                                   csa_store ckv, int64_t n_entries, const int32_t* sel, int k,
                                   csa_store win, int W, const float* sink, float sm_scale,
                                   void* out, float* lse, int flags, const csa_norm_rope* q_post,
                                   hipStream_t stream);

/* Workspace bytes of csa_sparse_attn_decode / hca_attn for these sizes. */
size_t csa_attn_workspace(int B, int Tq, int H, int dim, int64_t max_list);

/*
 * csa_sparse_attn_decode -- CSA attention for one new token per sequence.
 * q: [B][H][dim]; sel: [B][k]; ring: window ring of W slots (position p in
 * slot p mod W) holding positions pos-W+1 .. pos; pos: int64 [B] (device).
 * Same arithmetic as the prefill.  ws: optional; NULL runs each sequence in
 * one workgroup per head group, otherwise >= csa_attn_workspace(B, 1, H,
 * dim, k + W) bytes (CSA_EWORKSPACE if smaller) lets long lists be split
 * across workgroups and merged in a fixed order.  q_post as for the prefill.
 */
csa_status csa_sparse_attn_decode(const void* q, int q_fmt, int B, int H, csa_store ckv,
                                  int64_t n_entries, const int32_t* sel, int k, csa_store ring,
                                  const int64_t* pos, int W, const float* sink, float sm_scale,
                                  void* out, float* lse, int flags, void* ws, size_t ws_bytes,
                                  const csa_norm_rope* q_post, hipStream_t stream);

/*
 * csa_sparse_attn_decode_noalloc -- csa_sparse_attn_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same operation, arguments
 * and results as csa_sparse_attn_decode, but the split partials go to a
 * scratch array the library holds in each device's memory (48 MiB per
 * device, held until the process ends) instead of a caller workspace.  The
 * call allocates nothing.  Sizes whose split partials need more than 48 MiB
 * (csa_attn_workspace(B, 1, H, dim, k + W) > 48 MiB) return CSA_EINVAL.
 * Every call on a device shares that device's scratch: calls that overlap in
 * time on one device (other streams, other threads) race and must not be
 * issued; calls on one stream are ordered and safe.  The scratch keeps the
 * last call's partials; nothing in it needs to start at zero.
 */
csa_status csa_sparse_attn_decode_noalloc(const void* q, int q_fmt, int B, int H, csa_store ckv,
                                          int64_t n_entries, const int32_t* sel, int k, csa_store ring,
                                          const int64_t* pos, int W, const float* sink, float sm_scale,
                                          void* out, float* lse, int flags, const csa_norm_rope* q_post,
                                          hipStream_t stream);

/*
 * hca_attn -- HCA dense attention (kenelite analysis section 6; model-card
 * notes: heavier compression with dense attention) over every visible entry
 * j < n_t = min(n_entries, floor((t+1)/m_prime)) plus the window and sink.
 * q: [B][Tq][H][dim].  q_pos: int64 [B][Tq] or NULL (prefill, t = row).
 * win: position-indexed raw rows, or a ring with CSA_WIN_RING.
 * ws: optional, as for csa_sparse_attn_decode, sized by
 * csa_attn_workspace(B, Tq, H, dim, n_entries + W) (0 for calls with enough
 * queries to fill the GPU).  q_post as for csa_sparse_attn_prefill.
 */
csa_status hca_attn(const void* q, int q_fmt, int B, int Tq, int H, csa_store hkv, int m_prime,
                    int64_t n_entries, const int64_t* q_pos, csa_store win, int W,
                    const float* sink, float sm_scale, void* out, float* lse, int flags,
                    void* ws, size_t ws_bytes, const csa_norm_rope* q_post, hipStream_t stream);

/*
 * swa_merge -- sliding-window attention merged with a partial result
 * (o_p, lse_p) of CSA_ATTN_PARTIAL, with the sink in the denominator:
 *   o = (e^{lse_p} o_p + sum_w e^{l_w} v_w) / (e^{lse_p} + sum_w e^{l_w} + e^{sink}).
 * part_out: float32 [B][Tq][H][dim]; part_lse: float32 [B][Tq][H].
 * q_pos / win / flags as in hca_attn (CSA_WIN_RING only).  out: q_fmt.
 * q_post as for csa_sparse_attn_prefill (the partial must come from the
 * same processed queries).
 */
csa_status swa_merge(const void* q, int q_fmt, int B, int Tq, int H, csa_store win,
                     const int64_t* q_pos, int W, int flags, const float* part_out,
                     const float* part_lse, const float* sink, float sm_scale, void* out,
                     const csa_norm_rope* q_post, hipStream_t stream);

/*
 * csa_diag_counters -- diagnostics for tests and benchmarks.
 * Copies min(n, CSA_DIAG_COUNT) event counters of the current device into
 * the HOST array out (uint64) and, if reset != 0, clears them.  Synchronises
 * the device first (not for use inside stream capture).  The counted events
 * leave results exact; they only cost time.
 *
 * Environment switches, read at each call of the entry points:
 *   CSA_INDEXER_SPIN_LIMIT=n  (0 <= n <= 65536) the number of polls a
 *       one-pass long-list indexer workgroup spends waiting for its query's
 *       other chunks before it stops waiting (default 65536); 0 makes every
 *       workgroup stop at once.  For tests of that path.
 *   CSA_DEBUG_SYNC=1  every entry point synchronises its stream after
 *       enqueueing and reports an asynchronous kernel failure as CSA_EHIP
 *       (not for use inside stream capture).
 */
csa_status csa_diag_counters(uint64_t* out, int n, int reset);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
