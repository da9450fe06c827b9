/*
 * csa2.h - C ABI of libcsa2, the MI355X (gfx950) CSA2 global-attention hot path.
 *
 * The path, per query (decode token or prefill token):
 *   1. score the visible compressed KV with the sparse indexer (Full mode:
 *      every visible entry; Reindex mode: the 16,384-position candidate pool),
 *   2. select the top-k positions,
 *   3. gather and dequantise the MXFP4 main KV of those positions,
 *   4. append the layer's sliding-window (SWA) KV,
 *   5. run one softmax attention over the joined set.
 * Reuse layers skip 1-2 and pass the previous layer's index list to step 5.
 *
 * Sources (page title, section):
 *   [KVC] "DeepSeek-V4.1-Flash KV Cache Compression" reading notes, sections 2-5.
 *   [SUM] DeepSeek-V4.1-Flash summary page, "Methodology / Architecture Components".
 *   [DR]  "DeepSeek-V4.1-Flash: reading a model through its three memory costs",
 *         section 03 (mode table).
 *   [THR] "Notes on DeepSeek V4.1 Flash" thread, posts 4-6.
 *
 * Conventions for every call
 *   - Tensor arguments are DEVICE pointers owned by the caller (row-major,
 *     contiguous unless a leading dimension is given).  Argument structs and
 *     scalars live on the host.  The library never allocates, frees or
 *     synchronises: scratch comes from the caller's (ws, ws_bytes), sized by
 *     the matching *_workspace_size call (0 means none is needed).
 *   - `stream` is a hipStream_t passed as void* (NULL = legacy default
 *     stream).  Work is enqueued asynchronously on it, on the current device.
 *   - Return value: CSA2_OK, or an error code; csa2_last_error() then holds a
 *     message (thread-local).  No C++ exception crosses the ABI.  Argument
 *     errors are detected on the host before anything is enqueued.
 *   - Data preconditions that live in device memory are not validated on the
 *     host: inputs must be finite; index/position entries outside [0, cap)
 *     are treated as empty (-1) by the kernels rather than read.
 *   - Index lists are int32 entry positions, ascending, padded with -1.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum csa2_status {
    CSA2_OK = 0,
    CSA2_E_INVALID = 1,     /* null pointer, bad shape or size, bad dtype value */
    CSA2_E_UNSUPPORTED = 2, /* shape valid in principle but not instantiated here */
    CSA2_E_WORKSPACE = 3,   /* ws is NULL or ws_bytes below the *_workspace_size value */
    CSA2_E_DEVICE = 4       /* a HIP launch or runtime call failed */
};

enum csa2_dtype { CSA2_F32 = 0, CSA2_BF16 = 1 };

const char *csa2_version(void);
const char *csa2_last_error(void);

/* ------------------------------------------------------------------------
 * mxfp4_kv_write - quantise main-KV rows into the MXFP4 cache and append
 * indexer-K rows.  Format ([KVC] section 4; [SUM] item 5): per block of 16
 * consecutive channels one E4M3 scale byte (OCP FN encoding, sign 0) and 16
 * E2M1 nibbles; no second-level scale.
 *   scale = E4M3 value nearest to amax/6 (ties to the even code, saturating
 *           at 448; amax = largest |x| of the block),
 *   code  = E2M1 value nearest to |x|/scale (ties to even, saturating at 6),
 *           sign bit set only for a nonzero negative code; a scale of 0
 *           gives all-zero codes.
 *   Channel 2j is the low nibble of code byte j.
 *
 * x          [n_rows][D] (x_dtype: CSA2_F32 or CSA2_BF16)
 * dst_row    [n_rows] int64, flat destination row b*cap + pos; rows outside
 *            [0, n_cache_rows) are skipped
 * codes      [n_cache_rows][D/2] uint8   (written at dst rows)
 * scales     [n_cache_rows][D/16] uint8  (written at dst rows)
 * idx_k_rows [n_rows][d_I] (idx_k_dtype) or NULL; when given, row i is
 *            copied unchanged to flat row dst_row[i] of idx_k_cache, which
 *            uses the TILED indexer-K layout described at csa2_index_score
 *            (n_cache_rows % 64 == 0, d_I * elem_size % 16 == 0).
 * Requires D % 16 == 0, n_rows >= 0.
 * ------------------------------------------------------------------------ */
int mxfp4_kv_write(const void *x, int x_dtype, int64_t n_rows, int32_t D,
                   const int64_t *dst_row, int64_t n_cache_rows, uint8_t *codes, uint8_t *scales,
                   const void *idx_k_rows, int idx_k_dtype, int32_t d_I, void *idx_k_cache,
                   void *stream);

/* ------------------------------------------------------------------------
 * csa2_kv_write_project - mxfp4_kv_write with the indexer key derived from
 * the same rows instead of passed in.  A Full layer projects its indexer K
 * directly from its main KV ([KVC] section 2); the pages give neither the
 * weights nor the precision, and this library reads the projection as
 *     acc = +0; for c in 0..D-1: acc = fma(x[c], w_ik[c][j], acc)   (float32)
 *     k[j] = acc rounded to the nearest bfloat16 (ties to the even mantissa;
 *            a value past the largest finite bfloat16 stays finite)
 * over the pre-quantisation latent row x (bf16 inputs widened exactly), so
 * the indexer keys, and every score and index chosen from them, are
 * bit-reproducible.  One launch does both jobs.
 *
 * x           [n_rows][D] (x_dtype: CSA2_F32 or CSA2_BF16), 16-byte aligned
 * dst_row     [n_rows] int64 flat destination rows; rows outside
 *             [0, n_cache_rows) are skipped (codes, scales and key alike)
 * codes, scales  as mxfp4_kv_write
 * w_ik        [D][d_I] float32 projection weights, row-major (device), 16-byte aligned
 * idx_k_cache bfloat16, TILED layout (see csa2_index_score), n_cache_rows
 *             rows of d_I; 16-byte aligned
 * Requires D % 16 == 0, d_I % 8 == 0, n_cache_rows % 64 == 0 (else
 * CSA2_E_INVALID), D <= 512 (else CSA2_E_UNSUPPORTED: a workgroup keeps 32
 * latent rows and a 32-column weight slice in LDS), and x, w_ik and
 * idx_k_cache 16-byte aligned.  Caller owns every buffer; nothing is allocated.
 * ------------------------------------------------------------------------ */
int csa2_kv_write_project(const void *x, int x_dtype, int64_t n_rows, int32_t D,
                          const int64_t *dst_row, int64_t n_cache_rows, uint8_t *codes,
                          uint8_t *scales, const float *w_ik, int32_t d_I, void *idx_k_cache,
                          void *stream);

/* ------------------------------------------------------------------------
 * csa2_index_score - sparse-indexer scores ([KVC] sections 2-3; [DR] 03).
 * The pages give no score formula; this library fixes
 *     s_t = sum_h w_h * ReLU(q_h . k_t)
 * with one indexer key per position shared by all H_I heads, in float32 as
 * ordered fma chains (bf16 inputs widened exactly):
 *     d_h = +0; for c in 0..d_I-1: d_h = fma(q[h][c], k_t[c], d_h)
 *     s   = +0; for h in 0..H_I-1: s = fma(w[h], d_h > 0 ? d_h : +0, s)
 * so the scores, and every index chosen from them, are bit-reproducible.
 *
 * A query row is (b, t).  Its visible entry count is
 *     vis = ctx_len[b]                                   (q_pos == NULL)
 *     vis = min(ctx_len[b], floor((q_pos[b][t] + 1) / m)) (q_pos given:
 *           only complete m-token blocks are visible, [KVC] section 2)
 * Full mode (pool_blocks == NULL): scores[row][j] for j < ld_scores is s_j
 *     when j < vis, else -inf.  If block_max != NULL it also writes
 *     block_max[row][b] for b < ceil(ld_scores/8): the largest visible score
 *     in positions [8b, 8b+8) (-inf if none; zero reported as +0), the input
 *     of csa2_build_candidate_pool ([KVC] section 3, step 1).
 * Indexer-K cache layout (TILED): k_idx holds B*cap flat rows (flat row
 *     r = b*cap + pos, cap % 64 == 0) of d_I elements, grouped in tiles of
 *     64 consecutive rows.  With NCH = d_I*elem_size/16 sixteen-byte chunks
 *     per row, chunk c of flat row r is stored at byte offset
 *         ((r / 64) * NCH + c) * 1024 + (r % 64) * 16.
 *     A wave then reads chunk c of 64 positions as one contiguous 1 KiB
 *     block and each lane receives its own row's chunk (the fma chain needs
 *     one lane per position walking every channel in order).
 * Reindex mode (pool_blocks != NULL, [P_b] per row, ascending, -1 padded):
 *     scores[row][s] for s < 8*P_b scores position 8*pool[s/8] + s%8, or
 *     -inf when the block id is -1 or the position is not visible.
 *     ld_scores must be >= 8*P_b; block_max must be NULL.
 * ------------------------------------------------------------------------ */
typedef struct csa2_score_args {
    const void *q_idx;  int32_t q_dtype;  /* [B][Tq][H_I][d_I] */
    const float *w;                       /* [B][Tq][H_I] */
    const void *k_idx;  int32_t k_dtype;  /* B*cap rows of d_I, tiled layout, 16-byte aligned */
    int64_t B, Tq, cap;
    int32_t H_I, d_I;
    const int32_t *ctx_len;               /* [B] */
    const int64_t *q_pos;                 /* [B][Tq] or NULL */
    int32_t m;                            /* tokens per entry (>= 1) */
    const int32_t *pool_blocks;           /* [B][Tq][P_b] or NULL */
    int32_t P_b;
    float *scores;  int64_t ld_scores;    /* [B][Tq][ld_scores] */
    float *block_max;                     /* [B][Tq][ceil(ld_scores/8)] or NULL */
} csa2_score_args;

size_t csa2_index_score_workspace_size(const csa2_score_args *a);
int csa2_index_score(const csa2_score_args *a, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * csa2_write_and_score - a decode token's cache write ([KVC] section 4, as
 * mxfp4_kv_write) and the first scan of its step (as csa2_index_score, Full
 * or Reindex mode) in one launch.  The results are those of
 *     mxfp4_kv_write(x, x_dtype, a->B, D, dst_row, a->B * a->cap, codes,
 *                    scales, idx_k_rows, a->k_dtype, a->d_I, a->k_idx)
 *     csa2_index_score(a)
 * in that order, with one rule on the rows: sequence b's entry is written
 * only when dst_row[b] lies in sequence b (b*cap <= dst_row[b] < (b+1)*cap);
 * any other row is skipped (nothing written, nothing scored differently).
 * The scan reads each new entry's indexer key from idx_k_rows, so no part
 * of the launch reads a row another part writes.
 *
 * x          [B][D] new main-KV rows (CSA2_F32 or CSA2_BF16), 16-byte aligned
 * dst_row    [B] int64 flat destination rows (see above)
 * codes, scales  the MXFP4 cache (as mxfp4_kv_write), codes 8-byte aligned
 * idx_k_rows [B][d_I] new indexer keys in a->k_dtype, 16-byte aligned
 * a          as csa2_index_score, with Tq == 1; a->k_idx is the tiled
 *            indexer cache that receives the keys
 * Errors: those of csa2_index_score; Tq != 1, bad D (D % 16 != 0) or
 * x_dtype, null or misaligned pointers give CSA2_E_INVALID; D/16 plus the
 * indexer row's 16-byte chunks above 256 gives CSA2_E_UNSUPPORTED.  No
 * workspace is needed (ws may be NULL).  Caller owns every buffer.
 * ------------------------------------------------------------------------ */
int csa2_write_and_score(const void *x, int x_dtype, int32_t D, const int64_t *dst_row, uint8_t *codes,
                         uint8_t *scales, const void *idx_k_rows, const csa2_score_args *a, void *ws,
                         size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * csa2_topk - exact top-k per row ([KVC] sections 2-3): order by score
 * descending, then slot ascending (-0 equals +0); -inf slots are never
 * chosen.  Writes min(k, #finite) entries in ascending order, then -1.
 * scores     [rows][ld] float32, n <= ld slots per row
 * pool_blocks NULL: the output entry is the slot itself (a position).
 *            else [rows][P_b] ascending block ids: slot s is position
 *            8*pool[row][s/8] + s%8 (n must equal 8*P_b), so slot order is
 *            position order and ties go to the lower position.
 * out_idx    [rows][k] int32
 * ------------------------------------------------------------------------ */
size_t csa2_topk_workspace_size(int64_t rows, int64_t n, int32_t k);
int csa2_topk(const float *scores, int64_t rows, int64_t n, int64_t ld, int32_t k,
              const int32_t *pool_blocks, int32_t P_b, int32_t *out_idx,
              void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * csa2_build_candidate_pool - the hierarchical indexer's pool ([KVC]
 * section 3, steps 1-2; [SUM] item 3): the P_b blocks (2,048 on the pages)
 * with the largest block maxima, ties to the lower block id, as ascending
 * block ids padded with -1.  Pool positions are 8b..8b+7 of each block.
 * block_max [rows][ld], n_blocks <= ld; out_blocks [rows][P_b].
 * For more than 32,768 blocks the selection runs through super-blocks of 8
 * blocks: by the same argument as at csa2_topk_from_pool, the P_b best
 * blocks all lie in the P_b best super-blocks (super-block value = max of its
 * block maxima, ties to the lower id), so it first picks those and then the
 * P_b best blocks among their 8*P_b blocks (exact, no workspace for
 * P_b <= 2048 and n_blocks <= 262,144; other sizes use csa2_topk's path).
 * ------------------------------------------------------------------------ */
size_t csa2_build_candidate_pool_workspace_size(int64_t rows, int64_t n_blocks, int32_t P_b);
int csa2_build_candidate_pool(const float *block_max, int64_t rows, int64_t n_blocks, int64_t ld,
                              int32_t P_b, int32_t *out_blocks, void *ws, size_t ws_bytes,
                              void *stream);

/* ------------------------------------------------------------------------
 * csa2_topk_from_pool - the Full-mode top-k of position-ordered score rows,
 * found inside the row's candidate pool.  Requires k <= P_b (and
 * 8*P_b <= 32768).  Then the k best positions (score desc, position asc)
 * all lie in the pool: a position t in a block b outside the pool is
 * preceded by the argmax position of each of the P_b pool blocks (each has
 * a larger block max, or an equal one and a lower block id, hence a lower
 * position), so t ranks below P_b >= k.  The result therefore equals
 * csa2_topk over the whole row, bit for bit, while reading only the 8*P_b
 * pool scores ([KVC] section 3: the first Full layer scores every position
 * and builds the pool in the same pass).
 * scores [rows][ld] (position order, -inf where invisible);
 * pool_blocks [rows][P_b] ascending, -1 padded (csa2_build_candidate_pool);
 * out_idx [rows][k] ascending positions, -1 padded.  No workspace.
 * ------------------------------------------------------------------------ */
int csa2_topk_from_pool(const float *scores, int64_t rows, int64_t ld, const int32_t *pool_blocks,
                        int32_t P_b, int32_t k, int32_t *out_idx, void *stream);

/* ------------------------------------------------------------------------
 * csa2_pool_topk - csa2_build_candidate_pool followed by csa2_topk_from_pool
 * in one launch ([KVC] section 3: the first Full layer scores every
 * position and builds the pool in the same pass).  Same outputs, bit for
 * bit, as the two calls: out_blocks [rows][P_b] as csa2_build_candidate_pool
 * writes it, out_idx [rows][k] as csa2_topk_from_pool writes it.  Two
 * workgroups per row run side by side: one selects and writes the pool, the
 * other selects the top-k among the scores of every block whose maximum
 * reaches a one-pass lower bound of the pool threshold (a superset of the
 * pool, so the same top-k).  Requires 0 < k <= P_b <= 2048,
 * n_blocks <= 32,768 (the pool selected directly, without super-blocks)
 * and rows <= 2^30; other sizes return CSA2_E_UNSUPPORTED (CSA2_E_INVALID
 * for rows) and the two calls remain.
 * block_max [rows][ld_bm]; scores [rows][ld] (position order, -inf where
 * invisible).  No workspace.
 * ------------------------------------------------------------------------ */
int csa2_pool_topk(const float *block_max, int64_t rows, int64_t n_blocks, int64_t ld_bm, int32_t P_b,
                   int32_t *out_blocks, const float *scores, int64_t ld, int32_t k, int32_t *out_idx,
                   void *stream);

/* ------------------------------------------------------------------------
 * csa2_sparse_attn_decode - gather, dequantise, join with SWA, attend
 * ([DR] 03; [THR] post 4).  For each sequence b and head h:
 *   rows  = [MXFP4 main rows idx[b][j] (j < k, entries -1 skipped)]
 *           ++ [swa[b][r] for r < min(swa_len[b], W)]
 *   z_j   = sm_scale * (q[b][h] . row_j);  p = softmax(z);  out = sum p_j row_j
 * The latent is both key and value and all H heads read the same rows.
 * An empty row set gives zeros.
 * q     [B][H][D] bf16 (or f32); codes [B][cap][D/2], scales [B][cap][D/16];
 * idx   [B][k] int32;  swa [B][W][D] bf16 (or f32);  swa_len [B] int32;
 * out   [B][H][D] float32.
 * Instantiated for D = 512 with H a multiple of 64, and for the small
 * parity shape D = 64 with H <= 64 (else CSA2_E_UNSUPPORTED).
 * Arithmetic: rows exactly in fp16 (every MXFP4 value is an fp16 number; q
 * and SWA values in [2^-14, 65504] convert exactly), MFMA with float32
 * accumulation, float32 softmax, probabilities rounded to fp16 for P.V.
 * ------------------------------------------------------------------------ */
typedef struct csa2_attn_args {
    const void *q;  int32_t q_dtype;
    const uint8_t *codes;  const uint8_t *scales;  int64_t cap;
    const int32_t *idx;  int32_t k;
    const void *swa;  int32_t swa_dtype;  int32_t W;  const int32_t *swa_len;
    int64_t B;  int32_t H, D;
    float sm_scale;
    float *out;
} csa2_attn_args;

size_t csa2_sparse_attn_decode_workspace_size(const csa2_attn_args *a);
int csa2_sparse_attn_decode(const csa2_attn_args *a, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * csa2_sparse_attn_decode_noalloc - csa2_sparse_attn_decode without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, kernels and outputs as
 * csa2_sparse_attn_decode; the key-split partials go to a scratch array of
 * CSA2_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one
 * copy per GPU, from the first call on that GPU until the process ends.
 * The call allocates nothing and calls no allocating routine.
 * Calls whose workspace (csa2_sparse_attn_decode_workspace_size) exceeds
 * CSA2_NOALLOC_SCRATCH_BYTES return CSA2_E_WORKSPACE and enqueue nothing.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in
 * time on one GPU (on different streams, or from different host threads
 * without ordering) race and give wrong results.  Calls ordered on one
 * stream are safe.  The scratch keeps the last call's partials; nothing in
 * it needs to start at zero.
 * ------------------------------------------------------------------------ */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int csa2_sparse_attn_decode_noalloc(const csa2_attn_args *a, void *stream);

/* ------------------------------------------------------------------------
 * csa2_sparse_attn_prefill - the same per query token of one sequence's
 * chunk.  Query t sits at token position i = q_pos0 + t and uses its own
 * idx[t] row plus the window [max(swa_start, i - W + 1), i] ([KVC] section
 * 5 writes the window as [max(s, i - n_win + 1), i]; swa_start = s, 0 when
 * nothing was replayed).  The window buffer holds T + W - 1 rows; row r is
 * token position q_pos0 - (W - 1) + r (rows before position 0 are unused).
 * q [T][H][D]; codes [cap][D/2]; scales [cap][D/16]; idx [T][k];
 * swa [T + W - 1][D]; out [T][H][D] float32.
 * ------------------------------------------------------------------------ */
typedef struct csa2_attn_prefill_args {
    const void *q;  int32_t q_dtype;
    const uint8_t *codes;  const uint8_t *scales;  int64_t cap;
    const int32_t *idx;  int32_t k;
    const void *swa;  int32_t swa_dtype;  int32_t W;
    int64_t q_pos0, swa_start;
    int64_t T;  int32_t H, D;
    float sm_scale;
    float *out;
} csa2_attn_prefill_args;

size_t csa2_sparse_attn_prefill_workspace_size(const csa2_attn_prefill_args *a);
int csa2_sparse_attn_prefill(const csa2_attn_prefill_args *a, void *ws, size_t ws_bytes,
                             void *stream);


/* ------------------------------------------------------------------------
 * csa2_prefill_topk - Full-mode top-k indices for a chunk of prefill query
 * tokens ([KVC] sections 1-2: encoder Full layers score every visible
 * entry; [KVC] section 2 for m-token entries).  The result is identical to
 * csa2_index_score (q_pos = q_pos0 + t, Tq = T, B = 1) followed by csa2_topk
 * with k: the same exact scores, the same (score desc, position asc) order.
 * The scores are formed on the matrix cores; keys whose approximate score
 * lies within a proven error band of the k-th are rescored with the exact
 * float32 chains, so no index differs.
 *
 * Query t (0 <= t < T) sits at absolute token position q_pos0 + t and sees
 * vis(t) = min(ctx_len, floor((q_pos0 + t + 1) / m)) entries.
 *   q_idx  [T][H_I][d_I] bf16, w [T][H_I] f32   (H_I = 8, d_I = 128 only)
 *   k_idx  one sequence's indexer cache, tiled layout (csa2_index_score),
 *          cap rows (cap % 64 == 0), bf16
 *   out_idx [T][k] int32: min(k, vis(t)) ascending positions, then -1.
 * 1 <= k <= 4096 and vis(T-1) <= 2^24 (CSA2_E_UNSUPPORTED beyond).  Inputs
 * must be finite with scores far from float32 overflow.  Workspace:
 * csa2_prefill_topk_workspace_size, 256-byte aligned: per row of a chunk of
 * min(T, 1024) rows, about 8.3 * vis(T-1) bytes of candidate slots, sample
 * scores and counts, plus 128 KiB.
 * ------------------------------------------------------------------------ */
typedef struct csa2_prefill_topk_args {
    const void *q_idx;  int32_t q_dtype;  /* [T][H_I][d_I] */
    const float *w;                       /* [T][H_I] */
    const void *k_idx;  int32_t k_dtype;  /* cap rows, tiled layout */
    int64_t T, cap;
    int32_t H_I, d_I;
    int32_t ctx_len;
    int64_t q_pos0;
    int32_t m;
    int32_t k;
    int32_t *out_idx;                     /* [T][k] */
} csa2_prefill_topk_args;

size_t csa2_prefill_topk_workspace_size(const csa2_prefill_topk_args *a);
int csa2_prefill_topk(const csa2_prefill_topk_args *a, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * csa2_decode_scan, csa2_decode_select - the decode Full layer's candidate
 * pool and top-k ([KVC] sections 2-3) from the indexer query, with the
 * products on the matrix cores.  csa2_decode_scan computes the approximate
 * scores, their block maxima and each row's largest key norm into the
 * workspace; csa2_decode_select, called next with the same arguments and
 * workspace (on the same stream, or after it), selects.  Together: the same
 * outputs, bit for bit, as csa2_index_score (Tq = 1, with block maxima)
 * followed by csa2_build_candidate_pool and csa2_topk_from_pool: the
 * approximate scores carry a proven error bound (from ||q_h||, |w_h| and
 * the row's largest key norm), and the keys and
 * blocks whose approximate value lies within that bound of a threshold are
 * rescored with the exact float32 chains.  A row whose band of such keys
 * outgrows the fixed on-chip budget is redone from exact scores (same
 * result, slower).
 *   q_idx [B][H_I][d_I] bf16, w [B][H_I] f32   (H_I = 8, d_I = 128 only)
 *   k_idx [B][cap] tiled indexer cache (csa2_index_score), bf16,
 *         cap % 64 == 0, cap <= 262,144
 *   ctx_len [B] int32 (device): visible entries per sequence
 *   out_pool [B][P_b] ascending block ids, -1 padded (P_b <= 2048)
 *   out_idx [B][k] ascending positions, -1 padded (1 <= k <= P_b)
 * Workspace: csa2_decode_select_workspace_size (4 B per cache entry, plus
 * block maxima and one key-norm maximum per 256 entries); 256-byte aligned.
 * Errors: CSA2_E_INVALID (bad arguments), CSA2_E_UNSUPPORTED (shape outside
 * this path), CSA2_E_WORKSPACE (short workspace); nothing is launched then.
 * ------------------------------------------------------------------------ */
typedef struct csa2_decode_select_args {
    const void *q_idx;  int32_t q_dtype;  /* [B][H_I][d_I] */
    const float *w;                       /* [B][H_I] */
    const void *k_idx;  int32_t k_dtype;  /* [B][cap] tiled */
    const int32_t *ctx_len;               /* [B] */
    int64_t B, cap;
    int32_t H_I, d_I;
    int32_t P_b, k;
    int32_t *out_pool;                    /* [B][P_b] */
    int32_t *out_idx;                     /* [B][k] */
} csa2_decode_select_args;

size_t csa2_decode_select_workspace_size(const csa2_decode_select_args *a);
int csa2_decode_scan(const csa2_decode_select_args *a, void *ws, size_t ws_bytes, void *stream);
int csa2_decode_select(const csa2_decode_select_args *a, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * csa2_mhc_step - one fused pass of single-pass mHC ([KVC] section 6; [SUM]
 * Methodology item 4, equation (6)).  The residual stream of a token is n
 * streams X_l [n][d]; the pages shift the input-mixing coefficient by one
 * block,
 *     X_{l+1} = B_l X_l + C_l F_l(A_{l-1} X_l),  (A_l, B_l, C_l) = H(X_l),
 * so that one read of X_l serves the residual update, the next block's input
 * mixing and the statistics of H.  Per token this call computes, from X_l,
 * the block output f_l = F_l(A_{l-1} X_l) and the coefficients (A_l, B_l, C_l)
 * of the previous pass:
 *     X_next = bf16(B_l X_l + C_l f_l)            (float32, rounded once)
 *     u_next = bf16(A_l X_next)                   (input of F_{l+1})
 *     (A_next, B_next, C_next) = H(X_next)
 * reading (n + 1) d and writing (n + 1) d bfloat16 values: the (2n+2)d bound.
 * H is not defined on the pages; this library reads it as the manifold-
 * constrained hyper-connection form over x = X_next flattened stream-major
 * (index i*d + c):
 *     r = sqrt(mean(x^2) + 1e-6),   z = (phiT . x) / r   (z has 2n + n^2 entries)
 *     A_next = sigmoid(alpha_pre * z[0:n] + bias[0:n])
 *     C_next = 2 * sigmoid(alpha_post * z[n:2n] + bias[n:2n])
 *     B_next = Sinkhorn_iters(exp(alpha_res * z[2n:] + bias[2n:]) as n x n,
 *              row-major), each round dividing every row by its sum, then
 *              every column by its sum.
 * The projection runs on the matrix cores in float32 accumulation and the
 * epilogue in float32, so A/B/C_next are not bit-reproducible across
 * implementations; X_next is within one bfloat16 ulp of the exactly rounded
 * value.
 *
 * Layouts (row-major, device pointers, caller-owned; nothing is allocated):
 *   X, X_next [T][n][d] bf16;  f, u_next [T][d] bf16;  phiT [2n+n^2][n*d] bf16;
 *   A, A_next, C, C_next [T][n] f32;  B, B_next [T][n][n] f32;  bias [2n+n^2] f32.
 * Supported: n = 4, d a multiple of 128 (else CSA2_E_UNSUPPORTED).  X, f, phiT,
 * X_next and u_next must be 16-byte aligned.  X_next must not alias X, nor u_next
 * f (CSA2_E_INVALID).
 * ------------------------------------------------------------------------ */
typedef struct csa2_mhc_args {
    const void *X;       /* [T][n][d] bf16 */
    const void *f;       /* [T][d] bf16 */
    const float *A;      /* [T][n] */
    const float *B;      /* [T][n][n] */
    const float *C;      /* [T][n] */
    const void *phiT;    /* [2n+n^2][n*d] bf16 */
    const float *bias;   /* [2n+n^2] */
    float alpha_pre, alpha_post, alpha_res;
    int64_t T;
    int32_t n, d, iters;
    void *X_next;        /* [T][n][d] bf16 */
    void *u_next;        /* [T][d] bf16 */
    float *A_next;       /* [T][n] */
    float *B_next;       /* [T][n][n] */
    float *C_next;       /* [T][n] */
} csa2_mhc_args;

int csa2_mhc_step(const csa2_mhc_args *args, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
