/*
 * CSA2 global-attention hot path: plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library and its binding) never calls it, and the two share no
 * code, header, table or constant.
 *
 * Everything here is the slow, obvious form of the definition: linear scans
 * over the format grids, full sorts for top-k, float64 attention.  The one
 * place the arithmetic is float32 on purpose is the indexer score, because
 * its value decides an integer (the top-k set) and the GPU must take that
 * decision in the same precision; its summation order is part of the
 * definition (see csa2o_score_one).
 *
 * Sources, cited by page and section:
 *   [KVC] "DeepSeek-V4.1-Flash KV Cache Compression" reading notes
 *         (jianyuh.github.io), sections 2-5.
 *   [SUM] DeepSeek-V4.1-Flash summary page (picx.dev), "Methodology /
 *         Architecture Components", items 2, 3 and 5.
 *   [DR]  "DeepSeek-V4.1-Flash: reading a model through its three memory
 *         costs", section 03 (CSA2 mode table) and 04.
 *   [THR] "Notes on DeepSeek V4.1 Flash" thread, posts 4-6 and 9.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared csa2_oracle.c -lm
 * (no fast-math: denormals are kept, nothing is contracted or reassociated).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* MXFP4 as the pages state it: E2M1 elements, one E4M3 scale per 16        */
/* channels, no second-level scale ([KVC] section 4; [SUM] item 5;          */
/* [THR] post 6, "NVFP4 without the second scale").                          */
/* ------------------------------------------------------------------------ */

/* E2M1 nibble: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent 0 is subnormal: value = mantissa * 0.5. */
double csa2o_e2m1_value(int nibble)
{
    int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* E4M3 byte, OCP "FN" variant: bit 7 sign, bits 6..3 exponent (bias 7),
 * bits 2..0 mantissa, no infinities, S.1111.111 is NaN, largest 448. */
double csa2o_e4m3_value(int byte)
{
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Scale = E4M3 value nearest to amax/6 (round to nearest, ties to the even
 * code), saturating at 448.  Walks the ascending non-negative finite codes
 * 0..126 and compares amax with 6 * (midpoint of neighbours); 6 * midpoint
 * has at most 7 significant bits, so every comparison is exact. */
static int scale_code_for(double amax)
{
    for (int c = 0; c < 126; ++c) {
        double t = 3.0 * (csa2o_e4m3_value(c) + csa2o_e4m3_value(c + 1));
        if (amax < t) return c;
        if (amax == t) return (c & 1) ? c + 1 : c;
    }
    return 126;
}

/* E2M1 magnitude code nearest to a/s (ties to even code, saturating at 6):
 * compares a with s * midpoint, exact for the same reason as above. */
static int mag_code_for(double a, double s)
{
    for (int c = 0; c < 7; ++c) {
        double t = s * 0.5 * (csa2o_e2m1_value(c) + csa2o_e2m1_value(c + 1));
        if (a < t) return c;
        if (a == t) return (c & 1) ? c + 1 : c;
    }
    return 7;
}

/* Encode n_rows rows of D channels (D % 16 == 0).  Per row: D/2 code bytes
 * (channel 2j in the low nibble of byte j, channel 2j+1 in the high nibble)
 * and D/16 scale bytes.  A block whose scale rounds to zero gets scale byte
 * 0 and zero codes; a zero magnitude always has sign bit 0. */
void csa2o_mxfp4_encode(const float *x, int64_t n_rows, int D, uint8_t *codes, uint8_t *scales)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        const float *xr = x + r * D;
        uint8_t *cr = codes + r * (D / 2);
        uint8_t *sr = scales + r * (D / 16);
        memset(cr, 0, (size_t)(D / 2));
        for (int blk = 0; blk < D / 16; ++blk) {
            double amax = 0.0;
            for (int i = 0; i < 16; ++i) {
                double a = fabs((double)xr[blk * 16 + i]);
                if (a > amax) amax = a;
            }
            int sc = scale_code_for(amax);
            sr[blk] = (uint8_t)sc;
            if (sc == 0) continue;
            double s = csa2o_e4m3_value(sc);
            for (int i = 0; i < 16; ++i) {
                int c = blk * 16 + i;
                double v = (double)xr[c];
                int mag = mag_code_for(fabs(v), s);
                int nib = mag | ((v < 0.0 && mag != 0) ? 8 : 0);
                cr[c / 2] |= (uint8_t)(nib << (4 * (c & 1)));
            }
        }
    }
}

/* Decode: value = E2M1(nibble) * E4M3(scale), exact in float64. */
void csa2o_mxfp4_decode(const uint8_t *codes, const uint8_t *scales, int64_t n_rows, int D, double *out)
{
    for (int64_t r = 0; r < n_rows; ++r)
        for (int c = 0; c < D; ++c) {
            int nib = (codes[r * (D / 2) + c / 2] >> (4 * (c & 1))) & 15;
            out[r * D + c] = csa2o_e2m1_value(nib) * csa2o_e4m3_value(scales[r * (D / 16) + c / 16]);
        }
}

/* ------------------------------------------------------------------------ */
/* Indexer-K projection.  A Full layer projects its indexer K directly from  */
/* its main KV ([KVC] section 2).  The pages give neither the weights nor    */
/* the precision; this library reads it as a projection of the latent row   */
/* before MXFP4 encoding (the row the entry is made from), with float32     */
/* weights W[D][d_I]:                                                        */
/*   acc = +0; for c = 0..D-1: acc = fma(x[c], W[c][j], acc)                 */
/*   k[j] = acc rounded to bfloat16 (nearest, ties to the even mantissa)     */
/* ------------------------------------------------------------------------ */

/* The bfloat16 nearest to a finite float: of the two bfloat16 values that
 * bracket f (f with its low 16 bits cleared, and the next bfloat16 away
 * from zero), the closer one; at equal distance the one whose last mantissa
 * bit is 0.  Returns the bfloat16 bit pattern. */
static uint16_t bf16_nearest(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lo = u & 0xffff0000u, hi = lo + 0x10000u;
    float flo, fhi;
    memcpy(&flo, &lo, 4);
    memcpy(&fhi, &hi, 4);
    double dlo = fabs((double)f - (double)flo), dhi = fabs((double)fhi - (double)f);
    if (dlo < dhi) return (uint16_t)(lo >> 16);
    if (dhi < dlo) return (uint16_t)(hi >> 16);
    return ((lo >> 16) & 1u) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);
}

uint16_t csa2o_bf16_nearest(float f) { return bf16_nearest(f); }

void csa2o_project_kidx(const float *x, int64_t n_rows, int D, const float *W, int d_I, uint16_t *out)
{
    for (int64_t r = 0; r < n_rows; ++r)
        for (int j = 0; j < d_I; ++j) {
            float acc = 0.0f;
            for (int c = 0; c < D; ++c) acc = fmaf(x[r * D + c], W[(int64_t)c * d_I + j], acc);
            out[r * d_I + j] = bf16_nearest(acc);
        }
}

/* ------------------------------------------------------------------------ */
/* Indexer score.  The pages give no formula ([KVC] sections 2-3 say only   */
/* that Full mode scores every visible entry with its own indexer Q against */
/* an indexer K projected from main KV; [DR] section 03).  This library     */
/* fixes  s_t = sum_h w_h * ReLU(q_h . k_t)  with one key vector per        */
/* position shared by all indexer heads, evaluated in float32 as fma chains:*/
/*   d_h = +0; for c = 0..d_I-1: d_h = fma(q[h][c], k[c], d_h)              */
/*   r_h = d_h > 0 ? d_h : +0                                               */
/*   s   = +0; for h = 0..H_I-1: s = fma(w[h], r_h, s)                      */
/* ------------------------------------------------------------------------ */
float csa2o_score_one(const float *q, const float *w, const float *k, int H_I, int d_I)
{
    float s = 0.0f;
    for (int h = 0; h < H_I; ++h) {
        float d = 0.0f;
        for (int c = 0; c < d_I; ++c) d = fmaf(q[h * d_I + c], k[c], d);
        float r = d > 0.0f ? d : 0.0f;
        s = fmaf(w[h], r, s);
    }
    return s;
}

/* Full mode over one query: scores[t] for t < vis, -inf for vis <= t < n_out
 * ([KVC] section 2, Full mode: "scores the entire visible context"). */
void csa2o_full_scores(const float *q, const float *w, const float *kcache, int H_I, int d_I,
                       int64_t vis, int64_t n_out, float *scores)
{
    for (int64_t t = 0; t < n_out; ++t)
        scores[t] = (t < vis) ? csa2o_score_one(q, w, kcache + t * d_I, H_I, d_I) : -INFINITY;
}

/* Block maxima for the candidate pool ([KVC] section 3, step 1): block b
 * covers positions [8b, 8b+8); its value is the largest visible score in it,
 * -inf when none of its positions is visible.  Zero is reported as +0. */
void csa2o_block_max(const float *scores, int64_t vis, int64_t n_blocks, float *bm)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        float m = -INFINITY;
        for (int64_t t = 8 * b; t < 8 * b + 8 && t < vis; ++t)
            if (scores[t] > m) m = scores[t];
        bm[b] = (m == 0.0f) ? 0.0f : m;
    }
}

/* ------------------------------------------------------------------------ */
/* Top-k selection ([KVC] sections 2-3; ties go to the lower index).        */
/* Order: a before b iff v_a > v_b, or v_a == v_b and pos_a < pos_b (so -0  */
/* and +0 tie).  -inf entries are never selected.  The first min(k, #finite)*/
/* entries are returned in ascending position order, then -1 padding.       */
/* ------------------------------------------------------------------------ */
typedef struct { float v; int64_t pos; } cand_t;

static int cand_cmp(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->pos < b->pos) ? -1 : (a->pos > b->pos);
}

static int pos_cmp(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

static int64_t select_sorted(cand_t *c, int64_t nc, int64_t k, int32_t *out)
{
    qsort(c, (size_t)nc, sizeof(cand_t), cand_cmp);
    int64_t take = nc < k ? nc : k;
    for (int64_t i = 0; i < take; ++i) out[i] = (int32_t)c[i].pos;
    qsort(out, (size_t)take, sizeof(int32_t), pos_cmp);
    for (int64_t i = take; i < k; ++i) out[i] = -1;
    return take;
}

/* Top-k over vals[0..n): position = array index. */
int64_t csa2o_topk(const float *vals, int64_t n, int64_t k, int32_t *out)
{
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
    int64_t nc = 0;
    for (int64_t i = 0; i < n; ++i)
        if (vals[i] != -INFINITY) { c[nc].v = vals[i]; c[nc].pos = i; ++nc; }
    int64_t r = select_sorted(c, nc, k, out);
    free(c);
    return r;
}

/* ------------------------------------------------------------------------ */
/* Reindex over the candidate pool ([KVC] section 3, steps 2-3; [DR] 03).   */
/* Pool slot s stands for position 8*pool[s/8] + s%8; a slot whose block id */
/* is -1 or whose position is not visible scores -inf.                      */
/* ------------------------------------------------------------------------ */
void csa2o_pool_scores(const float *q, const float *w, const float *kcache, int H_I, int d_I,
                       int64_t vis, const int32_t *pool, int P_b, float *scores)
{
    for (int64_t s = 0; s < (int64_t)P_b * 8; ++s) {
        int32_t b = pool[s / 8];
        int64_t pos = (int64_t)b * 8 + s % 8;
        scores[s] = (b >= 0 && pos < vis) ? csa2o_score_one(q, w, kcache + pos * d_I, H_I, d_I)
                                          : -INFINITY;
    }
}

/* Top-k among pool slots, ties broken by the lower position; returns
 * positions (ascending, -1 padded). */
int64_t csa2o_pool_topk(const float *scores, const int32_t *pool, int P_b, int64_t k, int32_t *out)
{
    int64_t n = (int64_t)P_b * 8;
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)n);
    int64_t nc = 0;
    for (int64_t s = 0; s < n; ++s)
        if (scores[s] != -INFINITY) {
            c[nc].v = scores[s];
            c[nc].pos = (int64_t)pool[s / 8] * 8 + s % 8;
            ++nc;
        }
    int64_t r = select_sorted(c, nc, k, out);
    free(c);
    return r;
}

/* ------------------------------------------------------------------------ */
/* Sparse attention ([DR] 03: selected main-KV entries joined with the local*/
/* SWA KV, then one softmax attention; [THR] post 4: selection on the main  */
/* KV, concatenation with the windowed KV, then attention).  The latent is  */
/* both key and value; every query head reads the same rows.  Float64.      */
/* ------------------------------------------------------------------------ */
static void attend_rows(const float *q, int H, int D, const double *rows, int64_t n_rows,
                        double sm_scale, float *out)
{
    if (n_rows == 0) {
        memset(out, 0, sizeof(float) * (size_t)H * (size_t)D);
        return;
    }
    double *z = (double *)malloc(sizeof(double) * (size_t)n_rows);
    double *acc = (double *)malloc(sizeof(double) * (size_t)D);
    for (int h = 0; h < H; ++h) {
        const float *qh = q + (int64_t)h * D;
        double zmax = -INFINITY;
        for (int64_t j = 0; j < n_rows; ++j) {
            double dot = 0.0;
            for (int c = 0; c < D; ++c) dot += (double)qh[c] * rows[j * D + c];
            z[j] = sm_scale * dot;
            if (z[j] > zmax) zmax = z[j];
        }
        double l = 0.0;
        for (int c = 0; c < D; ++c) acc[c] = 0.0;
        for (int64_t j = 0; j < n_rows; ++j) {
            double p = exp(z[j] - zmax);
            l += p;
            for (int c = 0; c < D; ++c) acc[c] += p * rows[j * D + c];
        }
        for (int c = 0; c < D; ++c) out[(int64_t)h * D + c] = (float)(acc[c] / l);
    }
    free(z);
    free(acc);
}

/* Decode query: rows = decoded main-KV rows idx[0..k) (entries equal to -1
 * skipped, duplicates kept) followed by SWA rows 0..swa_len-1. */
void csa2o_attn_decode(const float *q, int H, int D, const uint8_t *codes, const uint8_t *scales,
                       const int32_t *idx, int k, const float *swa, int swa_len, double sm_scale,
                       float *out)
{
    int64_t n = 0;
    for (int j = 0; j < k; ++j) n += (idx[j] >= 0);
    n += swa_len;
    double *rows = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)D);
    int64_t r = 0;
    for (int j = 0; j < k; ++j) {
        if (idx[j] < 0) continue;
        int64_t p = idx[j];
        csa2o_mxfp4_decode(codes + p * (D / 2), scales + p * (D / 16), 1, D, rows + r * D);
        ++r;
    }
    for (int i = 0; i < swa_len; ++i, ++r)
        for (int c = 0; c < D; ++c) rows[r * D + c] = (double)swa[(int64_t)i * D + c];
    attend_rows(q, H, D, rows, n, sm_scale, out);
    free(rows);
}

/* ------------------------------------------------------------------------ */
/* Prefill chunk (encoder at m tokens per entry, [KVC] section 2 layout).   */
/* Query t sits at absolute token position q_pos[t]; the entries it sees    */
/* are the complete m-blocks before and including it:                      */
/*   vis(t) = min(ctx_len, floor((q_pos[t] + 1) / m)).                      */
/* ------------------------------------------------------------------------ */
int64_t csa2o_prefill_vis(int64_t q_pos, int64_t ctx_len, int m)
{
    int64_t v = (q_pos + 1) / m;
    return v < ctx_len ? v : ctx_len;
}

void csa2o_prefill_scores(const float *q, const float *w, const float *kcache, int H_I, int d_I,
                          const int64_t *q_pos, int64_t T, int64_t ctx_len, int m, int64_t ld,
                          float *scores)
{
    for (int64_t t = 0; t < T; ++t)
        csa2o_full_scores(q + t * H_I * d_I, w + t * H_I, kcache, H_I, d_I,
                          csa2o_prefill_vis(q_pos[t], ctx_len, m), ld, scores + t * ld);
}

/* Prefill attention for query t: its own idx row, plus the window
 * [max(swa_start, i - W + 1), i] with i = q_pos0 + t ([KVC] section 5 gives
 * the window [max(s, i - n_win + 1), i]).  The window buffer holds T + W - 1
 * rows; row r is token position q_pos0 - (W - 1) + r. */
void csa2o_attn_prefill(const float *q, int64_t T, int H, int D, const uint8_t *codes,
                        const uint8_t *scales, const int32_t *idx, int k, const float *swa, int W,
                        int64_t q_pos0, int64_t swa_start, double sm_scale, float *out)
{
    for (int64_t t = 0; t < T; ++t) {
        int64_t i = q_pos0 + t;
        int64_t lo = i - W + 1;
        if (lo < swa_start) lo = swa_start;
        if (lo < 0) lo = 0;
        int64_t nwin = i - lo + 1;
        if (nwin < 0) nwin = 0;
        const float *first = swa + (lo - (q_pos0 - (W - 1))) * D;
        csa2o_attn_decode(q + t * H * D, H, D, codes, scales, idx + t * k, k, first, (int)nwin,
                          sm_scale, out + t * H * D);
    }
}
