/*
 * bsp_oracle.c -- plain, slow CPU oracle for causal block-sparse prefill
 * attention with dynamic block skipping inside the online softmax.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this file. It shares no code, header, table or
 * helper with the HIP library; the product path never calls it.
 *
 * What it computes (page "长上下文推理加速方案部署实战：基于动态稀疏注意力机制的推理服务
 * 优化指南", sections 3.2 and 6.1): attention is evaluated as an online softmax
 * that keeps, per query row, the running maximum of the scores seen so far.
 * Key blocks are taken in ascending order. For each block the local maximum
 * score is formed; when the running maximum exceeds the block's local maximum
 * by more than a threshold lambda, the block is negligible and the softmax
 * exponentials, the V-block load and the product with V are all skipped. The
 * decision uses only quantities the online softmax already has.
 *
 * Readings taken where the page is silent (each is restated next to the code
 * that implements it):
 *   - lambda is a gap in natural-log units on scaled logits,
 *     score = <q, k> / sqrt(D); lambda = +inf means dense attention.
 *   - the block decision is taken for the whole query tile: a block is
 *     skipped only when EVERY valid row of the tile has gap > lambda (strict).
 *     A row with no unmasked key in the block has gap = +inf.
 *   - the running maximum is the maximum over the blocks kept so far; before
 *     the first block it is -inf, so block 0 is never skipped.
 *   - skipped keys leave both the numerator and the denominator.
 *   - causal masking per sequence: key c is visible to query r iff c <= r.
 *   - chunked prefill against a cached prefix (the FlowPrefill page, sections
 *     2.1 and 4.5.2, on prefill in fixed-size chunks): a sequence's queries are the LAST Lq of its Lk
 *     keys (bottom-right alignment), so query row r of the chunk sits at key
 *     position (Lk - Lq) + r and sees keys 0 .. (Lk - Lq) + r. Lq = Lk is the
 *     plain prefill.
 *   - lambda may be given per sequence (the guide's per-request threshold,
 *     sections 3.3 and 9.3).
 *   - LSE is m + ln(l) over the kept keys, natural log.
 *
 * Arithmetic: every input element is widened exactly to double from its
 * storage type (fp32; bf16 bit patterns; OCP fp8 e4m3 codes) and multiplied by
 * its per-head dequantisation scale (1 when none is given); all sums, maxima,
 * exponentials and logarithms are in double precision.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* forced[] entries: 0 = keep, 1 = skip, anything else = apply the rule. */
#define BSP_ORACLE_RULE 255

int bsp_oracle_version(void) { return 3; }

/* Storage types of the inputs. */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_FP8_E4M3 = 2 };

/* Value of an OCP fp8 e4m3 code: s.eeee.mmm with exponent bias 7, exponent
 * field 0 for subnormals (m/8 * 2^-6), 0x7F / 0xFF NaN, no infinities. */
static double fp8_e4m3_value(uint8_t c)
{
    const int e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return (c & 0x80) ? -mag : mag;
}

/* Element i of a storage array, widened exactly to double. */
static double elem(const void *base, size_t i, int dtype)
{
    if (dtype == ORACLE_F32) return (double)((const float *)base)[i];
    if (dtype == ORACLE_BF16) {
        const uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return fp8_e4m3_value(((const uint8_t *)base)[i]);
}

/*
 * bsp_oracle_fwd
 *
 * q  : [total_tokens][n_heads_q][head_dim]   storage type `in_dtype`
 * k,v: [total_tokens][n_heads_kv][head_dim]  same storage type
 * q_scale/k_scale/v_scale: double per head, or NULL (= 1.0)
 * cu_seqlens: int32 [n_seqs+1], cu[0] = 0, non-decreasing (query rows)
 * cu_seqlens_k: int32 [n_seqs+1] for the keys/values, or NULL (= cu_seqlens);
 *             each sequence needs Lk >= Lq
 * lambda_seq: double [n_seqs] per-sequence lambda, or NULL (= lambda)
 * work: int32 [n_work][3] = (sequence, query head, query tile)
 * forced: uint8 [n_work][j_max] or NULL
 * Outputs, per work item w (row r of the tile is query row t*block_q + r of
 * the sequence's chunk; key indices are sequence-local):
 *   o_out     double [n_work][block_q][head_dim]  (rows past the sequence: 0)
 *   lse_out   double [n_work][block_q]            (rows past the sequence: NaN)
 *   skip_out  uint8  [n_work][j_max]  1 = visited and skipped, 0 otherwise
 *   visit_out uint8  [n_work][j_max]  1 = block visited (causal), may be NULL
 *   mingap_out double [n_work][j_max] min over valid rows of the gap (NaN
 *                                     for blocks not visited), may be NULL
 *   p_out     double [n_work][block_q][p_cols] or NULL: the normalised
 *             probability of every key (sequence-local index) for each row;
 *             exactly 0 for masked and skipped keys.
 * Returns 0 on success, a negative number on invalid arguments.
 */
int bsp_oracle_fwd(const void *q, const void *k, const void *v, int in_dtype,
                   const double *q_scale, const double *k_scale, const double *v_scale,
                   const int32_t *cu_seqlens, const int32_t *cu_seqlens_k, int n_seqs,
                   int n_heads_q, int n_heads_kv, int head_dim,
                   int block_q, int block_k, double lambda, const double *lambda_seq,
                   const int32_t *work, int64_t n_work,
                   const uint8_t *forced, int j_max,
                   double *o_out, double *lse_out, uint8_t *skip_out, uint8_t *visit_out,
                   double *mingap_out, double *p_out, int p_cols, int n_threads)
{
    if (!q || !k || !v || !cu_seqlens || !work || !o_out || !lse_out || !skip_out)
        return -1;
    if (n_heads_q <= 0 || n_heads_kv <= 0 || n_heads_q % n_heads_kv != 0)
        return -2;
    if (head_dim <= 0 || block_q <= 0 || block_k <= 0 || j_max <= 0)
        return -3;
    if (isnan(lambda) || lambda < 0.0)
        return -4;
    if (lambda_seq)
        for (int s = 0; s < n_seqs; ++s)
            if (isnan(lambda_seq[s]) || lambda_seq[s] < 0.0) return -4;
    if (in_dtype < ORACLE_F32 || in_dtype > ORACLE_FP8_E4M3)
        return -6;
    const int group = n_heads_q / n_heads_kv;
    const double scale = 1.0 / sqrt((double)head_dim);
    const int D = head_dim;
    int bad = 0;

#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

#pragma omp parallel
    {
        double *qrow = (double *)malloc(sizeof(double) * (size_t)block_q * D);
        double *kblk = (double *)malloc(sizeof(double) * (size_t)block_k * D);
        double *vblk = (double *)malloc(sizeof(double) * (size_t)block_k * D);
        double *sc = (double *)malloc(sizeof(double) * (size_t)block_q * block_k);
        double *m = (double *)malloc(sizeof(double) * block_q);
        double *l = (double *)malloc(sizeof(double) * block_q);
        double *mloc = (double *)malloc(sizeof(double) * block_q);
        double *acc = (double *)malloc(sizeof(double) * (size_t)block_q * D);
        uint8_t *kept = (uint8_t *)malloc((size_t)j_max);

#pragma omp for schedule(dynamic, 1)
        for (int64_t w = 0; w < n_work; ++w) {
            const int s = work[3 * w + 0];
            const int h = work[3 * w + 1];
            const int t = work[3 * w + 2];
            double *o_w = o_out + (size_t)w * block_q * D;
            double *lse_w = lse_out + (size_t)w * block_q;
            uint8_t *skip_w = skip_out + (size_t)w * j_max;
            memset(o_w, 0, sizeof(double) * (size_t)block_q * D);
            for (int r = 0; r < block_q; ++r) lse_w[r] = NAN;
            memset(skip_w, 0, (size_t)j_max);
            if (visit_out) memset(visit_out + (size_t)w * j_max, 0, (size_t)j_max);
            if (mingap_out)
                for (int j = 0; j < j_max; ++j) mingap_out[(size_t)w * j_max + j] = NAN;
            if (p_out) memset(p_out + (size_t)w * block_q * p_cols, 0, sizeof(double) * (size_t)block_q * p_cols);
            if (s < 0 || s >= n_seqs || h < 0 || h >= n_heads_q || t < 0) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            const int base = cu_seqlens[s];
            const int L = cu_seqlens[s + 1] - base;                    /* query rows */
            const int kbase = cu_seqlens_k ? cu_seqlens_k[s] : base;
            const int Lk = cu_seqlens_k ? cu_seqlens_k[s + 1] - kbase : L;  /* keys */
            const int off = Lk - L;                 /* query row r sits at key position off + r */
            const double lam = lambda_seq ? lambda_seq[s] : lambda;
            if (off < 0) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            const int r0 = t * block_q;             /* first query of the tile */
            if (L <= 0 || r0 >= L) continue;        /* empty tile: nothing to do */
            const int r1 = (r0 + block_q < L) ? r0 + block_q : L;
            const int nrows = r1 - r0;
            /* causal: the last key block touched by the tile holds key off+r1-1 */
            const int nblk = (off + r1 - 1) / block_k + 1;
            if (nblk > j_max) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            const int g = h / group;                /* KV head of this query head */
            const double sq = q_scale ? q_scale[h] : 1.0;
            const double sk = k_scale ? k_scale[g] : 1.0;
            const double sv = v_scale ? v_scale[g] : 1.0;

            for (int r = 0; r < nrows; ++r)
                for (int d = 0; d < D; ++d)
                    qrow[(size_t)r * D + d] =
                        elem(q, ((size_t)(base + r0 + r) * n_heads_q + h) * D + d, in_dtype) * sq;

            /* online-softmax state per query row */
            for (int r = 0; r < nrows; ++r) {
                m[r] = -INFINITY;
                l[r] = 0.0;
            }
            memset(acc, 0, sizeof(double) * (size_t)nrows * D);

            for (int j = 0; j < nblk; ++j) {        /* key blocks in ascending order */
                const int c0 = j * block_k;
                const int c1 = (c0 + block_k < Lk) ? c0 + block_k : Lk;
                const int nc = c1 - c0;
                if (visit_out) visit_out[(size_t)w * j_max + j] = 1;
                for (int c = 0; c < nc; ++c)
                    for (int d = 0; d < D; ++d)
                        kblk[(size_t)c * D + d] =
                            elem(k, ((size_t)(kbase + c0 + c) * n_heads_kv + g) * D + d, in_dtype) * sk;

                /* scaled scores with the causal mask, and the block's local max */
                for (int r = 0; r < nrows; ++r) {
                    const int qi = off + r0 + r;        /* key position of this query */
                    double mx = -INFINITY;
                    for (int c = 0; c < nc; ++c) {
                        double val = -INFINITY;
                        if (c0 + c <= qi) {
                            double dot = 0.0;
                            for (int d = 0; d < D; ++d)
                                dot += qrow[(size_t)r * D + d] * kblk[(size_t)c * D + d];
                            val = scale * dot;
                        }
                        sc[(size_t)r * block_k + c] = val;
                        if (val > mx) mx = val;
                    }
                    mloc[r] = mx;
                }

                /* gap between running max and local max; the tile-wide minimum */
                double mingap = INFINITY;
                for (int r = 0; r < nrows; ++r) {
                    double gap;
                    if (mloc[r] == -INFINITY)
                        gap = INFINITY;             /* nothing visible in this block */
                    else if (m[r] == -INFINITY)
                        gap = -INFINITY;            /* no running max yet */
                    else
                        gap = m[r] - mloc[r];
                    if (gap < mingap) mingap = gap;
                }
                if (mingap_out) mingap_out[(size_t)w * j_max + j] = mingap;

                int skip = (mingap > lam);          /* strictly greater */
                if (forced) {
                    const uint8_t f = forced[(size_t)w * j_max + j];
                    if (f == 0) skip = 0;
                    else if (f == 1) skip = 1;
                }
                skip_w[j] = (uint8_t)skip;
                kept[j] = (uint8_t)!skip;
                if (skip) continue;                 /* no exp, no V, no PV */

                for (int c = 0; c < nc; ++c)
                    for (int d = 0; d < D; ++d)
                        vblk[(size_t)c * D + d] =
                            elem(v, ((size_t)(kbase + c0 + c) * n_heads_kv + g) * D + d, in_dtype) * sv;

                for (int r = 0; r < nrows; ++r) {
                    const double mnew = (mloc[r] > m[r]) ? mloc[r] : m[r];
                    if (mnew == -INFINITY) continue;        /* row still empty */
                    const double alpha = exp(m[r] - mnew);  /* exp(-inf) = 0 */
                    double rowsum = 0.0;
                    double *a = acc + (size_t)r * D;
                    for (int d = 0; d < D; ++d) a[d] *= alpha;
                    for (int c = 0; c < nc; ++c) {
                        const double sv_ = sc[(size_t)r * block_k + c];
                        if (sv_ == -INFINITY) continue;
                        const double p = exp(sv_ - mnew);
                        rowsum += p;
                        for (int d = 0; d < D; ++d) a[d] += p * vblk[(size_t)c * D + d];
                    }
                    l[r] = alpha * l[r] + rowsum;
                    m[r] = mnew;
                }
            }

            for (int r = 0; r < nrows; ++r) {
                for (int d = 0; d < D; ++d) o_w[(size_t)r * D + d] = acc[(size_t)r * D + d] / l[r];
                lse_w[r] = m[r] + log(l[r]);
            }

            if (p_out) {
                /* normalised probabilities of the kept keys, from the final m and l */
                double *p_w = p_out + (size_t)w * block_q * p_cols;
                for (int j = 0; j < nblk; ++j) {
                    if (!kept[j]) continue;
                    const int c0 = j * block_k;
                    const int c1 = (c0 + block_k < Lk) ? c0 + block_k : Lk;
                    for (int r = 0; r < nrows; ++r) {
                        const int qi = off + r0 + r;
                        for (int c = c0; c < c1 && c < p_cols; ++c) {
                            if (c > qi) continue;
                            double dot = 0.0;
                            for (int d = 0; d < D; ++d)
                                dot += qrow[(size_t)r * D + d] *
                                       elem(k, ((size_t)(kbase + c) * n_heads_kv + g) * D + d, in_dtype) * sk;
                            p_w[(size_t)r * p_cols + c] = exp(scale * dot - m[r]) / l[r];
                        }
                    }
                }
            }
        }
        free(qrow); free(kblk); free(vblk); free(sc); free(m); free(l); free(mloc); free(acc); free(kept);
    }
    return bad ? -5 : 0;
}
