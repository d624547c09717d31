/*
 * attn_oracle.c -- plain, slow fp64 CPU oracle for non-causal joint attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code,
 * header, table or constant with the HIP path and must never be used to
 * produce a product result.
 *
 * What it computes (the plain definition, no blocking, no fusion):
 *   joint attention runs one softmax attention over the concatenation of the
 *   separately embedded text and image-latent token streams
 *   (bpdata.com "FLUX 3 Image Klein optimalizálása", section "Modellezés és
 *   pipeline jellemzők"); "VANILLA BF16 attention" is the baseline backend
 *   whose cost the pages measure (scopeai.cc page, section
 *   "各项优化的效果与质量代价").  For one query row i of one (batch, head):
 *
 *       s_j  = scale * sum_d q_id k_jd         for every key j that is kept
 *       m    = max_j s_j
 *       p_j  = exp(s_j - m)
 *       l    = sum_j p_j
 *       o_id = (sum_j p_j v_jd) / l
 *       lse  = m + ln l
 *
 *   A key is dropped when its 128x128 (query block, key block) mask entry is
 *   zero, which is the same as giving it a -inf logit (block-sparse
 *   attention, bpdata.com page, section "Mi szerepel az optimalizálásban").
 *   A row with no kept key gets o = 0 and lse = -inf.
 *
 * Everything is double precision on the given inputs, libm exp/log, no BLAS,
 * no fast-math.  OpenMP over rows only.
 *
 * The fp8 part (OCP E4M3, dynamic per-block scales, P quantised with the
 * fixed scale 448) follows the quantised-attention recipe; FP8 dynamic
 * quantisation of activations is what the wavespeed.ai FLUX.1-dev page calls
 * "FP8 Dynamische Quantisierung".  See the comments at each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* Dense / block-masked attention, fp64 two-pass definition.                  */
/* ------------------------------------------------------------------------- */

/* q, k, v: [BH][N][D] doubles, contiguous.  mask: NULL (dense) or uint8
 * [nmask][nb][nb] with nb = ceil(N / block); (b,h) slice bh uses
 * mask + bh * mask_stride_bh.  rows: flat row ids (bh * N + i), or NULL for
 * all BH*N rows in order.  o: [nrows][D], lse: [nrows] (lse may be NULL).
 * Returns 0, or -1 on a bad argument. */
int oracle_attn_f64(int64_t BH, int64_t N, int64_t D,
                    const double* q, const double* k, const double* v,
                    const uint8_t* mask, int64_t mask_stride_bh, int64_t block,
                    double scale, const int64_t* rows, int64_t nrows,
                    double* o, double* lse)
{
    if (BH <= 0 || N <= 0 || D <= 0 || !q || !k || !v || !o) return -1;
    if (mask && block <= 0) return -1;
    if (!rows) nrows = BH * N;
    const int64_t nb = mask ? (N + block - 1) / block : 1;
    int bad = 0;

#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
        unsigned char* keep = (unsigned char*)malloc((size_t)N);
        if (!s || !keep) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < nrows; ++r) {
                const int64_t row = rows ? rows[r] : r;
                if (row < 0 || row >= BH * N) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                const int64_t bh = row / N, i = row % N;
                const double* qi = q + (bh * N + i) * D;
                const double* kb = k + bh * N * D;
                const double* vb = v + bh * N * D;
                double* oi = o + r * D;
                const uint8_t* mrow = mask ? mask + bh * mask_stride_bh + (i / block) * nb : NULL;

                /* pass 1: logits of kept keys and their maximum */
                double m = -INFINITY;
                int64_t nkeep = 0;
                for (int64_t j = 0; j < N; ++j) {
                    keep[j] = (unsigned char)(mrow ? (mrow[j / block] != 0) : 1);
                    if (!keep[j]) continue;
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += qi[d] * kb[j * D + d];
                    s[j] = scale * dot;
                    if (s[j] > m) m = s[j];
                    ++nkeep;
                }
                if (nkeep == 0) {
                    for (int64_t d = 0; d < D; ++d) oi[d] = 0.0;
                    if (lse) lse[r] = -INFINITY;
                    continue;
                }
                /* pass 2: weights, their sum, and the weighted sum of values */
                double l = 0.0;
                for (int64_t d = 0; d < D; ++d) oi[d] = 0.0;
                for (int64_t j = 0; j < N; ++j) {
                    if (!keep[j]) continue;
                    const double p = exp(s[j] - m);
                    l += p;
                    for (int64_t d = 0; d < D; ++d) oi[d] += p * vb[j * D + d];
                }
                for (int64_t d = 0; d < D; ++d) oi[d] /= l;
                if (lse) lse[r] = m + log(l);
            }
        }
        free(s);
        free(keep);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------- */
/* OCP 8-bit floating point E4M3 ("E4M3FN").                                  */
/* Written from the OCP 8-bit floating point specification (v1.0):           */
/*   sign | 4 exponent bits, bias 7 | 3 mantissa bits.                        */
/*   exponent field 0: subnormal, value 2^-6 * m/8;                          */
/*   exponent field 1..15: normal, value 2^(e-7) * (1 + m/8);                */
/*   field 15 with mantissa 7 (0x7F / 0xFF) is NaN; there is no infinity,     */
/*   so the largest finite magnitude is 2^8 * 1.75 = 448.                    */
/* ------------------------------------------------------------------------- */

double oracle_e4m3_decode(uint8_t c)
{
    const int sign = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Round-to-nearest-even encode of a finite value already inside [-448, 448].
 * Values outside that range are clamped first (saturating conversion).
 * NaN encodes to 0x7F. */
uint8_t oracle_e4m3_encode(double x)
{
    if (isnan(x)) return 0x7F;
    const uint8_t sign = (x < 0.0 || (x == 0.0 && signbit(x))) ? 0x80 : 0x00;
    double a = fabs(x);
    if (a > 448.0) a = 448.0;
    if (a < ldexp(1.0, -6)) {
        /* subnormal grid: multiples of 2^-9; rint rounds ties to even */
        double m = rint(ldexp(a, 9));          /* exact scaling by a power of two */
        return (uint8_t)(sign | (uint8_t)m);  /* m == 8 is exactly the smallest normal, code 0x08 */
    }
    int e2;
    double fr = frexp(a, &e2);                 /* a = fr * 2^e2, fr in [0.5, 1) */
    int e = e2 - 1;                            /* a = (2 fr) * 2^e, 2 fr in [1, 2) */
    double mant = rint((2.0 * fr - 1.0) * 8.0);/* 3-bit mantissa, ties to even */
    if (mant == 8.0) { mant = 0.0; e += 1; }
    int field = e + 7;
    if (field > 15 || (field == 15 && mant > 6.0)) { field = 15; mant = 6.0; } /* cannot happen after clamp */
    return (uint8_t)(sign | (uint8_t)(field << 3) | (uint8_t)mant);
}

/* Per-(b,h, block-of-tokens) dynamic quantisation of one tensor.
 *   absmax = max |x| over the block's valid tokens and all d   (fp32)
 *   inv    = 448 / absmax                                      (fp32 divide)
 *   code   = e4m3(clamp(x * inv, -448, 448))                   (fp32 multiply)
 *   scale  = absmax / 448                                      (fp32 divide)
 * absmax == 0, or an absmax so small that the fp32 quotient 448 / absmax
 * overflows to infinity, gives scale 1 and all-zero codes (+0): there is no
 * finite fp32 scale that maps such a block onto the e4m3 range, and its
 * values (below 1.3e-36) are zero to every tolerance used.  The quantised code is an
 * integer decided by floating point, so it is decided in fp32, the precision
 * the device quantiser uses.
 * x: [BH][N][D] fp32 (bf16 values), codes: [BH][N][D], scales: [BH][nb]. */
void oracle_fp8_quantize(int64_t BH, int64_t N, int64_t D, int64_t block,
                         const float* x, uint8_t* codes, float* scales)
{
    const int64_t nb = (N + block - 1) / block;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < BH * nb; ++t) {
        const int64_t bh = t / nb, kb = t % nb;
        const int64_t j0 = kb * block, j1 = (j0 + block < N) ? j0 + block : N;
        const float* xb = x + bh * N * D;
        uint8_t* cb = codes + bh * N * D;
        float amax = 0.0f;
        for (int64_t j = j0; j < j1; ++j)
            for (int64_t d = 0; d < D; ++d) {
                const float a = fabsf(xb[j * D + d]);
                if (a > amax) amax = a;
            }
        const float inv = 448.0f / amax;
        if (amax == 0.0f || isinf(inv)) {
            /* nothing to scale: an all-zero block, or one so small that
             * 448 / absmax overflows fp32 (absmax < 448 / FLT_MAX) */
            scales[t] = 1.0f;
            for (int64_t j = j0; j < j1; ++j) memset(cb + j * D, 0, (size_t)D);
            continue;
        }
        scales[t] = amax / 448.0f;
        for (int64_t j = j0; j < j1; ++j)
            for (int64_t d = 0; d < D; ++d) {
                float y = xb[j * D + d] * inv;
                if (y > 448.0f) y = 448.0f;
                if (y < -448.0f) y = -448.0f;
                cb[j * D + d] = oracle_e4m3_encode((double)y);
            }
    }
}

/* The fp8 attention recipe, step by step, for sampled rows.
 * Inputs are e4m3 codes of Q, K, V ([BH][N][D]) and their per-(bh, block)
 * scales ([BH][nb]).  Keys are visited in blocks of `block` tokens, the same
 * blocks the scales use, in increasing order.  For query row i in block qb:
 *
 *   t_j   = scale * sq[qb] * sk[kb] * sum_d dec(q8_id) dec(k8_jd)
 *   m_kb  = max(m_{kb-1}, max_{j in kb} t_j)                 (running max)
 *   w_j   = exp(t_j - m_kb)                                  (in [0, 1])
 *   P8_j  = e4m3(448 * w_j)          if quantize_p, else 448 * w_j
 *   l     = exp(m_{kb-1} - m_kb) * l + sum_j P8_j / 448      (the same weights
 *                                                             that multiply V)
 *   acc_d = exp(m_{kb-1} - m_kb) * acc_d + sum_j (P8_j / 448) * sv[kb] * dec(v8_jd)
 *   o_d   = acc_d / l,   lse = m_last + ln l
 *
 * 448 * w_j is formed in fp32 (the precision the device uses for that
 * rounding decision) before encoding; everything else is fp64.
 *
 * recipe_range runs these steps for one row over key blocks [kb0, kb1),
 * starting from m = -inf, l = 0, acc = 0, and leaves acc, m and l. */
typedef struct {
    int64_t N, D, block, nb;
    const uint8_t *k8, *v8;
    const float *sq, *sk, *sv;
    double scale;
    int quantize_p;
    const double* dec;
} recipe_in;

static void recipe_range(const recipe_in* in, int64_t bh, int64_t qb, const double* qd, int64_t kb0,
                         int64_t kb1, double* t, double* acc, double* m_out, double* l_out)
{
    const int64_t N = in->N, D = in->D, block = in->block, nb = in->nb;
    const double* dec = in->dec;
    double m = -INFINITY, l = 0.0;
    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
    for (int64_t kb = kb0; kb < kb1; ++kb) {
        const int64_t j0 = kb * block, j1 = (j0 + block < N) ? j0 + block : N;
        const double f = in->scale * (double)in->sq[bh * nb + qb] * (double)in->sk[bh * nb + kb];
        double mt = -INFINITY;
        for (int64_t j = j0; j < j1; ++j) {
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += qd[d] * dec[in->k8[(bh * N + j) * D + d]];
            t[j - j0] = f * dot;
            if (t[j - j0] > mt) mt = t[j - j0];
        }
        const double mnew = (mt > m) ? mt : m;
        const double alpha = (m == -INFINITY) ? 0.0 : exp(m - mnew);
        l *= alpha;
        for (int64_t d = 0; d < D; ++d) acc[d] *= alpha;
        const double svk = (double)in->sv[bh * nb + kb];
        for (int64_t j = j0; j < j1; ++j) {
            const double w = exp(t[j - j0] - mnew);
            const float y = (float)w * 448.0f;
            const double p = in->quantize_p ? dec[oracle_e4m3_encode((double)y)] : 448.0 * w;
            l += p / 448.0;
            const double c = p / 448.0 * svk;
            for (int64_t d = 0; d < D; ++d) acc[d] += c * dec[in->v8[(bh * N + j) * D + d]];
        }
        m = mnew;
    }
    *m_out = m;
    *l_out = l;
}

/* The recipe with each row's key blocks cut into nsplit consecutive ranges
 * (range p = blocks p*nb/nsplit .. (p+1)*nb/nsplit - 1, integer division),
 * each run by recipe_range from its own fresh running max, and the ranges
 * merged exactly:
 *   M = max_p m_p,   o = sum_p exp(m_p - M) acc_p / sum_p exp(m_p - M) l_p,
 *   lse = M + ln sum_p exp(m_p - M) l_p.
 * nsplit = 1 is the recipe above (M = m, every factor exp(0) = 1).  This is
 * what a query block computes when its key range is split over several
 * workers: each range rounds its P against its own running max.
 * 1 <= nsplit <= nb, else -1. */
int oracle_attn_fp8_recipe_split(int64_t BH, int64_t N, int64_t D, int64_t block,
                                 const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                                 const float* sq, const float* sk, const float* sv,
                                 double scale, int quantize_p, int64_t nsplit,
                                 const int64_t* rows, int64_t nrows,
                                 double* o, double* lse)
{
    if (BH <= 0 || N <= 0 || D <= 0 || block <= 0) return -1;
    const int64_t nb = (N + block - 1) / block;
    if (nsplit < 1 || nsplit > nb) return -1;
    if (!rows) nrows = BH * N;
    double dec[256];
    for (int c = 0; c < 256; ++c) dec[c] = oracle_e4m3_decode((uint8_t)c);
    const recipe_in in = {N, D, block, nb, k8, v8, sq, sk, sv, scale, quantize_p, dec};
    int bad = 0;

#pragma omp parallel
    {
        double* acc = (double*)malloc(sizeof(double) * (size_t)(D * nsplit));
        double* mp = (double*)malloc(sizeof(double) * (size_t)nsplit);
        double* lp = (double*)malloc(sizeof(double) * (size_t)nsplit);
        double* t = (double*)malloc(sizeof(double) * (size_t)block);
        double* qd = (double*)malloc(sizeof(double) * (size_t)D);
        if (!acc || !mp || !lp || !t || !qd) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < nrows; ++r) {
                const int64_t row = rows ? rows[r] : r;
                if (row < 0 || row >= BH * N) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                const int64_t bh = row / N, i = row % N, qb = i / block;
                for (int64_t d = 0; d < D; ++d) qd[d] = dec[q8[(bh * N + i) * D + d]];
                double M = -INFINITY;
                for (int64_t p = 0; p < nsplit; ++p) {
                    recipe_range(&in, bh, qb, qd, p * nb / nsplit, (p + 1) * nb / nsplit, t, acc + p * D,
                                 &mp[p], &lp[p]);
                    if (mp[p] > M) M = mp[p];
                }
                double l = 0.0;
                for (int64_t d = 0; d < D; ++d) o[r * D + d] = 0.0;
                for (int64_t p = 0; p < nsplit; ++p) {
                    const double wgt = exp(mp[p] - M);
                    l += wgt * lp[p];
                    for (int64_t d = 0; d < D; ++d) o[r * D + d] += wgt * acc[p * D + d];
                }
                for (int64_t d = 0; d < D; ++d) o[r * D + d] /= l;
                if (lse) lse[r] = M + log(l);
            }
        }
        free(acc);
        free(mp);
        free(lp);
        free(t);
        free(qd);
    }
    return bad ? -1 : 0;
}

int oracle_attn_fp8_recipe(int64_t BH, int64_t N, int64_t D, int64_t block,
                           const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                           const float* sq, const float* sk, const float* sv,
                           double scale, int quantize_p,
                           const int64_t* rows, int64_t nrows,
                           double* o, double* lse)
{
    return oracle_attn_fp8_recipe_split(BH, N, D, block, q8, k8, v8, sq, sk, sv, scale, quantize_p, 1, rows,
                                        nrows, o, lse);
}

/* Block-mask selection in the manner of Sol-Attention (block-sparse attention
 * whose sparsity a parameter tau controls: bpdata.com page, section
 * "Részletes optimalizációs lépések és hatásuk"; the rule itself is a reading,
 * stated here in full because the pages do not give one).  For one (b, h):
 *
 *   qm_i = mean of q over the valid tokens of query block i   (fp64)
 *   km_j = mean of k over the valid tokens of key block j
 *   s_ij = scale * <qm_i, km_j>
 *   p_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij)
 *   keep_ij = p_ij >= tau / nb   or   i == j   or   i < tb   or   j < tb
 *
 * with nb = ceil(N / block) and tb = ceil(text_tokens / block): a key block
 * is kept when its estimated share of the row's attention is at least tau
 * times the uniform share; the diagonal and the text blocks' rows and
 * columns are always kept.  q, k: [BH][N][D] doubles.  mask: uint8
 * [BH][nb][nb]; share (nullable): [BH][nb][nb] doubles, the p_ij. */
void oracle_select_blocks(int64_t BH, int64_t N, int64_t D, int64_t block,
                          const double* q, const double* k, double scale, double tau,
                          int64_t text_tokens, uint8_t* mask, double* share)
{
    const int64_t nb = (N + block - 1) / block, tb = (text_tokens + block - 1) / block;
#pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < BH; ++bh) {
        double* qm = (double*)calloc((size_t)(nb * D), sizeof(double));
        double* km = (double*)calloc((size_t)(nb * D), sizeof(double));
        double* s = (double*)malloc(sizeof(double) * (size_t)nb);
        if (!qm || !km || !s) { free(qm); free(km); free(s); continue; }
        for (int64_t b = 0; b < nb; ++b) {
            const int64_t j0 = b * block, j1 = (j0 + block < N) ? j0 + block : N;
            for (int64_t j = j0; j < j1; ++j)
                for (int64_t d = 0; d < D; ++d) {
                    qm[b * D + d] += q[(bh * N + j) * D + d];
                    km[b * D + d] += k[(bh * N + j) * D + d];
                }
            for (int64_t d = 0; d < D; ++d) {
                qm[b * D + d] /= (double)(j1 - j0);
                km[b * D + d] /= (double)(j1 - j0);
            }
        }
        for (int64_t i = 0; i < nb; ++i) {
            double m = -INFINITY;
            for (int64_t j = 0; j < nb; ++j) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += qm[i * D + d] * km[j * D + d];
                s[j] = scale * dot;
                if (s[j] > m) m = s[j];
            }
            double z = 0.0;
            for (int64_t j = 0; j < nb; ++j) z += exp(s[j] - m);
            for (int64_t j = 0; j < nb; ++j) {
                const double p = exp(s[j] - m) / z;
                const int forced = (i == j) || (i < tb) || (j < tb);
                mask[(bh * nb + i) * nb + j] = (uint8_t)((p >= tau / (double)nb) || forced);
                if (share) share[(bh * nb + i) * nb + j] = p;
            }
        }
        free(qm);
        free(km);
        free(s);
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
