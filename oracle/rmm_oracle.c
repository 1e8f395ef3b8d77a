/*
 * rmm_oracle.c -- reference ("oracle") implementation of Reduced Matrix
 * Multiplication (RMM).
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
 * CPU-baseline leg of the benchmark are the only users of this library.  The
 * GPU library (input_adaptive_reduced_02_amd/) never includes, links or calls
 * it, and the two share no code, header, table or helper.
 *
 * Plain, slow, single-threaded C.  All arithmetic is IEEE binary64, built with
 * -O2 -ffp-contract=off so that every a*b + c rounds twice, exactly as
 * written.  Callers pass the exact values the GPU consumes (bf16 or fp32 bit
 * patterns widened to double).
 *
 * Source: "Reduced Matrix Multiplication: Input-Adaptive Matrix-Product
 * Reduction for LLM Inference" (Lan, Li, Zhou), technical summary on
 * gist.science, section "Metodologia":
 *   - every Transformer matmul is read as Y = A B, A being the activation and
 *     B a weight or an intermediate ("Metodologia", first paragraph);
 *   - for the current input an index set I along the shared contraction
 *     dimension is picked and only A[:, I] B[I, :] is formed ("Mecanismo
 *     Central");
 *   - each contraction index j is scored by the L2 norm of activation column
 *     j, and the ceil(rho * d) best-scored indices are kept, rho being the
 *     retention ratio the user sets ("Estrategia de Selecao");
 *   - the reduction is applied to the hidden dimension of XW projections, the
 *     feature dimension of QK^T and the token dimension of PV ("Escopo de
 *     Aplicacao").
 *
 * Readings taken where the pages are silent:
 *   R1 score of slice k in group g = ||A[rows_g, k]||_2 * ||B[k, :]||_2.
 *      Passing b == NULL gives the pages' activation-only score.
 *   R2 selection is made per group of consecutive rows; a whole matrix is a
 *      single group.  The last group may be short.
 *   R3 k = ceil(r * K), with a snap for decimal r: x = r*K; if x lies within
 *      1e-9*K of an integer n then k = n, else k = ceil(x); clamp to [1, K].
 *   R4 equal scores go to the lower index; the keep/drop decision compares the
 *      scores after one rounding to IEEE binary32, the key precision of the
 *      GPU select.
 *   R5 P.V: for query block g the candidate keys are its causal prefix
 *      k < K_g = min(L, qblock*(g+1)); the score of key k is
 *      (sum over the block's queries of P[q,k]) * ||V[k,:]||_2; k_g = kk(r, K_g).
 *   R6 every sum runs in ascending index order.
 *   R10 QK^T ("Escopo de Aplicacao": the feature dimension of QK^T).  Here A
 *      is a block of queries Q_g and B is K^T restricted to the keys the block
 *      is multiplied with (its causal prefix k < K_g, as in R5; all L keys
 *      without the mask), so the contraction runs over the head dimension D.
 *      Feature j of block g scores ||Q[rows_g, j]||_2 * ||K[0 .. K_g-1, j]||_2
 *      (the second factor dropped: the pages' activation-only rule) and
 *      kk(r, D) features are kept per (head, block) with the R4 order.
 *   R11 the logit of query q and candidate key k is the reduced dot product
 *      over the kept features divided by sqrt(D), D the full head dimension
 *      (the reduced product stands in for the full one, so the softmax keeps
 *      the model's temperature).  P[q, .] is the softmax of row q over its
 *      candidates (k <= q causal, else every k < L) and 0 elsewhere.  The
 *      P.V scores of R5 are taken on P as stored for the product (bf16).
 *   R9 int8 weights ("Resultados Experimentais", item "Compatibilidade":
 *      the method works on INT8-quantised weights; the pages fix no scheme).
 *      Symmetric absmax quantisation with one binary32 scale per output
 *      column n: s_n = max_k |B[k,n]| / 127, q[k,n] = round-half-even(B[k,n]
 *      / s_n) clamped to [-127, 127] (s_n = 0 and q = 0 for an all-zero
 *      column), both divisions in binary32 because they decide integers.  The
 *      method then runs on the dequantised weight s_n * q[k,n] (exact in
 *      binary64): its row norms score the slices and its kept rows are
 *      multiplied.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- retained count ("Estrategia de Selecao": k = ceil(rho d)), reading R3 */
int64_t oracle_kk(double r, int64_t K)
{
    if (!(r > 0.0) || !(r <= 1.0) || K < 1)
        return -1;
    double x = r * (double)K;
    double n = nearbyint(x);
    int64_t kk;
    if (fabs(x - n) <= 1e-9 * (double)K)
        kk = (int64_t)n;
    else
        kk = (int64_t)ceil(x);
    if (kk < 1)
        kk = 1;
    if (kk > K)
        kk = K;
    return kk;
}

/* ---- L2 norm of every row of B (K x N, row stride ldb), reading R1 */
void oracle_rownorms(const double *B, int64_t K, int64_t N, int64_t ldb, double *b)
{
    for (int64_t k = 0; k < K; ++k) {
        double s = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double v = B[k * ldb + n];
            s += v * v;
        }
        b[k] = sqrt(s);
    }
}

/* ---- L2 norm of every column of a rows x K block of A ("Estrategia de
 * Selecao": the activation column norm) */
void oracle_colnorms(const double *A, int64_t rows, int64_t K, int64_t lda, double *a)
{
    for (int64_t k = 0; k < K; ++k) {
        double s = 0.0;
        for (int64_t m = 0; m < rows; ++m) {
            double v = A[m * lda + k];
            s += v * v;
        }
        a[k] = sqrt(s);
    }
}

/* ---- scores of every slice k for every group g (readings R1, R2).
 * s64[g*K + k] = a_{g,k} * b_k   (b == NULL: b_k = 1)
 * s32[g*K + k] = s64 rounded once to binary32. */
void oracle_scores(const double *A, int64_t M, int64_t K, int64_t lda, const double *b,
                   int64_t group_rows, double *s64, float *s32)
{
    int64_t G = (M + group_rows - 1) / group_rows;
    double *a = (double *)malloc((size_t)K * sizeof(double));
    for (int64_t g = 0; g < G; ++g) {
        int64_t r0 = g * group_rows;
        int64_t rows = M - r0 < group_rows ? M - r0 : group_rows;
        oracle_colnorms(A + r0 * lda, rows, K, lda, a);
        for (int64_t k = 0; k < K; ++k) {
            double s = a[k] * (b ? b[k] : 1.0);
            s64[g * K + k] = s;
            s32[g * K + k] = (float)s;
        }
    }
    free(a);
}

/* ---- top-k by a full sort (reading R4).  Order: score descending, then
 * index ascending.  The first kk of that order are kept and returned in
 * ascending index order. */
static const float *sort_keys;

static int by_rank(const void *x, const void *y)
{
    int32_t i = *(const int32_t *)x, j = *(const int32_t *)y;
    float si = sort_keys[i], sj = sort_keys[j];
    if (si > sj)
        return -1;
    if (si < sj)
        return 1;
    return (i > j) - (i < j);
}

static int by_index(const void *x, const void *y)
{
    int32_t i = *(const int32_t *)x, j = *(const int32_t *)y;
    return (i > j) - (i < j);
}

int oracle_topk(const float *s, int64_t K, int64_t kk, int32_t *idx)
{
    if (kk < 1 || kk > K)
        return -1;
    int32_t *order = (int32_t *)malloc((size_t)K * sizeof(int32_t));
    for (int64_t k = 0; k < K; ++k)
        order[k] = (int32_t)k;
    sort_keys = s;
    qsort(order, (size_t)K, sizeof(int32_t), by_rank);
    memcpy(idx, order, (size_t)kk * sizeof(int32_t));
    qsort(idx, (size_t)kk, sizeof(int32_t), by_index);
    free(order);
    return 0;
}

/* ---- the reduced product ("Mecanismo Central": A[:, I] B[I, :]) for rows
 * [m0, m1).  Row m belongs to group m / group_rows, whose kept indices are
 * idx[g*ldidx + 0 .. kk-1].  Outer-product form, ascending j (reading R6).
 * Y row m is written at Y[(m - m0)*ldy]. */
void oracle_reduced(const double *A, int64_t lda, const double *B, int64_t ldb, int64_t N,
                    int64_t group_rows, const int32_t *idx, int64_t ldidx, int64_t kk,
                    int64_t m0, int64_t m1, double *Y, int64_t ldy)
{
    for (int64_t m = m0; m < m1; ++m) {
        const int32_t *I = idx + (m / group_rows) * ldidx;
        double *y = Y + (m - m0) * ldy;
        for (int64_t n = 0; n < N; ++n)
            y[n] = 0.0;
        for (int64_t j = 0; j < kk; ++j) {
            int64_t k = I[j];
            double a = A[m * lda + k];
            const double *brow = B + k * ldb;
            for (int64_t n = 0; n < N; ++n)
                y[n] += a * brow[n];
        }
    }
}

/* ---- single entries of the reduced product: out[i] = Y[ms[i], ns[i]], the
 * same sum in the same order as oracle_reduced. */
void oracle_reduced_entries(const double *A, int64_t lda, const double *B, int64_t ldb,
                            int64_t group_rows, const int32_t *idx, int64_t ldidx, int64_t kk,
                            const int64_t *ms, const int64_t *ns, int64_t count, double *out)
{
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        const int32_t *I = idx + (m / group_rows) * ldidx;
        double y = 0.0;
        for (int64_t j = 0; j < kk; ++j) {
            int64_t k = I[j];
            y += A[m * lda + k] * B[k * ldb + n];
        }
        out[i] = y;
    }
}

/* ---- error bound of one group: beta = sum over the dropped slices of
 * ||A[rows_g, k]|| * ||B[k, :]||, i.e. the sum of the dropped unrounded
 * scores.  By the triangle inequality and ||a b^T||_F = ||a|| ||b|| it bounds
 * ||A_g B - A_g[:, I] B[I, :]||_F. */
double oracle_bound(const double *s64, int64_t K, const int32_t *idx, int64_t kk)
{
    unsigned char *kept = (unsigned char *)calloc((size_t)K, 1);
    for (int64_t j = 0; j < kk; ++j)
        kept[idx[j]] = 1;
    double beta = 0.0;
    for (int64_t k = 0; k < K; ++k)
        if (!kept[k])
            beta += s64[k];
    free(kept);
    return beta;
}

/* ---- threshold of one group (reading R4): the score of rank kk in the order
 * (score descending, index ascending), which is the smallest binary32 key
 * among the kept indices idx[0 .. kk-1]. */
float oracle_thresh(const float *s32, const int32_t *idx, int64_t kk)
{
    float t = s32[idx[0]];
    for (int64_t j = 1; j < kk; ++j)
        if (s32[idx[j]] < t)
            t = s32[idx[j]];
    return t;
}

/* ---- near-tie band of one group.  The element of rank kk is the kept index
 * with the smallest binary32 key, and among kept indices sharing that key the
 * highest one (lower indices rank first).  t is its unrounded score; the band
 * is every k in [0, K) with |s64[k] - t| <= rel * |t|, written ascending to
 * out.  Returns the band's size.  Within the band a kept set may legitimately
 * differ when the two sides' keys are not bit-identical. */
int64_t oracle_near_ties(const double *s64, const float *s32, int64_t K, const int32_t *idx,
                         int64_t kk, double rel, int32_t *out)
{
    int32_t last = idx[0];
    for (int64_t j = 1; j < kk; ++j) {
        int32_t i = idx[j];
        if (s32[i] < s32[last] || (s32[i] == s32[last] && i > last))
            last = i;
    }
    double t = s64[last];
    int64_t n = 0;
    for (int64_t k = 0; k < K; ++k)
        if (fabs(s64[k] - t) <= rel * fabs(t))
            out[n++] = (int32_t)k;
    return n;
}

/* ---- P.V ("Escopo de Aplicacao": the token dimension of PV), reading R5.
 * P is stored key-major: Pt[k*L + q] = P[q, k].  The functions below see one
 * head and one query block: Ptb[k*ldp + i] = P[q0 + i, k] for i < nq. */
int64_t oracle_pv_prefix(int64_t L, int64_t qblock, int64_t g, int causal)
{
    if (!causal)
        return L;
    int64_t e = qblock * (g + 1);
    return e < L ? e : L;
}

void oracle_pv_scores(const double *Ptb, int64_t ldp, int64_t nq, const double *V, int64_t D,
                      int64_t Kg, double *s64, float *s32)
{
    for (int64_t k = 0; k < Kg; ++k) {
        double mass = 0.0;
        for (int64_t i = 0; i < nq; ++i)
            mass += Ptb[k * ldp + i];
        double vv = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            double v = V[k * D + d];
            vv += v * v;
        }
        double s = mass * sqrt(vv);
        s64[k] = s;
        s32[k] = (float)s;
    }
}

/* O[i*D + d] = sum_j P[q0+i, I_j] V[I_j, d] over the kept keys, ascending j. */
void oracle_pv_block(const double *Ptb, int64_t ldp, int64_t nq, const double *V, int64_t D,
                     const int32_t *idx, int64_t kk, double *O)
{
    for (int64_t i = 0; i < nq; ++i) {
        double *o = O + i * D;
        for (int64_t d = 0; d < D; ++d)
            o[d] = 0.0;
        for (int64_t j = 0; j < kk; ++j) {
            int64_t k = idx[j];
            double p = Ptb[k * ldp + i];
            const double *v = V + k * D;
            for (int64_t d = 0; d < D; ++d)
                o[d] += p * v[d];
        }
    }
}

/* Bound for one block: sum over dropped keys k < Kg of
 * ||P[block, k]||_2 * ||V[k, :]||_2 (L2 column norm of P, not its mass). */
double oracle_pv_bound(const double *Ptb, int64_t ldp, int64_t nq, const double *V, int64_t D,
                       int64_t Kg, const int32_t *idx, int64_t kk)
{
    unsigned char *kept = (unsigned char *)calloc((size_t)Kg, 1);
    for (int64_t j = 0; j < kk; ++j)
        kept[idx[j]] = 1;
    double beta = 0.0;
    for (int64_t k = 0; k < Kg; ++k) {
        if (kept[k])
            continue;
        double pp = 0.0;
        for (int64_t i = 0; i < nq; ++i) {
            double p = Ptb[k * ldp + i];
            pp += p * p;
        }
        double vv = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            double v = V[k * D + d];
            vv += v * v;
        }
        beta += sqrt(pp) * sqrt(vv);
    }
    free(kept);
    return beta;
}

/* ---- QK^T feature scores of one query block, reading R10.  One head: Q and
 * K are L x D row-major.  The block holds queries q0 .. q0+nq-1, its candidate
 * keys are k < Kg.  s64[j] = ||Q[q0.., j]||_2 * ||K[0..Kg-1, j]||_2 (use_k == 0:
 * ||Q[q0.., j]||_2 alone); s32 = s64 rounded once to binary32. */
void oracle_qk_scores(const double *Q, const double *K, int64_t D, int64_t q0, int64_t nq, int64_t Kg,
                      int use_k, double *s64, float *s32)
{
    for (int64_t j = 0; j < D; ++j) {
        double qq = 0.0;
        for (int64_t i = 0; i < nq; ++i) {
            double v = Q[(q0 + i) * D + j];
            qq += v * v;
        }
        double kn = 1.0;
        if (use_k) {
            double kq = 0.0;
            for (int64_t k = 0; k < Kg; ++k) {
                double v = K[k * D + j];
                kq += v * v;
            }
            kn = sqrt(kq);
        }
        double s = sqrt(qq) * kn;
        s64[j] = s;
        s32[j] = (float)s;
    }
}

/* ---- attention probabilities of queries q0 .. q0+nq-1 of one head, reading
 * R11.  Kept features idx[0 .. kk-1] (idx == NULL: every feature, kk = D).
 * Writes P[i*L + k] for the row of query q0+i: the softmax over the row's
 * candidate keys of S[k] = (sum over kept j, ascending, of Q[q, j] K[k, j]) /
 * sqrt(D), computed as exp(S[k] - max S) / sum of those terms; 0 for the keys
 * the row does not see. */
void oracle_attn_probs(const double *Q, const double *K, int64_t L, int64_t D, int64_t q0, int64_t nq,
                       int causal, const int32_t *idx, int64_t kk, double *P)
{
    double *S = (double *)malloc((size_t)L * sizeof(double));
    const int64_t nf = idx ? kk : D;
    for (int64_t i = 0; i < nq; ++i) {
        const int64_t q = q0 + i;
        const int64_t n = causal ? q + 1 : L;
        double *p = P + i * L;
        double mx = -INFINITY;
        for (int64_t k = 0; k < n; ++k) {
            double dot = 0.0;
            for (int64_t j = 0; j < nf; ++j) {
                int64_t f = idx ? idx[j] : j;
                dot += Q[q * D + f] * K[k * D + f];
            }
            S[k] = dot / sqrt((double)D);
            if (S[k] > mx)
                mx = S[k];
        }
        double sum = 0.0;
        for (int64_t k = 0; k < n; ++k) {
            p[k] = exp(S[k] - mx);
            sum += p[k];
        }
        for (int64_t k = 0; k < n; ++k)
            p[k] /= sum;
        for (int64_t k = n; k < L; ++k)
            p[k] = 0.0;
    }
    free(S);
}

/* ---- int8 weight quantisation, reading R9.  B is K x N binary32 (row stride
 * ldb); writes q (row stride ldq) and one scale per column. */
void oracle_quantize_q8(const float *B, int64_t K, int64_t N, int64_t ldb, int8_t *q, int64_t ldq,
                        float *scale)
{
    for (int64_t n = 0; n < N; ++n) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(B[k * ldb + n]);
            if (a > amax)
                amax = a;
        }
        float s = amax / 127.0f;
        scale[n] = s;
        for (int64_t k = 0; k < K; ++k) {
            if (s == 0.0f) {
                q[k * ldq + n] = 0;
                continue;
            }
            float t = rintf(B[k * ldb + n] / s);
            if (t > 127.0f)
                t = 127.0f;
            if (t < -127.0f)
                t = -127.0f;
            q[k * ldq + n] = (int8_t)t;
        }
    }
}

/* ---- the dequantised weight of reading R9: Bd[k][n] = s_n * q[k][n], exact
 * in binary64 (a 24-bit by 8-bit product). */
void oracle_dequant_q8(const int8_t *q, int64_t ldq, const float *scale, int64_t K, int64_t N,
                       double *Bd, int64_t ldd)
{
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            Bd[k * ldd + n] = (double)scale[n] * (double)q[k * ldq + n];
}

/* ---- row norms of the dequantised weight (reading R9 with R1):
 * b[k] = ||(s_n q[k][n])_n||_2, ascending n. */
void oracle_rownorms_q8(const int8_t *q, int64_t ldq, const float *scale, int64_t K, int64_t N,
                        double *b)
{
    for (int64_t k = 0; k < K; ++k) {
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double v = (double)scale[n] * (double)q[k * ldq + n];
            acc += v * v;
        }
        b[k] = sqrt(acc);
    }
}
