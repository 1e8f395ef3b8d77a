/*
 * rmm.h -- C ABI of librmm.so: the hot path of Reduced Matrix Multiplication
 * (RMM) on AMD Instinct MI355X (gfx950).
 *
 * Method: "Reduced Matrix Multiplication: Input-Adaptive Matrix-Product
 * Reduction for LLM Inference" (Lan, Li, Zhou).  Its technical summary
 * (gist.science, section "Metodologia") writes each Transformer matmul as
 * Y = A B, scores every index of the shared contraction dimension from the
 * current input, keeps the ceil(rho d) best and forms only A[:, I] B[I, :];
 * it applies this to XW projections, to QK^T and to P V along the token
 * dimension ("Escopo de Aplicacao").  The authors' abstract (arXiv
 * 2608.13426) states the reduction keeps model weights unmodified and needs no
 * training.
 *
 * Readings of this library where the pages are silent:
 *   - score of slice k in a group of rows = ||A[rows, k]||_2 * ||B[k, :]||_2;
 *     with no B norms it is the pages' activation-only score ||A[rows, k]||_2;
 *   - one selection per group of `group_rows` consecutive rows (the last group
 *     may be short); a whole matrix is one group when group_rows >= M;
 *   - kk = rmm_kk(r, K) (ceil(r*K) for decimal r, see below);
 *   - equal scores go to the lower index;
 *   - scores are accumulated in binary64 and rounded once to binary32, which
 *     is the precision of the keep/drop decision: the linear path's column
 *     norms in ascending row order, the attention-side sums (QK^T feature
 *     norms, P.V key masses) in a fixed order of partial sums added pairwise
 *     (within one binary32 ulp of an ascending sum);
 *   - P.V: per query block g the candidate keys are the causal prefix
 *     k < min(L, qblock*(g+1)); score = block column mass of P * ||V[k, :]||_2.
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *     allocates and frees nothing; scratch memory comes from a caller-owned
 *     workspace sized by the *_workspace_bytes functions (except
 *     rmm_select_gather_noalloc, whose scratch is a fixed per-GPU array).
 *   - Matrices are row-major with explicit leading dimensions in elements.
 *   - Every device pointer is 16-byte aligned, and every leading dimension is
 *     a multiple of 8 (bf16) or 4 (fp32) elements: rows start 16-byte aligned.
 *     A matrix with leading dimension ld is readable for rows*ld elements.
 *   - bf16 tensors are passed as their 16-bit patterns (uint16_t).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; no entry point synchronises the host.
 *   - Return value: RMM_OK, or RMM_EINVAL (bad argument, detected on the host
 *     before anything is enqueued), RMM_EUNSUPPORTED (valid but outside what
 *     the kernels handle, also before anything is enqueued), RMM_EHIP (the
 *     HIP runtime reported an error when enqueueing) or RMM_ESCRATCH (only
 *     rmm_select_gather_noalloc: the call needs more than its fixed scratch).
 *   - Inputs are assumed finite.  Entry points are re-entrant and stateless;
 *     calls on different streams that share no output buffer may overlap
 *     (rmm_select_gather_noalloc excepted: its calls on one GPU share one
 *     scratch array).
 */
#ifndef RMM_H
#define RMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RMM_OK 0
#define RMM_EINVAL (-1)
#define RMM_EUNSUPPORTED (-2)
#define RMM_EHIP (-3)
#define RMM_ESCRATCH (-4)   /* rmm_select_gather_noalloc: the call needs more than its scratch */

/* Bytes of the fixed per-GPU scratch of rmm_select_gather_noalloc. */
#define RMM_NOALLOC_SCRATCH_BYTES (8u << 20)

#define RMM_F32 0
#define RMM_BF16 1

/* Column padding of panels and index rows: kk is rounded up to this. */
#define RMM_KPAD 64

/* Retained count: the number of contraction slices kept out of K at
 * retention ratio r ("Metodologia" > "Estrategia de Selecao": keep
 * ceil(rho d)).  r is read as the decimal the user meant: with x = r*K in
 * binary64, if x is within 1e-9*K of an integer n the result is n, else
 * ceil(x); the result is clamped to [1, K].  Returns -1 when r is not in
 * (0, 1] (NaN included) or K < 1.  Pure host function. */
int64_t rmm_kk(double r, int64_t K);

/* kk rounded up to a multiple of RMM_KPAD (the width of panels and index
 * rows).  Returns -1 for kk < 1. */
int64_t rmm_kk_pad(int64_t kk);

/* Static text of a status code. */
const char *rmm_strerror(int status);

/* B row norms: bnorm[k] = ||B[k, :]||_2 for k < K, summed in binary64 in
 * ascending column order.  This is the weight factor of the score; it depends
 * only on B, so callers compute it once per weight and pass it to every
 * rmm_select call (B itself is never modified).
 *   B      [K][ldb] of type dt (RMM_BF16 or RMM_F32), device
 *   bnorm  [K] binary64, device, written
 * Errors: RMM_EINVAL for NULL pointers, K < 1, N < 1, ldb < N, misalignment. */
int rmm_rownorms(const void *B, int dt, int64_t K, int64_t N, int64_t ldb, double *bnorm,
                 void *stream);

/* Workspace bytes rmm_select needs: room for the [G][K] binary32 scores when
 * the caller passes no `scores` buffer (G = ceil(M / group_rows)), plus K
 * binary64 row norms when it passes B instead of bnorm.  Returns 0 when the
 * caller supplies both or needs neither. */
size_t rmm_select_workspace_bytes(int64_t M, int64_t K, int64_t group_rows, int have_scores,
                                  int norms_from_B);

/* Score and select ("Estrategia de Selecao").  For every group g of
 * group_rows consecutive rows of A:
 *     s[g][k] = binary32( ||A[rows_g, k]||_2 * b_k )
 * with b_k = bnorm[k] if bnorm != NULL; else the row norms of B computed now
 * (a full read of B) if B != NULL; else 1 (the pages' activation-only rule).
 * Then the kk = rmm_kk(r, K) best slices under the order (score descending,
 * index ascending) are written to idx[g*ldidx + 0 .. kk-1] in ascending
 * order; entries kk .. rmm_kk_pad(kk)-1 repeat the last kept index.
 *   A       [M][lda] of type dt, device
 *   bnorm   [K] binary64 or NULL; B [K][ldb] of type dt or NULL (N columns)
 *   idx     [G][ldidx] int32, ldidx >= rmm_kk_pad(kk), ldidx % 4 == 0
 *   scores  [G][K] binary32 or NULL (then held in the workspace)
 *   thresh  [G] binary32 or NULL: the kk-th best score of each group
 *   bound   [G] binary64 or NULL: sum of the dropped scores of each group, an
 *           upper bound of ||A_g B - A_g[:, I] B[I, :]||_F (triangle
 *           inequality, ||a b^T||_F = ||a|| ||b||) when b is the B norms
 *   ws      rmm_select_workspace_bytes(...) bytes, device (NULL if 0)
 * Errors: RMM_EINVAL for bad pointers, sizes, r or a short workspace;
 * RMM_EUNSUPPORTED for K > 32768. */
int rmm_select(const void *A, int dt, int64_t M, int64_t K, int64_t lda, const double *bnorm,
               const void *B, int64_t N, int64_t ldb, double r, int64_t group_rows,
               int32_t *idx, int64_t ldidx, float *scores, float *thresh, double *bound,
               void *ws, size_t ws_bytes, void *stream);

/* The two halves of rmm_select as calls of their own, so a caller (or a
 * benchmark) can run or time the score and the selection separately; their
 * outputs are bit for bit those rmm_select forms.
 * rmm_scores ("Estrategia de Selecao": the score of every slice):
 *   scores[g][k] = binary32( ||A[rows_g, k]||_2 * b_k ), b_k as in rmm_select
 *   (bnorm; else the row norms of B, computed now into the workspace; else 1)
 *   scores  [G][K] binary32, device; ws rmm_select_workspace_bytes(M, K,
 *   group_rows, 1, bnorm == NULL && B != NULL) bytes (0 unless norms come from B)
 * rmm_select_scores (the top-kk selection of every group from given scores):
 *   scores [G][ld_scores] binary32 (ld_scores >= K), kk = rmm_kk(r, K); idx,
 *   thresh and bound exactly as rmm_select writes them (bound is the sum of
 *   the dropped scores as given).  No workspace.
 * Errors: as rmm_select. */
int rmm_scores(const void *A, int dt, int64_t M, int64_t K, int64_t lda, const double *bnorm,
               const void *B, int64_t N, int64_t ldb, int64_t group_rows, float *scores, void *ws,
               size_t ws_bytes, void *stream);
int rmm_select_scores(const float *scores, int64_t G, int64_t K, int64_t ld_scores, double r,
                      int32_t *idx, int64_t ldidx, float *thresh, double *bound, void *stream);

/* Gather ("Mecanismo Central": the columns A[:, I] of the reduced product)
 * into a contiguous bf16 panel:
 *   Apanel[m][j] = bf16(A[m][idx[g*ldidx + j]])  for j < kk, g = m / group_rows
 *   Apanel[m][j] = 0                             for kk <= j < rmm_kk_pad(kk)
 * for rows m < M (binary32 A is rounded to nearest-even bf16).  When Bpanel is
 * not NULL (only with a single group, G == 1) the kept rows of B are packed
 * too: Bpanel[j][:] = bf16(B[idx[j]][:]) for j < kk, zero rows after that.
 *   A       [M][lda] of type dt; idx [G][ldidx] int32 (ldidx >= kk)
 *   Apanel  [M][ldp] bf16, ldp >= rmm_kk_pad(kk)
 *   B       [K][ldb] of type dt (N columns, N % 8 == 0) or NULL
 *   Bpanel  [rmm_kk_pad(kk)][ldbp] bf16 or NULL, ldbp >= N
 * Errors: RMM_EINVAL for bad pointers/sizes, or Bpanel with more than one group. */
int rmm_gather(const void *A, int dt, int64_t M, int64_t K, int64_t lda, const int32_t *idx,
               int64_t ldidx, int64_t kk, int64_t group_rows, uint16_t *Apanel, int64_t ldp,
               const void *B, int64_t N, int64_t ldb, uint16_t *Bpanel, int64_t ldbp,
               void *stream);

/* Selection and gather in one call: the same outputs as rmm_select followed
 * by rmm_gather(A, dt, M, K, lda, idx, ldidx, rmm_kk(r, K), group_rows,
 * Apanel, ldp, NULL, 0, 0, NULL, 0), bit for bit ("Estrategia de Selecao"
 * then "Mecanismo Central").  For bf16 A with K <= 8192 and fewer than 512
 * groups the gather runs inside the selection launch (each group's rows are
 * split over several workgroups that stage them in LDS while the threshold is
 * found), so the kept columns are formed without a second pass over idx;
 * other shapes run the two launches.
 *   arguments as rmm_select, plus
 *   Apanel  [M][ldp] bf16, ldp >= rmm_kk_pad(rmm_kk(r, K)), device
 *   ws      rmm_select_workspace_bytes(...) bytes (the same workspace)
 * Errors: as rmm_select, and RMM_EINVAL for a bad Apanel or ldp. */
int rmm_select_gather(const void *A, int dt, int64_t M, int64_t K, int64_t lda, const double *bnorm,
                      const void *B, int64_t N, int64_t ldb, double r, int64_t group_rows,
                      int32_t *idx, int64_t ldidx, uint16_t *Apanel, int64_t ldp, float *scores,
                      float *thresh, double *bound, void *ws, size_t ws_bytes, void *stream);

/* rmm_select_gather without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs and errors as
 * rmm_select_gather minus ws / ws_bytes; the scratch it needs (the G x K
 * binary32 scores unless `scores` is given, plus K binary64 B norms when they
 * are computed from B) lives in a fixed array of RMM_NOALLOC_SCRATCH_BYTES
 * (8 MiB) in device memory, one per GPU, that the library holds until the
 * process ends.  Nothing is allocated or freed by the call.
 *   - The array is found on the device current at the call (the stream must
 *     belong to it); its address is looked up on the first call on each
 *     device and kept.
 *   - Every call on one GPU shares that GPU's array: calls that may overlap
 *     on one GPU (different streams, or host threads) race and must be
 *     serialised by the caller.  The array keeps the last call's contents;
 *     nothing in it needs to start at zero.
 *   - rmm_select_workspace_bytes(M, K, group_rows, scores != NULL,
 *     bnorm == NULL && B != NULL) must not exceed RMM_NOALLOC_SCRATCH_BYTES
 *     (e.g. G * K <= 2^21 with bnorm given): otherwise RMM_ESCRATCH, before
 *     anything is enqueued.
 * Errors: those of rmm_select_gather (argument errors are decided on the host
 * before any HIP call), RMM_ESCRATCH, RMM_EHIP if the scratch address cannot
 * be obtained. */
int rmm_select_gather_noalloc(const void *A, int dt, int64_t M, int64_t K, int64_t lda,
                              const double *bnorm, const void *B, int64_t N, int64_t ldb, double r,
                              int64_t group_rows, int32_t *idx, int64_t ldidx, uint16_t *Apanel,
                              int64_t ldp, float *scores, float *thresh, double *bound, void *stream);

/* Workspace bytes rmm_gemm needs (currently 0 for every shape). */
size_t rmm_gemm_workspace_bytes(int64_t M, int64_t N, int64_t kk, int64_t group_rows);

/* The reduced product ("Mecanismo Central"), bf16 inputs, fp32 accumulation:
 *   Y[m][n] = sum_{j < kk} A[m][j] * B[row(g, j)][n],   g = m / group_rows,
 *   row(g, j) = idx[g*ldidx + j] if idx != NULL, else j.
 * With idx the kept rows of B are read in place (no B panel); A is the
 * gathered panel.  With idx == NULL, A and B are read as they are: this is
 * the dense product when kk == K (the r = 1 baseline, same kernels), or the
 * product of an A panel with a packed B panel.  Accumulation is ascending in
 * j within each 64-wide slab of a tile, so results are deterministic.
 *   A    [M][lda] bf16, lda >= kk
 *   B    bf16 rows of length N (N % 8 == 0) with leading dimension ldb
 *   idx  [G][ldidx] int32 or NULL, ldidx >= kk, ldidx % 4 == 0
 *   Y    [M][ldy] of type ydt (RMM_BF16: rounded to nearest-even; RMM_F32)
 * Errors: RMM_EINVAL for bad pointers/sizes. */
int rmm_gemm(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, const int32_t *idx,
             int64_t ldidx, int64_t M, int64_t N, int64_t kk, int64_t group_rows, void *Y,
             int ydt, int64_t ldy, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes rmm_attn_pv needs for H heads of length L: per-key V norms,
 * the [H][G][L] block scores (unless scores_out is given) and the kept-key
 * lists (unless idx_out is given), G = ceil(L / qblock).  r == 1 needs none. */
size_t rmm_attn_pv_workspace_bytes(int64_t H, int64_t L, int64_t D, double r, int64_t qblock,
                                   int causal, int have_idx_out, int have_scores_out);

/* P.V reduced along the key (token) dimension ("Escopo de Aplicacao": PV,
 * token dimension).  For head h and query block g (queries
 * q0 = g*qblock .. min(L, q0+qblock)-1), with candidate keys k < K_g
 * (K_g = min(L, qblock*(g+1)) if causal, else L):
 *   score[h][g][k] = binary32( (sum_{q in block} P[h][q][k]) * ||V[h][k][:]||_2 )
 * (the sum in binary64 as eight partial sums, query mod 8, added pairwise)
 *   I = the kk_g = rmm_kk(r, K_g) best keys (ties to the lower index)
 *   O[h][q][:] = sum_{k in I} P[h][q][k] * V[h][k][:]
 * r == 1 skips scoring and selection: the dense causal product, same kernel.
 *   Pt   [H][L][L] bf16, KEY-MAJOR: Pt[h][k][q] = P[h][q][k]
 *   V    [H][L][D] bf16;  O [H][L][D] of type odt
 *   idx_out    [H*G][ldidx_out] int32 or NULL: kept keys, ascending, padded
 *              by repeating the last one up to rmm_kk_pad(kk_g)
 *   scores_out [H][G][L] binary32 or NULL (entries k >= K_g untouched)
 * Supported: D == 128, qblock == 128, L % 8 == 0, L <= 32768, else
 * RMM_EUNSUPPORTED.  Errors: RMM_EINVAL for bad pointers/sizes/r/workspace. */
int rmm_attn_pv(const uint16_t *Pt, const uint16_t *V, int64_t H, int64_t L, int64_t D, double r,
                int64_t qblock, int causal, void *O, int odt, int32_t *idx_out,
                int64_t ldidx_out, float *scores_out, void *ws, size_t ws_bytes, void *stream);

/* The two halves of rmm_attn_pv, for callers that score once and multiply
 * later, or time the product alone.
 *
 * rmm_pv_select: the block scores and kept-key lists of rmm_attn_pv (same
 * definitions, same layouts), without the product.  idx_out is required
 * (ldidx_out % 4 == 0, >= rmm_kk_pad(L)); 0 < r < 1.  Workspace:
 * rmm_attn_pv_workspace_bytes(H, L, D, r, qblock, causal, 1, scores_out != NULL)
 * bytes.  Errors and supported shapes as rmm_attn_pv. */
int rmm_pv_select(const uint16_t *Pt, const uint16_t *V, int64_t H, int64_t L, int64_t D, double r,
                  int64_t qblock, int causal, int32_t *idx_out, int64_t ldidx_out, float *scores_out,
                  void *ws, size_t ws_bytes, void *stream);

/* rmm_pv_gemm: O[h][q][:] = sum over the kept keys k of block g of
 * P[h][q][k] * V[h][k][:], the kept keys of (h, g) being the first
 * rmm_kk(r, K_g) entries of idx[h*G + g][:] (ascending, as rmm_pv_select
 * writes them, ldidx % 4 == 0).  idx == NULL: every key of the causal prefix
 * (the dense product; r is then ignored).  No workspace.  Errors and
 * supported shapes as rmm_attn_pv. */
int rmm_pv_gemm(const uint16_t *Pt, const uint16_t *V, int64_t H, int64_t L, int64_t D, double r,
                int64_t qblock, int causal, const int32_t *idx, int64_t ldidx, void *O, int odt,
                void *stream);

/* ---- int8 weights.  The pages ("Resultados Experimentais", item
 * "Compatibilidade") state that the method works on INT8-quantised weights
 * and fix no scheme.  Format used here: Bq [K][ldq] int8 codes and one
 * binary32 scale per output column,
 *   scale[n] = max_k |B[k][n]| / 127,   Bq[k][n] = round-half-even(B[k][n] / scale[n]),
 * both divisions correctly rounded in binary32, codes in [-127, 127]; an
 * all-zero column has scale 0 and codes 0.  The method runs on the
 * dequantised weight scale[n] * Bq[k][n]: rmm_rownorms_q8 gives its row norms
 * (the B norms rmm_select takes), rmm_gemm_q8 multiplies its kept rows, read
 * as int8 (half the bytes of a bf16 row).  The activation side (score,
 * select, gather) is unchanged.  Layout rules: N % 16 == 0, ldq % 16 == 0,
 * Bq 16-byte aligned, scale 4-byte aligned.
 *
 * rmm_quantize_q8: quantise a bf16 weight B [K][ldb] (finite values) into Bq
 * and scale [N].  Runs once per weight; `scale` doubles as the column-maximum
 * accumulator while it runs. */
int rmm_quantize_q8(const uint16_t *B, int64_t K, int64_t N, int64_t ldb, int8_t *Bq, int64_t ldq,
                    float *scale, void *stream);

/* Row norms of the dequantised weight, binary64 [K]:
 *   bnorm[k] = sqrt(sum_n (scale[n] * Bq[k][n])^2), each term exact, the sum
 * taken in ascending n with one rounding per square and per addition. */
int rmm_rownorms_q8(const int8_t *Bq, int64_t ldq, const float *scale, int64_t K, int64_t N,
                    double *bnorm, void *stream);

/* Workspace bytes rmm_gemm_q8 needs: 0, or, when the output has at most 128
 * tiles of 64 x 256 (each then split over two workgroups along the kept
 * rows), two fp32 64 x 256 partial tiles and one 4-byte arrival counter per
 * tile.  Calls with groups of at most 64 rows, kk <= 4096 and lda and ldidx
 * of at least kk rounded up to 64 run a kernel without split tiles and leave
 * the workspace untouched. */
size_t rmm_gemm_q8_workspace_bytes(int64_t M, int64_t N, int64_t kk, int64_t group_rows);

/* The reduced product on an int8 weight:
 *   Y[m][n] = scale[n] * sum_{j < kk} A[m][j] * Bq[row(g, j)][n],
 * g and row(g, j) as rmm_gemm (idx == NULL: row j, the dense product when
 * kk == K).  A is the bf16 panel of rmm_gemm.  Each product of a bf16 value
 * and a code is exact in fp32; the sum is accumulated in fp32 in a fixed
 * order (deterministic), and the scale multiplies it once; Y as rmm_gemm.
 * ws: rmm_gemm_q8_workspace_bytes(...) bytes, 16-byte aligned, ZERO-FILLED
 * before its first use; each completed call leaves every arrival counter at
 * zero again, so a zero-filled workspace can be reused by later calls of any
 * shape that fits it, also by launches replayed from a HIP graph.  Calls that
 * share a workspace must not overlap.  Errors: RMM_EINVAL for bad
 * pointers/sizes/workspace. */
int rmm_gemm_q8(const uint16_t *A, int64_t lda, const int8_t *Bq, int64_t ldq, const float *scale,
                const int32_t *idx, int64_t ldidx, int64_t M, int64_t N, int64_t kk, int64_t group_rows,
                void *Y, int ydt, int64_t ldy, void *ws, size_t ws_bytes, void *stream);

/* ---- attention: the feature dimension of QK^T and the probabilities
 * ("Escopo de Aplicacao": the method reduces the feature dimension of QK^T
 * and, optionally, the token dimension of PV).  Q, K, V are [H][L][D] bf16
 * (D contiguous).  Query block g holds queries q0 = g*qblock ..
 * min(L, q0+qblock)-1; its candidate keys are k < K_g = min(L, qblock*(g+1))
 * when causal, else every k < L.  Supported: D == 128, qblock == 128,
 * L % 8 == 0, L <= 32768, else RMM_EUNSUPPORTED.  Q, K, V, Pt 16-byte aligned.
 *
 * rmm_qk_select: per (head h, block g), feature j scores
 *   s[h][g][j] = binary32( ||Q[h][block, j]||_2 * ||K[h][0 .. K_g-1, j]||_2 )
 * (use_k == 0: the first factor alone, the pages' activation-only rule), each
 * sum of squares in binary64 -- per 128-row tile four partial sums (row mod
 * 4, ascending) added as (p0 + p1) + (p2 + p3), a causal prefix as the
 * ascending sum of its tiles' sums; the kk = rmm_kk(r, D) best
 * features are kept (ties to the lower index) and written ascending to
 * idx_out[h*G + g][0 .. kk-1], padded by repeating the last one up to
 * rmm_kk_pad(kk).  0 < r <= 1; ldidx_out % 4 == 0, >= rmm_kk_pad(D).
 * scores_out [H][G][D] binary32 or NULL (then the workspace holds them).
 * The workspace (rmm_qk_select_workspace_bytes, 16-byte aligned, device)
 * always holds the binary64 key sums of squares per 128-key tile, H*G*D*8
 * bytes rounded up to 256, followed by the scores when scores_out is NULL. */
size_t rmm_qk_select_workspace_bytes(int64_t H, int64_t L, int64_t D, int64_t qblock, int have_scores_out);
int rmm_qk_select(const uint16_t *Q, const uint16_t *K, int64_t H, int64_t L, int64_t D, double r,
                  int64_t qblock, int causal, int use_k, int32_t *idx_out, int64_t ldidx_out,
                  float *scores_out, void *ws, size_t ws_bytes, void *stream);

/* rmm_attn_probs: the attention probabilities over the kept features,
 *   S[q][k] = sum_{j in I(h, g)} Q[h][q][j] * K[h][k][j] / sqrt(D)
 *   P[q][k] = exp(S[q][k] - max) / sum over the row's keys (k <= q if causal)
 * I(h, g) = idx_qk[(h*G + g)*ldidx_qk + 0 .. kk-1], kk = rmm_kk(r_qk, D), as
 * rmm_qk_select writes it; idx_qk == NULL: every feature (r_qk ignored).
 * Products are exact, sums fp32; exp2 and the final rounding in binary32,
 * stored bf16 (round to nearest even) KEY-MAJOR: Pt[h][k][q] = P[q][k] for
 * every block's candidate keys (0 where k > q); entries past a block's
 * candidates are not written.  Pt is [H][L][L].
 * pv_scores [H][G][L] binary32 or NULL: for k < K_g,
 *   pv_scores[h][g][k] = binary32( (sum over the block's queries of the
 *                                   stored P[q][k]) * ||V[h][k][:]||_2 )
 * in binary64, the sum as eight partial sums (query mod 8, ascending) added
 * pairwise -- the scores rmm_attn_pv forms from Pt, bit for bit, here without reading
 * Pt again; V is then required.  Workspace:
 * rmm_attn_probs_workspace_bytes(H, L, D, pv_scores != NULL) bytes. */
size_t rmm_attn_probs_workspace_bytes(int64_t H, int64_t L, int64_t D, int have_pv_scores);
int rmm_attn_probs(const uint16_t *Q, const uint16_t *K, int64_t H, int64_t L, int64_t D, int64_t qblock,
                   int causal, const int32_t *idx_qk, int64_t ldidx_qk, double r_qk, uint16_t *Pt,
                   const uint16_t *V, float *pv_scores, void *ws, size_t ws_bytes, void *stream);

/* rmm_pv_select_scores: the kept keys of every (head, block) from the
 * pv_scores of rmm_attn_probs, exactly as rmm_pv_select keeps them from its
 * own scores: kk_g = rmm_kk(r, K_g) keys, ascending in idx_out[h*G + g][:],
 * padded by repeating the last one.  0 < r < 1; ldidx_out % 4 == 0,
 * >= rmm_kk_pad(L).  No workspace.  The product is then rmm_pv_gemm. */
int rmm_pv_select_scores(const float *scores, int64_t H, int64_t L, double r, int64_t qblock, int causal,
                         int32_t *idx_out, int64_t ldidx_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RMM_H */
