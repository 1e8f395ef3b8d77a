// rmm_api.hip -- the extern "C" entry points of librmm.so (include/rmm.h).
//
// Host code only: argument validation (every RMM_EINVAL / RMM_EUNSUPPORTED is
// decided before anything is enqueued), workspace carving, and kernel
// launches on the caller's stream.  No allocation, no host synchronisation.
#include "../../include/rmm.h"
#include "rmm_internal.h"
#include "rmm_select.h"

#include <atomic>
#include <cmath>
#include <mutex>

using namespace rmm;

namespace {

constexpr size_t kWsAlign = 256;

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned8(const void *p) { return ((uintptr_t)p & 7u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

int elem_size(int dt) { return dt == RMM_BF16 ? 2 : dt == RMM_F32 ? 4 : 0; }

// a [rows][ld] matrix of type dt: non-NULL, 16-byte aligned, rows 16-byte aligned
bool ok_matrix(const void *p, int dt, int64_t cols, int64_t ld)
{
    const int es = elem_size(dt);
    if (!p || es == 0 || cols < 1 || ld < cols) return false;
    return aligned16(p) && (ld * es) % 16 == 0;
}

hipStream_t as_stream(void *s) { return (hipStream_t)s; }

int hip_status(hipError_t e) { return e == hipSuccess ? RMM_OK : RMM_EHIP; }

}  // namespace

extern "C" {

int64_t rmm_kk(double r, int64_t K)
{
    if (!(r > 0.0) || !(r <= 1.0) || K < 1) return -1;
    return kk_rule(r, K);
}

int64_t rmm_kk_pad(int64_t kk) { return kk < 1 ? -1 : pad_up(kk); }

const char *rmm_strerror(int status)
{
    switch (status) {
    case RMM_OK: return "success";
    case RMM_EINVAL: return "invalid argument";
    case RMM_EUNSUPPORTED: return "unsupported shape or type";
    case RMM_EHIP: return "HIP runtime error";
    case RMM_ESCRATCH: return "the call needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
    }
}

int rmm_rownorms(const void *B, int dt, int64_t K, int64_t N, int64_t ldb, double *bnorm, void *stream)
{
    if (K < 1 || !ok_matrix(B, dt, N, ldb) || !bnorm || !aligned8(bnorm)) return RMM_EINVAL;
    return hip_status(launch_rownorms(B, dt, K, N, ldb, bnorm, as_stream(stream)));
}

size_t rmm_select_workspace_bytes(int64_t M, int64_t K, int64_t group_rows, int have_scores,
                                  int norms_from_B)
{
    if (M < 1 || K < 1 || group_rows < 1) return 0;
    const int64_t G = (M + group_rows - 1) / group_rows;
    size_t n = 0;
    if (!have_scores) n += align_up((size_t)G * (size_t)K * sizeof(float));
    if (norms_from_B) n += align_up((size_t)K * sizeof(double));
    return n;
}

}  // extern "C"

namespace {

// Argument check of rmm_select and rmm_select_gather (host only, nothing is
// enqueued): RMM_OK, RMM_EINVAL or RMM_EUNSUPPORTED.
int linear_check(const void *A, int dt, int64_t M, int64_t K, int64_t lda, const double *bnorm, const void *B,
                 int64_t N, int64_t ldb, double r, int64_t group_rows, const int32_t *idx, int64_t ldidx,
                 const float *scores, const float *thresh, const double *bound, const void *ws, size_t ws_bytes)
{
    if (M < 1 || K < 1 || group_rows < 1 || !ok_matrix(A, dt, K, lda)) return RMM_EINVAL;
    const int64_t kk = rmm_kk(r, K);
    if (kk < 1) return RMM_EINVAL;
    if (!idx || !aligned16(idx) || ldidx < pad_up(kk) || ldidx % 4 != 0) return RMM_EINVAL;
    if (bnorm && !aligned8(bnorm)) return RMM_EINVAL;
    const bool from_B = !bnorm && B;
    if (from_B && !ok_matrix(B, dt, N, ldb)) return RMM_EINVAL;
    if (scores && !aligned4(scores)) return RMM_EINVAL;
    if (thresh && !aligned4(thresh)) return RMM_EINVAL;
    if (bound && !aligned8(bound)) return RMM_EINVAL;
    const size_t need = rmm_select_workspace_bytes(M, K, group_rows, scores != nullptr, from_B);
    if (need > ws_bytes || (need && (!ws || !aligned16(ws)))) return RMM_EINVAL;
    if (K > kSelectMaxK) return RMM_EUNSUPPORTED;
    return RMM_OK;
}

// Validation, B norms and column scores shared by rmm_select and
// rmm_select_gather; on RMM_OK `sc` holds the G x K scores on the stream and
// `sh` the selection shape.
int linear_scores(const void *A, int dt, int64_t M, int64_t K, int64_t lda, const double *bnorm, const void *B,
                  int64_t N, int64_t ldb, double r, int64_t group_rows, int32_t *idx, int64_t ldidx,
                  float *scores, float *thresh, double *bound, void *ws, size_t ws_bytes, hipStream_t s,
                  float *&sc, SelectShape &sh)
{
    if (int st = linear_check(A, dt, M, K, lda, bnorm, B, N, ldb, r, group_rows, idx, ldidx, scores, thresh,
                              bound, ws, ws_bytes))
        return st;
    const int64_t kk = rmm_kk(r, K);
    const bool from_B = !bnorm && B;

    const int64_t G = (M + group_rows - 1) / group_rows;
    char *w = (char *)ws;
    sc = scores;
    if (!sc) {
        sc = (float *)w;
        w += align_up((size_t)G * K * sizeof(float));
    }
    const double *bn = bnorm;
    if (from_B) {
        double *tmp = (double *)w;
        if (hipError_t e = launch_rownorms(B, dt, K, N, ldb, tmp, s)) return hip_status(e);
        bn = tmp;
    }
    if (hipError_t e = launch_colscore(A, dt, M, K, lda, bn, group_rows, sc, s)) return hip_status(e);
    sh = SelectShape{};
    sh.groups = G;
    sh.K = K;
    sh.lds = K;
    sh.kk = kk;
    sh.pv = 0;
    return RMM_OK;
}

}  // namespace

extern "C" {

int rmm_select(const void *A, int dt, int64_t M, int64_t K, int64_t lda, const double *bnorm,
               const void *B, int64_t N, int64_t ldb, double r, int64_t group_rows, int32_t *idx,
               int64_t ldidx, float *scores, float *thresh, double *bound, void *ws,
               size_t ws_bytes, void *stream)
{
    hipStream_t s = as_stream(stream);
    float *sc = nullptr;
    SelectShape sh;
    if (int st = linear_scores(A, dt, M, K, lda, bnorm, B, N, ldb, r, group_rows, idx, ldidx, scores, thresh,
                               bound, ws, ws_bytes, s, sc, sh))
        return st;
    return hip_status(launch_select(sc, sh, idx, ldidx, thresh, bound, s));
}

int rmm_scores(const void *A, int dt, int64_t M, int64_t K, int64_t lda, const double *bnorm, const void *B,
               int64_t N, int64_t ldb, int64_t group_rows, float *scores, void *ws, size_t ws_bytes, void *stream)
{
    if (M < 1 || K < 1 || group_rows < 1 || !ok_matrix(A, dt, K, lda)) return RMM_EINVAL;
    if (!scores || !aligned4(scores)) return RMM_EINVAL;
    if (bnorm && !aligned8(bnorm)) return RMM_EINVAL;
    const bool from_B = !bnorm && B;
    if (from_B && !ok_matrix(B, dt, N, ldb)) return RMM_EINVAL;
    const size_t need = rmm_select_workspace_bytes(M, K, group_rows, 1, from_B);
    if (need > ws_bytes || (need && (!ws || !aligned16(ws)))) return RMM_EINVAL;
    hipStream_t s = as_stream(stream);
    const double *bn = bnorm;
    if (from_B) {
        double *tmp = (double *)ws;
        if (hipError_t e = launch_rownorms(B, dt, K, N, ldb, tmp, s)) return hip_status(e);
        bn = tmp;
    }
    return hip_status(launch_colscore(A, dt, M, K, lda, bn, group_rows, scores, s));
}

int rmm_select_scores(const float *scores, int64_t G, int64_t K, int64_t ld_scores, double r, int32_t *idx,
                      int64_t ldidx, float *thresh, double *bound, void *stream)
{
    if (G < 1 || K < 1 || ld_scores < K || !scores || !aligned4(scores)) return RMM_EINVAL;
    const int64_t kk = rmm_kk(r, K);
    if (kk < 1) return RMM_EINVAL;
    if (!idx || !aligned16(idx) || ldidx < pad_up(kk) || ldidx % 4 != 0) return RMM_EINVAL;
    if (thresh && !aligned4(thresh)) return RMM_EINVAL;
    if (bound && !aligned8(bound)) return RMM_EINVAL;
    if (K > kSelectMaxK) return RMM_EUNSUPPORTED;
    SelectShape sh{};
    sh.groups = G;
    sh.K = K;
    sh.lds = ld_scores;
    sh.kk = kk;
    sh.pv = 0;
    return hip_status(launch_select(scores, sh, idx, ldidx, thresh, bound, as_stream(stream)));
}

int rmm_select_gather(const void *A, int dt, int64_t M, int64_t K, int64_t lda, const double *bnorm,
                      const void *B, int64_t N, int64_t ldb, double r, int64_t group_rows, int32_t *idx,
                      int64_t ldidx, uint16_t *Apanel, int64_t ldp, float *scores, float *thresh,
                      double *bound, void *ws, size_t ws_bytes, void *stream)
{
    const int64_t kk = rmm_kk(r, K);
    if (kk < 1 || !ok_matrix(Apanel, RMM_BF16, pad_up(kk), ldp)) return RMM_EINVAL;
    hipStream_t s = as_stream(stream);
    float *sc = nullptr;
    SelectShape sh;
    if (int st = linear_scores(A, dt, M, K, lda, bnorm, B, N, ldb, r, group_rows, idx, ldidx, scores, thresh,
                               bound, ws, ws_bytes, s, sc, sh))
        return st;
    SelectGather ga{};
    int nrb = 0;
    if (select_gather_plan(dt, M, K, lda, group_rows, ga, nrb)) {
        ga.A = (const uint16_t *)A;
        ga.Ap = Apanel;
        ga.ldp = ldp;
        return hip_status(launch_select_gather(sc, sh, idx, ldidx, thresh, bound, ga, nrb, s));
    }
    if (hipError_t e = launch_select(sc, sh, idx, ldidx, thresh, bound, s)) return hip_status(e);
    return hip_status(launch_gather(A, dt, M, K, lda, idx, ldidx, kk, group_rows, Apanel, ldp, nullptr, 0, 0,
                                    nullptr, 0, s));
}

int rmm_gather(const void *A, int dt, int64_t M, int64_t K, int64_t lda, const int32_t *idx,
               int64_t ldidx, int64_t kk, int64_t group_rows, uint16_t *Apanel, int64_t ldp,
               const void *B, int64_t N, int64_t ldb, uint16_t *Bpanel, int64_t ldbp, void *stream)
{
    if (M < 1 || K < 1 || group_rows < 1 || !ok_matrix(A, dt, K, lda)) return RMM_EINVAL;
    if (kk < 1 || kk > K) return RMM_EINVAL;
    if (!idx || !aligned16(idx) || ldidx < kk || ldidx % 4 != 0) return RMM_EINVAL;
    const int64_t kpad = pad_up(kk);
    if (!ok_matrix(Apanel, RMM_BF16, kpad, ldp)) return RMM_EINVAL;
    if (Bpanel) {
        if ((M + group_rows - 1) / group_rows != 1) return RMM_EINVAL;
        if (!ok_matrix(B, dt, N, ldb) || N % 8 != 0) return RMM_EINVAL;
        if (!ok_matrix(Bpanel, RMM_BF16, N, ldbp)) return RMM_EINVAL;
    }
    return hip_status(launch_gather(A, dt, M, K, lda, idx, ldidx, kk, group_rows, Apanel, ldp, B, N, ldb,
                                    Bpanel, ldbp, as_stream(stream)));
}

size_t rmm_gemm_workspace_bytes(int64_t, int64_t, int64_t, int64_t) { return 0; }

int rmm_gemm(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, const int32_t *idx,
             int64_t ldidx, int64_t M, int64_t N, int64_t kk, int64_t group_rows, void *Y, int ydt,
             int64_t ldy, void *ws, size_t ws_bytes, void *stream)
{
    (void)ws;
    (void)ws_bytes;
    if (M < 1 || N < 1 || kk < 1 || group_rows < 1) return RMM_EINVAL;
    if (!ok_matrix(A, RMM_BF16, kk, lda)) return RMM_EINVAL;
    if (!ok_matrix(B, RMM_BF16, N, ldb) || N % 8 != 0) return RMM_EINVAL;
    if (idx && (!aligned16(idx) || ldidx < kk || ldidx % 4 != 0)) return RMM_EINVAL;
    if (!ok_matrix(Y, ydt, N, ldy)) return RMM_EINVAL;
    if (kk > INT32_MAX || (M + group_rows - 1) / group_rows > INT32_MAX / 64) return RMM_EUNSUPPORTED;
    return hip_status(launch_gemm(A, lda, B, ldb, idx, ldidx, M, N, kk, group_rows, Y, ydt, ldy,
                                  as_stream(stream)));
}

int rmm_quantize_q8(const uint16_t *B, int64_t K, int64_t N, int64_t ldb, int8_t *Bq, int64_t ldq,
                    float *scale, void *stream)
{
    if (K < 1 || !ok_matrix(B, RMM_BF16, N, ldb) || N % 16 != 0) return RMM_EINVAL;
    if (!Bq || !aligned16(Bq) || ldq < N || ldq % 16 != 0 || !scale || !aligned4(scale)) return RMM_EINVAL;
    if (K > INT32_MAX || K * (N / 16) > (int64_t)INT32_MAX * 256) return RMM_EUNSUPPORTED;
    return hip_status(launch_quantize_q8(B, K, N, ldb, Bq, ldq, scale, as_stream(stream)));
}

int rmm_rownorms_q8(const int8_t *Bq, int64_t ldq, const float *scale, int64_t K, int64_t N,
                    double *bnorm, void *stream)
{
    if (K < 1 || N < 1 || N % 16 != 0 || !Bq || !aligned16(Bq) || ldq < N || ldq % 16 != 0) return RMM_EINVAL;
    if (!scale || !aligned4(scale) || !bnorm || !aligned8(bnorm)) return RMM_EINVAL;
    return hip_status(launch_rownorms_q8(Bq, ldq, scale, K, N, bnorm, as_stream(stream)));
}

size_t rmm_gemm_q8_workspace_bytes(int64_t M, int64_t N, int64_t kk, int64_t group_rows)
{
    (void)kk;
    if (M < 1 || N < 1 || group_rows < 1) return 0;
    return gemm_q8_workspace_bytes(M, N, group_rows);
}

int rmm_gemm_q8(const uint16_t *A, int64_t lda, const int8_t *Bq, int64_t ldq, const float *scale,
                const int32_t *idx, int64_t ldidx, int64_t M, int64_t N, int64_t kk, int64_t group_rows,
                void *Y, int ydt, int64_t ldy, void *ws, size_t ws_bytes, void *stream)
{
    if (M < 1 || N < 1 || kk < 1 || group_rows < 1) return RMM_EINVAL;
    if (!ok_matrix(A, RMM_BF16, kk, lda)) return RMM_EINVAL;
    if (!Bq || !aligned16(Bq) || N % 16 != 0 || ldq < N || ldq % 16 != 0) return RMM_EINVAL;
    if (!scale || !aligned4(scale)) return RMM_EINVAL;
    if (idx && (!aligned16(idx) || ldidx < kk || ldidx % 4 != 0)) return RMM_EINVAL;
    if (!ok_matrix(Y, ydt, N, ldy)) return RMM_EINVAL;
    if (kk > INT32_MAX || (M + group_rows - 1) / group_rows > INT32_MAX / 64 ||
        (double)((M + group_rows - 1) / group_rows) * ((group_rows + 63) / 64) * ((N + 127) / 128) > INT32_MAX / 2)
        return RMM_EUNSUPPORTED;
    const size_t need = gemm_q8_workspace_bytes(M, N, group_rows);
    if (need > ws_bytes || (need && (!ws || !aligned16(ws)))) return RMM_EINVAL;
    return hip_status(launch_gemm_q8(A, lda, Bq, ldq, scale, idx, ldidx, M, N, kk, group_rows, Y, ydt, ldy,
                                     ws, ws_bytes, as_stream(stream)));
}

size_t rmm_attn_pv_workspace_bytes(int64_t H, int64_t L, int64_t D, double r, int64_t qblock,
                                   int causal, int have_idx_out, int have_scores_out)
{
    (void)causal;
    if (H < 1 || L < 1 || D < 1 || qblock < 1) return 0;
    if (!(r > 0.0) || !(r < 1.0)) return 0;  // r == 1 (or invalid): no scoring, no selection
    const int64_t G = (L + qblock - 1) / qblock;
    size_t n = align_up((size_t)H * L * sizeof(double));
    if (!have_scores_out) n += align_up((size_t)H * G * L * sizeof(float));
    if (!have_idx_out) n += align_up((size_t)H * G * pad_up(L) * sizeof(int32_t));
    return n;
}

}  // extern "C"

namespace {

// argument checks shared by the P.V entry points; RMM_OK when all hold
int pv_check(const uint16_t *Pt, const uint16_t *V, int64_t H, int64_t L, int64_t D, int64_t qblock)
{
    if (H < 1 || L < 1 || D < 1 || qblock < 1) return RMM_EINVAL;
    if (!Pt || !V || !aligned16(Pt) || !aligned16(V)) return RMM_EINVAL;
    return RMM_OK;
}

int pv_shape_supported(int64_t L, int64_t D, int64_t qblock)
{
    return D == 128 && qblock == 128 && L % 8 == 0 && L <= kSelectMaxK;
}

// scores + kept-key lists into caller buffers (workspace carved as documented)
int pv_select_impl(const uint16_t *Pt, const uint16_t *V, int64_t H, int64_t L, int64_t D, double r,
                   int64_t qblock, int causal, int32_t *ix, int64_t ldix, float *scores_out, char *w,
                   hipStream_t s)
{
    const int64_t G = (L + qblock - 1) / qblock;
    double *vnorm = (double *)w;
    w += align_up((size_t)H * L * sizeof(double));
    float *sc = scores_out;
    if (!sc) sc = (float *)w;
    if (hipError_t e = launch_pv_score(Pt, V, H, L, D, qblock, causal, vnorm, sc, s)) return hip_status(e);
    SelectShape sh{};
    sh.groups = H * G;
    sh.K = L;
    sh.lds = L;
    sh.pv = 1;
    sh.Gq = G;
    sh.qblock = qblock;
    sh.causal = causal;
    sh.r = r;
    return hip_status(launch_select(sc, sh, ix, ldix, nullptr, nullptr, s));
}

}  // namespace

extern "C" {

int rmm_attn_pv(const uint16_t *Pt, const uint16_t *V, int64_t H, int64_t L, int64_t D, double r,
                int64_t qblock, int causal, void *O, int odt, int32_t *idx_out, int64_t ldidx_out,
                float *scores_out, void *ws, size_t ws_bytes, void *stream)
{
    if (int e = pv_check(Pt, V, H, L, D, qblock)) return e;
    if (!(r > 0.0) || !(r <= 1.0)) return RMM_EINVAL;
    if (!O || elem_size(odt) == 0 || !aligned16(O)) return RMM_EINVAL;
    if (scores_out && !aligned4(scores_out)) return RMM_EINVAL;
    if (idx_out && (!aligned16(idx_out) || ldidx_out % 4 != 0 || ldidx_out < pad_up(L)))
        return RMM_EINVAL;
    if (!pv_shape_supported(L, D, qblock)) return RMM_EUNSUPPORTED;
    const bool dense = r >= 1.0;
    const size_t need = rmm_attn_pv_workspace_bytes(H, L, D, r, qblock, causal, idx_out != nullptr,
                                                    scores_out != nullptr);
    if (need > ws_bytes || (need && (!ws || !aligned16(ws)))) return RMM_EINVAL;

    hipStream_t s = as_stream(stream);
    if (dense)
        return hip_status(launch_pv_gemm(Pt, V, H, L, qblock, causal, 1.0, nullptr, 0, O, odt, s));
    const int64_t G = (L + qblock - 1) / qblock;
    char *w = (char *)ws;
    // workspace: V norms, then scores (unless given), then kept keys (unless given)
    char *after = w + align_up((size_t)H * L * sizeof(double));
    if (!scores_out) after += align_up((size_t)H * G * L * sizeof(float));
    int32_t *ix = idx_out;
    int64_t ldix = ldidx_out;
    if (!ix) {
        ix = (int32_t *)after;
        ldix = pad_up(L);
    }
    if (int e = pv_select_impl(Pt, V, H, L, D, r, qblock, causal, ix, ldix, scores_out, w, s)) return e;
    return hip_status(launch_pv_gemm(Pt, V, H, L, qblock, causal, r, ix, ldix, O, odt, s));
}

int rmm_pv_select(const uint16_t *Pt, const uint16_t *V, int64_t H, int64_t L, int64_t D, double r,
                  int64_t qblock, int causal, int32_t *idx_out, int64_t ldidx_out, float *scores_out,
                  void *ws, size_t ws_bytes, void *stream)
{
    if (int e = pv_check(Pt, V, H, L, D, qblock)) return e;
    if (!(r > 0.0) || !(r < 1.0)) return RMM_EINVAL;
    if (!idx_out || !aligned16(idx_out) || ldidx_out % 4 != 0 || ldidx_out < pad_up(L)) return RMM_EINVAL;
    if (scores_out && !aligned4(scores_out)) return RMM_EINVAL;
    if (!pv_shape_supported(L, D, qblock)) return RMM_EUNSUPPORTED;
    const size_t need = rmm_attn_pv_workspace_bytes(H, L, D, r, qblock, causal, 1, scores_out != nullptr);
    if (need > ws_bytes || !ws || !aligned16(ws)) return RMM_EINVAL;
    return pv_select_impl(Pt, V, H, L, D, r, qblock, causal, idx_out, ldidx_out, scores_out, (char *)ws,
                          as_stream(stream));
}

int rmm_pv_gemm(const uint16_t *Pt, const uint16_t *V, int64_t H, int64_t L, int64_t D, double r,
                int64_t qblock, int causal, const int32_t *idx, int64_t ldidx, void *O, int odt,
                void *stream)
{
    if (int e = pv_check(Pt, V, H, L, D, qblock)) return e;
    if (!O || elem_size(odt) == 0 || !aligned16(O)) return RMM_EINVAL;
    if (idx) {
        if (!(r > 0.0) || !(r <= 1.0)) return RMM_EINVAL;
        if (!aligned16(idx) || ldidx % 4 != 0 || ldidx < pad_up(L)) return RMM_EINVAL;
    }
    if (!pv_shape_supported(L, D, qblock)) return RMM_EUNSUPPORTED;
    return hip_status(launch_pv_gemm(Pt, V, H, L, qblock, causal, idx ? r : 1.0, idx, idx ? ldidx : 0, O, odt,
                                     as_stream(stream)));
}

}  // extern "C"

// ------------------------------------------------------------------ attention producer
namespace {

bool attn_shape_supported(int64_t L, int64_t D, int64_t qblock)
{
    return D == 128 && qblock == 128 && L % 8 == 0 && L <= kSelectMaxK;
}

int attn_check(const uint16_t *Q, const uint16_t *K, int64_t H, int64_t L, int64_t D, int64_t qblock)
{
    if (H < 1 || L < 1 || D < 1 || qblock < 1) return RMM_EINVAL;
    if (!Q || !K || !aligned16(Q) || !aligned16(K)) return RMM_EINVAL;
    return RMM_OK;
}

}  // namespace

extern "C" {

size_t rmm_qk_select_workspace_bytes(int64_t H, int64_t L, int64_t D, int64_t qblock, int have_scores_out)
{
    if (H < 1 || L < 1 || D < 1 || qblock < 1) return 0;
    const int64_t G = (L + qblock - 1) / qblock;
    size_t n = align_up((size_t)H * G * D * sizeof(double));   // key sums of squares
    if (!have_scores_out) n += align_up((size_t)H * G * D * sizeof(float));
    return n;
}

int rmm_qk_select(const uint16_t *Q, const uint16_t *K, int64_t H, int64_t L, int64_t D, double r,
                  int64_t qblock, int causal, int use_k, int32_t *idx_out, int64_t ldidx_out,
                  float *scores_out, void *ws, size_t ws_bytes, void *stream)
{
    if (int e = attn_check(Q, K, H, L, D, qblock)) return e;
    if (!(r > 0.0) || !(r <= 1.0)) return RMM_EINVAL;
    if (!idx_out || !aligned16(idx_out) || ldidx_out % 4 != 0 || ldidx_out < pad_up(D)) return RMM_EINVAL;
    if (scores_out && !aligned4(scores_out)) return RMM_EINVAL;
    if (!attn_shape_supported(L, D, qblock)) return RMM_EUNSUPPORTED;
    const size_t need = rmm_qk_select_workspace_bytes(H, L, D, qblock, scores_out != nullptr);
    if (need > ws_bytes || (need && (!ws || !aligned16(ws)))) return RMM_EINVAL;
    hipStream_t s = as_stream(stream);
    const int64_t G = (L + qblock - 1) / qblock;
    char *w = (char *)ws;
    double *ksum = (double *)w;
    w += align_up((size_t)H * G * D * sizeof(double));
    float *sc = scores_out ? scores_out : (float *)w;
    if (hipError_t e = launch_qk_score(Q, K, H, L, causal ? 1 : 0, use_k ? 1 : 0, ksum, sc, s))
        return hip_status(e);
    SelectShape sh{};
    sh.groups = H * G;
    sh.K = D;
    sh.lds = D;
    sh.kk = kk_rule(r, D);
    return hip_status(launch_select(sc, sh, idx_out, ldidx_out, nullptr, nullptr, s));
}

size_t rmm_attn_probs_workspace_bytes(int64_t H, int64_t L, int64_t D, int have_pv_scores)
{
    (void)D;
    if (H < 1 || L < 1 || !have_pv_scores) return 0;
    return align_up((size_t)H * L * sizeof(double));
}

int rmm_attn_probs(const uint16_t *Q, const uint16_t *K, int64_t H, int64_t L, int64_t D, int64_t qblock,
                   int causal, const int32_t *idx_qk, int64_t ldidx_qk, double r_qk, uint16_t *Pt,
                   const uint16_t *V, float *pv_scores, void *ws, size_t ws_bytes, void *stream)
{
    if (int e = attn_check(Q, K, H, L, D, qblock)) return e;
    if (!Pt || !aligned16(Pt)) return RMM_EINVAL;
    int64_t kk = D;
    if (idx_qk) {
        if (!(r_qk > 0.0) || !(r_qk <= 1.0)) return RMM_EINVAL;
        kk = kk_rule(r_qk, D);
        if (!aligned4(idx_qk) || ldidx_qk < kk) return RMM_EINVAL;
    }
    if (pv_scores && (!aligned4(pv_scores) || !V || !aligned16(V))) return RMM_EINVAL;
    if (!attn_shape_supported(L, D, qblock)) return RMM_EUNSUPPORTED;
    const size_t need = rmm_attn_probs_workspace_bytes(H, L, D, pv_scores != nullptr);
    if (need > ws_bytes || (need && (!ws || !aligned16(ws)))) return RMM_EINVAL;
    hipStream_t s = as_stream(stream);
    double *vnorm = nullptr;
    if (pv_scores) {
        vnorm = (double *)ws;
        if (hipError_t e = launch_pv_vnorm(V, H, L, D, vnorm, s)) return hip_status(e);
    }
    return hip_status(launch_attn_probs(Q, K, H, L, causal ? 1 : 0, idx_qk, idx_qk ? ldidx_qk : 0, kk, Pt, vnorm,
                                        pv_scores, s));
}

int rmm_pv_select_scores(const float *scores, int64_t H, int64_t L, double r, int64_t qblock, int causal,
                         int32_t *idx_out, int64_t ldidx_out, void *stream)
{
    if (H < 1 || L < 1 || qblock < 1) return RMM_EINVAL;
    if (!scores || !aligned4(scores)) return RMM_EINVAL;
    if (!(r > 0.0) || !(r < 1.0)) return RMM_EINVAL;
    if (!idx_out || !aligned16(idx_out) || ldidx_out % 4 != 0 || ldidx_out < pad_up(L)) return RMM_EINVAL;
    if (qblock != 128 || L % 8 != 0 || L > kSelectMaxK) return RMM_EUNSUPPORTED;
    const int64_t G = (L + qblock - 1) / qblock;
    SelectShape sh{};
    sh.groups = H * G;
    sh.K = L;
    sh.lds = L;
    sh.pv = 1;
    sh.Gq = G;
    sh.qblock = qblock;
    sh.causal = causal;
    sh.r = r;
    return hip_status(launch_select(scores, sh, idx_out, ldidx_out, nullptr, nullptr, as_stream(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------- no-allocation variant
// Scratch of rmm_select_gather_noalloc: a fixed array in device memory, one
// copy per GPU the library runs on, held until the process ends.  Host code
// never passes the array's own name to a kernel or a copy (in host code it is
// a stand-in, not a device address): it passes the address
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[RMM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_ptr(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RMM_EHIP;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RMM_EHIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return RMM_OK;
}

}  // namespace

extern "C" int rmm_select_gather_noalloc(const void *A, int dt, int64_t M, int64_t K, int64_t lda,
                                         const double *bnorm, const void *B, int64_t N, int64_t ldb, double r,
                                         int64_t group_rows, int32_t *idx, int64_t ldidx, uint16_t *Apanel,
                                         int64_t ldp, float *scores, float *thresh, double *bound, void *stream)
{
    // every argument check of rmm_select_gather first, against a workspace of
    // unlimited size (nothing is enqueued and no HIP call is made on failure)
    const int64_t kk = rmm_kk(r, K);
    if (kk < 1 || !ok_matrix(Apanel, RMM_BF16, pad_up(kk), ldp)) return RMM_EINVAL;
    static const __attribute__((aligned(256))) unsigned char stand_in[16] = {};
    if (int st = linear_check(A, dt, M, K, lda, bnorm, B, N, ldb, r, group_rows, idx, ldidx, scores, thresh,
                              bound, stand_in, SIZE_MAX))
        return st;
    const size_t need = rmm_select_workspace_bytes(M, K, group_rows, scores != nullptr, !bnorm && B);
    if (need > RMM_NOALLOC_SCRATCH_BYTES) return RMM_ESCRATCH;
    void *ws = nullptr;
    if (int st = scratch_ptr(&ws)) return st;
    // the scores (and B norms computed on the fly) are written in full before
    // they are read, so the contents a previous call left need no clearing
    return rmm_select_gather(A, dt, M, K, lda, bnorm, B, N, ldb, r, group_rows, idx, ldidx, Apanel, ldp, scores,
                             thresh, bound, ws, RMM_NOALLOC_SCRATCH_BYTES, stream);
}
