// rmm_score.hip -- scoring kernels of the RMM hot path (gfx950).
//
// The score of contraction slice k for a group of rows is the activation
// column norm ||A[rows, k]||_2 ("Reduced Matrix Multiplication..." technical
// summary, Metodologia > Estrategia de Selecao), multiplied in this library
// by the weight row norm ||B[k, :]||_2.  For P.V the score of key k for a
// query block is the block's column mass of P times ||V[k, :]||_2 (reduction
// of the token dimension of PV, Metodologia > Escopo de Aplicacao).
//
// All three kernels are HBM-bound streams.  Each lane owns whole sums and
// adds its terms in ascending index order in binary64 (squares of bf16 and
// binary32 values are exact in binary64, and fma(x, x, acc) rounds once, the
// same as acc + x*x with an exact product), then takes a correctly rounded
// sqrt and rounds the score once to binary32.  Coalescing comes from
// neighbouring lanes owning neighbouring columns (colscore) or from wide
// per-lane loads of contiguous rows (rownorms, pv_score).
#include "rmm_internal.h"

namespace rmm {

// ------------------------------------------------------------------ B row norms
// One lane per row; the row is read in 16-byte vectors, summed left to right.
template <int DT>
__global__ void __launch_bounds__(256)
k_rownorms(const void *__restrict__ Bv, int64_t K, int64_t N, int64_t ldb, double *__restrict__ out)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= K) return;
    double acc = 0.0;
    if (DT == 1) {
        const uint16_t *row = (const uint16_t *)Bv + k * ldb;
        int64_t n = 0;
        for (; n + 32 <= N; n += 32) {
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *(const uint4 *)(row + n + 8 * u);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    double lo = bf16_lo(w[i]), hi = bf16_hi(w[i]);
                    acc = __builtin_fma(lo, lo, acc);
                    acc = __builtin_fma(hi, hi, acc);
                }
            }
        }
        for (; n < N; ++n) {
            double x = bf16_to_f32(row[n]);
            acc = __builtin_fma(x, x, acc);
        }
    } else {
        const float *row = (const float *)Bv + k * ldb;
        int64_t n = 0;
        for (; n + 4 <= N; n += 4) {
            float4 v = *(const float4 *)(row + n);
            double x0 = v.x, x1 = v.y, x2 = v.z, x3 = v.w;
            acc = __builtin_fma(x0, x0, acc);
            acc = __builtin_fma(x1, x1, acc);
            acc = __builtin_fma(x2, x2, acc);
            acc = __builtin_fma(x3, x3, acc);
        }
        for (; n < N; ++n) {
            double x = row[n];
            acc = __builtin_fma(x, x, acc);
        }
    }
    out[k] = __builtin_sqrt(acc);
}

hipError_t launch_rownorms(const void *B, int dt, int64_t K, int64_t N, int64_t ldb, double *out,
                           hipStream_t s)
{
    dim3 grid((unsigned)((K + 255) / 256));
    if (dt == 1)
        hipLaunchKernelGGL(k_rownorms<1>, grid, dim3(256), 0, s, B, K, N, ldb, out);
    else
        hipLaunchKernelGGL(k_rownorms<0>, grid, dim3(256), 0, s, B, K, N, ldb, out);
    return hipGetLastError();
}

// ------------------------------------------------------------------ column scores
// Grid (ceil(K / 128), G), 128 lanes per workgroup; each lane owns one column
// of one group and walks the group's rows top to bottom, the loads of up to
// kColUnroll rows in flight (consecutive lanes read consecutive columns, so
// every row load of a wave is one coalesced 128- or 256-byte segment).
constexpr int kColUnroll = 64;
constexpr int kColThreads = 128;

template <int DT>
__device__ __forceinline__ double load_elem(const void *p, int64_t i)
{
    if (DT == 1) return (double)bf16_to_f32(((const uint16_t *)p)[i]);
    return (double)((const float *)p)[i];
}

template <int DT>
__global__ void __launch_bounds__(kColThreads)
k_colscore(const void *__restrict__ Av, int64_t M, int64_t K, int64_t lda,
           const double *__restrict__ bnorm, int64_t gr, float *__restrict__ scores)
{
    const int64_t g = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * kColThreads + threadIdx.x;
    if (c >= K) return;
    const int64_t r0 = g * gr;
    const int64_t rows = (M - r0 < gr) ? (M - r0) : gr;
    const char *p = (const char *)Av + (r0 * lda + c) * (DT == 1 ? 2 : 4);
    const int64_t ld = lda * (DT == 1 ? 2 : 4);   // row stride in bytes
    double a = 0.0;
    int64_t m = 0;
    for (; m + kColUnroll <= rows; m += kColUnroll) {
        double x[kColUnroll];
#pragma unroll
        for (int u = 0; u < kColUnroll; ++u) x[u] = load_elem<DT>(p + (m + u) * ld, 0);
#pragma unroll
        for (int u = 0; u < kColUnroll; ++u) a = __builtin_fma(x[u], x[u], a);
    }
    for (; m < rows; ++m) {
        const double x = load_elem<DT>(p + m * ld, 0);
        a = __builtin_fma(x, x, a);
    }
    const double b = bnorm ? bnorm[c] : 1.0;
    scores[g * K + c] = (float)(__builtin_sqrt(a) * b);
}

hipError_t launch_colscore(const void *A, int dt, int64_t M, int64_t K, int64_t lda,
                           const double *bnorm, int64_t group_rows, float *scores, hipStream_t s)
{
    const int64_t G = (M + group_rows - 1) / group_rows;
    dim3 grid((unsigned)((K + kColThreads - 1) / kColThreads), (unsigned)G);
    if (dt == 1)
        hipLaunchKernelGGL(k_colscore<1>, grid, dim3(kColThreads), 0, s, A, M, K, lda, bnorm, group_rows,
                           scores);
    else
        hipLaunchKernelGGL(k_colscore<0>, grid, dim3(kColThreads), 0, s, A, M, K, lda, bnorm, group_rows,
                           scores);
    return hipGetLastError();
}

// ------------------------------------------------------------------ P.V scores
// Grid (ceil(L / 256), H).  Lane = key k of head h.  First ||V[h][k][:]||_2
// (ascending d), then for every query block g whose causal prefix contains k
// the mass of P over the block's queries (ascending q), read from the
// contiguous key-major row Pt[h][k][q0 .. q0+nq), 64 values in flight.
__global__ void __launch_bounds__(256)
k_pv_score(const uint16_t *__restrict__ Pt, const uint16_t *__restrict__ V, int64_t L, int64_t D,
           int64_t qblock, int causal, double *__restrict__ vnorm, float *__restrict__ scores)
{
    const int64_t h = blockIdx.y;
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= L) return;
    const int64_t G = (L + qblock - 1) / qblock;
    const uint16_t *vrow = V + (h * L + k) * D;
    double vv = 0.0;
    for (int64_t d = 0; d < D; d += 8) {
        uint4 v = *(const uint4 *)(vrow + d);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            double lo = bf16_lo(w[i]), hi = bf16_hi(w[i]);
            vv = __builtin_fma(lo, lo, vv);
            vv = __builtin_fma(hi, hi, vv);
        }
    }
    const double vn = __builtin_sqrt(vv);
    vnorm[h * L + k] = vn;
    const uint16_t *prow = Pt + (h * L + k) * L;
    float *srow = scores + (h * G) * L + k;
    const int64_t g0 = causal ? k / qblock : 0;
    for (int64_t g = g0; g < G; ++g) {
        const int64_t q0 = g * qblock;
        const int64_t nq = (L - q0 < qblock) ? (L - q0) : qblock;
        double mass = 0.0;
        int64_t i = 0;
        for (; i + 64 <= nq; i += 64) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = *(const uint4 *)(prow + q0 + i + 8 * u);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    mass += (double)bf16_lo(w[j]);
                    mass += (double)bf16_hi(w[j]);
                }
            }
        }
        for (; i < nq; ++i) mass += (double)bf16_to_f32(prow[q0 + i]);
        srow[g * L] = (float)(mass * vn);
    }
}

hipError_t launch_pv_score(const uint16_t *Pt, const uint16_t *V, int64_t H, int64_t L, int64_t D,
                           int64_t qblock, int causal, double *vnorm, float *scores, hipStream_t s)
{
    dim3 grid((unsigned)((L + 255) / 256), (unsigned)H);
    hipLaunchKernelGGL(k_pv_score, grid, dim3(256), 0, s, Pt, V, L, D, qblock, causal, vnorm, scores);
    return hipGetLastError();
}

}  // namespace rmm
