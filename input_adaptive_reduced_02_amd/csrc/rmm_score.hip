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
// Grid (ceil(K / 512), G); each lane owns two adjacent columns of one group
// and walks the group's rows top to bottom, UNROLL rows of loads in flight.
constexpr int kColUnroll = 32;

template <int DT>
__global__ void __launch_bounds__(256)
k_colscore(const void *__restrict__ Av, int64_t M, int64_t K, int64_t lda,
           const double *__restrict__ bnorm, int64_t gr, float *__restrict__ scores)
{
    const int64_t g = blockIdx.y;
    const int64_t c0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 2;
    if (c0 >= K) return;
    const int64_t r0 = g * gr;
    const int64_t rows = (M - r0 < gr) ? (M - r0) : gr;
    const bool pair = (c0 + 1 < K);
    double a0 = 0.0, a1 = 0.0;
    if (DT == 1) {
        const uint16_t *p = (const uint16_t *)Av + r0 * lda + c0;
        if (pair) {
            int64_t m = 0;
            for (; m + kColUnroll <= rows; m += kColUnroll) {
                uint32_t w[kColUnroll];
#pragma unroll
                for (int u = 0; u < kColUnroll; ++u) w[u] = *(const uint32_t *)(p + (m + u) * lda);
#pragma unroll
                for (int u = 0; u < kColUnroll; ++u) {
                    double lo = bf16_lo(w[u]), hi = bf16_hi(w[u]);
                    a0 = __builtin_fma(lo, lo, a0);
                    a1 = __builtin_fma(hi, hi, a1);
                }
            }
            for (; m < rows; ++m) {
                uint32_t w = *(const uint32_t *)(p + m * lda);
                double lo = bf16_lo(w), hi = bf16_hi(w);
                a0 = __builtin_fma(lo, lo, a0);
                a1 = __builtin_fma(hi, hi, a1);
            }
        } else {
            for (int64_t m = 0; m < rows; ++m) {
                double x = bf16_to_f32(p[m * lda]);
                a0 = __builtin_fma(x, x, a0);
            }
        }
    } else {
        const float *p = (const float *)Av + r0 * lda + c0;
        if (pair) {
            int64_t m = 0;
            for (; m + kColUnroll <= rows; m += kColUnroll) {
                float2 w[kColUnroll];
#pragma unroll
                for (int u = 0; u < kColUnroll; ++u) w[u] = *(const float2 *)(p + (m + u) * lda);
#pragma unroll
                for (int u = 0; u < kColUnroll; ++u) {
                    double x0 = w[u].x, x1 = w[u].y;
                    a0 = __builtin_fma(x0, x0, a0);
                    a1 = __builtin_fma(x1, x1, a1);
                }
            }
            for (; m < rows; ++m) {
                float2 w = *(const float2 *)(p + m * lda);
                double x0 = w.x, x1 = w.y;
                a0 = __builtin_fma(x0, x0, a0);
                a1 = __builtin_fma(x1, x1, a1);
            }
        } else {
            for (int64_t m = 0; m < rows; ++m) {
                double x = p[m * lda];
                a0 = __builtin_fma(x, x, a0);
            }
        }
    }
    float *out = scores + g * K + c0;
    const double b0 = bnorm ? bnorm[c0] : 1.0;
    out[0] = (float)(__builtin_sqrt(a0) * b0);
    if (pair) {
        const double b1 = bnorm ? bnorm[c0 + 1] : 1.0;
        out[1] = (float)(__builtin_sqrt(a1) * b1);
    }
}

hipError_t launch_colscore(const void *A, int dt, int64_t M, int64_t K, int64_t lda,
                           const double *bnorm, int64_t group_rows, float *scores, hipStream_t s)
{
    const int64_t G = (M + group_rows - 1) / group_rows;
    dim3 grid((unsigned)((K + 511) / 512), (unsigned)G);
    if (dt == 1)
        hipLaunchKernelGGL(k_colscore<1>, grid, dim3(256), 0, s, A, M, K, lda, bnorm, group_rows, scores);
    else
        hipLaunchKernelGGL(k_colscore<0>, grid, dim3(256), 0, s, A, M, K, lda, bnorm, group_rows, scores);
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
