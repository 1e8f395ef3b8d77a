// rmm_internal.h -- device helpers and kernel launchers shared by the HIP
// sources of librmm.so.  Not part of the public ABI (that is include/rmm.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rmm {

// native vector (not HIP's struct uint4): arrays of it stay in registers
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kPad = 64;        // panel / index-row padding (RMM_KPAD)
constexpr int kSelectThreads = 1024;
constexpr int64_t kSelectMaxK = 32768;

// Retained count, identical arithmetic on host and device: x = r*K in
// binary64; snap to the nearest integer when within 1e-9*K, else ceil;
// clamp to [1, K].  Both sides use IEEE multiply, rint (nearest-even),
// fabs and ceil, all exact or correctly rounded, so they agree bit for bit.
__host__ __device__ inline int64_t kk_rule(double r, int64_t K)
{
    double x = r * (double)K;
    double n = rint(x);
    int64_t kk = (fabs(x - n) <= 1e-9 * (double)K) ? (int64_t)n : (int64_t)ceil(x);
    if (kk < 1) kk = 1;
    if (kk > K) kk = K;
    return kk;
}

__host__ __device__ inline int64_t pad_up(int64_t kk) { return (kk + kPad - 1) / kPad * kPad; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// binary32 -> bf16 bits, round to nearest, ties to even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// 8x8 transpose of 16-bit elements held as 8 rows of uint4 (8 halves each):
// out[e] holds element e of every input row, rows in order.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8])
{
    uint32_t w[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        w[i][0] = in[i].x; w[i][1] = in[i].y; w[i][2] = in[i].z; w[i][3] = in[i].w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t a = w[2 * p][e >> 1], b = w[2 * p + 1][e >> 1];
            // even e: low halves of rows 2p, 2p+1; odd e: high halves
            o[p] = (e & 1) ? __builtin_amdgcn_perm(b, a, 0x07060302u)
                           : __builtin_amdgcn_perm(b, a, 0x05040100u);
        }
        out[e] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// ---- launchers (host side; each returns the launch's hipGetLastError())
hipError_t launch_rownorms(const void *B, int dt, int64_t K, int64_t N, int64_t ldb, double *out,
                           hipStream_t s);
hipError_t launch_colscore(const void *A, int dt, int64_t M, int64_t K, int64_t lda,
                           const double *bnorm, int64_t group_rows, float *scores, hipStream_t s);
hipError_t launch_pv_score(const uint16_t *Pt, const uint16_t *V, int64_t H, int64_t L, int64_t D,
                           int64_t qblock, int causal, double *vnorm, float *scores, hipStream_t s);
// linear: groups = G, every group has K candidates and keeps kk.
// pv: groups = H*Gq; group i is block (i % Gq) of its head, candidates
// K_g = min(L, qblock*(g+1)) when causal, kk_g = kk_rule(r, K_g).
struct SelectShape {
    int64_t groups;
    int64_t K;         // scores row length (linear: K, pv: L)
    int64_t lds;       // scores row stride
    int64_t kk;        // linear: fixed kk; pv: ignored
    int pv;            // 0 linear, 1 pv
    int64_t Gq;        // pv: blocks per head
    int64_t qblock;    // pv
    int causal;        // pv
    double r;          // pv
};
hipError_t launch_select(const float *scores, const SelectShape &sh, int32_t *idx, int64_t ldidx,
                         float *thresh, double *bound, hipStream_t s);
hipError_t launch_gather(const void *A, int dt, int64_t M, int64_t K, int64_t lda, const int32_t *idx,
                         int64_t ldidx, int64_t kk, int64_t group_rows, uint16_t *Ap, int64_t ldp,
                         const void *B, int64_t N, int64_t ldb, uint16_t *Bp, int64_t ldbp,
                         hipStream_t s);
hipError_t launch_gemm(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                       const int32_t *idx, int64_t ldidx, int64_t M, int64_t N, int64_t kk,
                       int64_t group_rows, void *Y, int ydt, int64_t ldy, hipStream_t s);
hipError_t launch_quantize_q8(const uint16_t *B, int64_t K, int64_t N, int64_t ldb, int8_t *q,
                              int64_t ldq, float *scale, hipStream_t s);
hipError_t launch_rownorms_q8(const int8_t *q, int64_t ldq, const float *scale, int64_t K, int64_t N,
                              double *out, hipStream_t s);
size_t gemm_q8_workspace_bytes(int64_t M, int64_t N, int64_t group_rows);
hipError_t launch_gemm_q8(const uint16_t *A, int64_t lda, const int8_t *Bq, int64_t ldq,
                          const float *scale, const int32_t *idx, int64_t ldidx, int64_t M, int64_t N,
                          int64_t kk, int64_t group_rows, void *Y, int ydt, int64_t ldy, void *ws, size_t ws_bytes,
                          hipStream_t s);
hipError_t launch_pv_vnorm(const uint16_t *V, int64_t H, int64_t L, int64_t D, double *vnorm, hipStream_t s);
hipError_t launch_qk_score(const uint16_t *Q, const uint16_t *K, int64_t H, int64_t L, int causal, int use_k,
                           double *ksum, float *scores, hipStream_t s);
hipError_t launch_attn_probs(const uint16_t *Q, const uint16_t *K, int64_t H, int64_t L, int causal,
                             const int32_t *idx, int64_t ldidx, int64_t kk, uint16_t *Pt, const double *vnorm,
                             float *pvs, hipStream_t s);
hipError_t launch_pv_gemm(const uint16_t *Pt, const uint16_t *V, int64_t H, int64_t L,
                          int64_t qblock, int causal, double r, const int32_t *idx, int64_t ldidx,
                          void *O, int odt, hipStream_t s);

}  // namespace rmm
