// rmm_pv.hip -- P.V reduced along the key (token) dimension on MFMA (gfx950).
//
// "Reduced Matrix Multiplication..." technical summary, Metodologia > Escopo
// de Aplicacao: the reduction also applies to the token dimension of PV.  For
// head h and query block g:
//     O[h, q0:q0+128, :] = sum over kept keys k of P[h, q, k] * V[h, k, :]
// P is stored key-major (Pt[h][k][q] = P[h][q][k]): the 128 probabilities a
// block needs from key k are one contiguous 256-byte segment, and V[h][k][:]
// is another.  Both operands are therefore gathered on load by key index --
// no gather pass -- and dropped keys are never read.  Both arrive
// contraction-major and are transposed in registers into the k-contiguous LDS
// layout the MFMA wants (rmm_tile.h).
//
// One workgroup per (head, block): a 128 x 128 output tile, 4 waves of 64x64,
// 64 keys per slab, double-buffered LDS (64 KiB, two workgroups per CU).
// Threads 0..127 load P units, 128..255 load V units.  Blocks are dispatched
// last-block first: with a causal mask the late blocks carry the most keys.
// With no index list the kept set is the whole causal prefix (r = 1).
#include "rmm_tile.h"

namespace rmm {

__global__ void __launch_bounds__(256)
k_pv_gemm(const uint16_t *__restrict__ Pt, const uint16_t *__restrict__ V, int64_t H, int64_t L,
          int64_t Gq, int64_t qb, int causal, double r, const int32_t *__restrict__ idx,
          int64_t ldidx, void *__restrict__ O, int odt)
{
    constexpr int TM = 128, TN = 128, BK = 64, WM = 64, WN = 64, FM = 2, FN = 2, D = 128;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][TM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][TN * BK];

    const int64_t b = blockIdx.x;
    const int64_t g = Gq - 1 - b / H;
    const int64_t h = b % H;
    const int64_t q0 = g * qb;
    const int64_t Kg = causal ? ((qb * (g + 1) < L) ? qb * (g + 1) : L) : L;
    const int64_t kk = idx ? kk_rule(r, Kg) : Kg;
    const int32_t *I = idx ? idx + (h * Gq + g) * ldidx : nullptr;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const bool is_p = tid < 128;
    const int u = tid & 127;
    const int n0 = 8 * (u & 15);     // query offset (P) or d offset (V)
    const int kb = u >> 4;           // 8-key chunk of the slab
    // P units: Pt[h][key][q0 + n0 .. +7]; V units: V[h][key][n0 .. +7]
    const bool col_ok = is_p ? (q0 + n0 < L) : true;
    const uint16_t *src = is_p ? Pt + h * L * L + q0 + n0 : V + h * L * D + n0;
    const int64_t stride = is_p ? L : D;
    uint16_t *dst0 = is_p ? As[0] : Bs[0];
    uint16_t *dst1 = is_p ? As[1] : Bs[1];

    floatx16 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.0f;

    uint4 rows[8];
    auto load = [&](int kt) {
        const int64_t j0 = (int64_t)kt * BK + kb * 8;
        if (j0 + 8 <= kk && col_ok) {
            int32_t ks[8];
            if (I) {
                const int4 x0 = *(const int4 *)(I + j0), x1 = *(const int4 *)(I + j0 + 4);
                ks[0] = x0.x; ks[1] = x0.y; ks[2] = x0.z; ks[3] = x0.w;
                ks[4] = x1.x; ks[5] = x1.y; ks[6] = x1.z; ks[7] = x1.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) ks[i] = (int32_t)(j0 + i);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) rows[i] = *(const uint4 *)(src + (int64_t)ks[i] * stride);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t j = j0 + i;
                if (j < kk && col_ok) {
                    const int64_t k = I ? (int64_t)I[j] : j;
                    rows[i] = *(const uint4 *)(src + k * stride);
                } else {
                    rows[i] = make_uint4(0, 0, 0, 0);
                }
            }
        }
    };

    const int nkt = (int)((kk + BK - 1) / BK);
    load(0);
    st_unit_t<BK>(dst0, n0, kb, rows);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nkt) load(kt + 1);
        mfma_slab<BK, FM, FN>(As[cur], Bs[cur], wm * WM, wn * WN, lane, acc);
        if (kt + 1 < nkt) st_unit_t<BK>(cur ? dst0 : dst1, n0, kb, rows);
        __syncthreads();
    }

    const int64_t nq = (L - q0 < qb) ? (L - q0) : qb;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int col = wn * WN + fn * 32 + acc_col(lane);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * WM + fm * 32 + acc_row(lane, v);
                if (row >= nq) continue;
                const int64_t o = (h * L + q0 + row) * D + col;
                if (odt == 1)
                    ((uint16_t *)O)[o] = (uint16_t)f32_to_bf16(acc[fm][fn][v]);
                else
                    ((float *)O)[o] = acc[fm][fn][v];
            }
        }
    }
}

hipError_t launch_pv_gemm(const uint16_t *Pt, const uint16_t *V, int64_t H, int64_t L,
                          int64_t qblock, int causal, double r, const int32_t *idx, int64_t ldidx,
                          void *O, int odt, hipStream_t s)
{
    const int64_t Gq = (L + qblock - 1) / qblock;
    hipLaunchKernelGGL(k_pv_gemm, dim3((unsigned)(H * Gq)), dim3(256), 0, s, Pt, V, H, L, Gq, qblock,
                       causal, r, idx, ldidx, O, odt);
    return hipGetLastError();
}

}  // namespace rmm
