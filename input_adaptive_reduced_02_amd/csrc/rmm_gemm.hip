// rmm_gemm.hip -- the reduced product A[:, I] B[I, :] on MFMA (gfx950).
//
// "Reduced Matrix Multiplication..." technical summary, Metodologia >
// Mecanismo Central: only the kept contraction slices enter the product.  Per
// selection group g (group_rows consecutive rows of Y):
//     Y[rows_g, :] = Apanel[rows_g, 0:kk] * B[I_g, :]
// with Apanel the gathered bf16 columns and the kept rows of B read in place
// by index (each kept row segment is contiguous, so the loads coalesce and
// dropped rows of B are never fetched).  With no index list the same kernel
// reads B rows 0..kk-1: the dense baseline at r = 1, or a packed B panel.
//
// Tiling: 256 threads = 4 waves; a workgroup owns a TM x TN tile of one group
// and walks the kept slices in BK-deep slabs through a double-buffered LDS
// pipeline (global loads of slab t+1 in flight while slab t feeds the MFMAs,
// one barrier per slab).  v_mfma_f32_32x32x16_bf16, fp32 accumulation.
// Workgroup w runs on XCD w % 8; tiles are numbered so that each XCD gets a
// contiguous range of N tiles with all their row tiles, so the B columns a
// tile strip needs are fetched into that XCD's L2 once and reused by every
// group.
//
// Kernels, by shape:
//   k_gemm_wb  128 x 256 tiles, 4 waves of 128 x 64, two workgroups per CU,
//              kept B rows straight into registers (an index list, groups of
//              more than 64 rows, at least 512 tiles, bf16 output)
//   k_gemm_wt  the same tiles with B through LDS by DMA (the dense product
//              on those shapes)
//   k_gemm_dl  128 x 256 tiles, 8 waves of 64 x 64 (other prefill shapes)
//   k_gemm_sk  64 x 128 tiles streaming the kept rows (<= 64 rows per group,
//              e.g. decode: many N tiles over the kept rows of a wide weight)
//   k_gemm     register-staged fallback (leading dimensions the DMA
//              pipelines do not cover)
#include "rmm_gemm_dl.h"
#include "rmm_gemm_sk.h"
#include "rmm_gemm_wt.h"
#include "rmm_gemm_wb.h"

#ifndef RMM_DL_WAVES
#define RMM_DL_WAVES 8
#endif
#ifndef RMM_DL_WM
#define RMM_DL_WM 2
#endif
#include "rmm_tile.h"

namespace rmm {

template <int TM, int TN, int BK, int WM, int WN>
__global__ void __launch_bounds__(256)
k_gemm(const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
       const int32_t *__restrict__ idx, int64_t ldidx, int64_t M, int64_t N, int64_t kk, int64_t gr,
       void *__restrict__ Y, int ydt, int64_t ldy, int tiles_per_group, int m_tiles, int n_tiles)
{
    constexpr int WAVES_N = TN / WN;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int CH = BK / 8;                  // 16-byte chunks per LDS row
    constexpr int A_CHUNKS = TM * CH / 256;     // A chunks loaded per thread per slab
    static_assert((TM / WM) * (TN / WN) == 4, "4 waves");
    static_assert((BK / 8) * (TN / 8) == 256, "one 8x8 B unit per thread");
    static_assert(TM * CH % 256 == 0, "A chunks divide evenly");

    __shared__ __attribute__((aligned(16))) uint16_t As[2][TM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][TN * BK];

    // ---- tile of this workgroup (XCD-aware numbering)
    const int total = m_tiles * n_tiles;
    const int per = (total + 7) / 8;
    const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (t >= total) return;
    const int nt = t / m_tiles, mt = t % m_tiles;
    const int64_t g = mt / tiles_per_group;
    const int64_t row0 = g * gr + (int64_t)(mt % tiles_per_group) * TM;
    const int64_t row_end = (g * gr + gr < M) ? g * gr + gr : M;
    const int64_t col0 = (int64_t)nt * TN;
    const int32_t *I = idx ? idx + g * ldidx : nullptr;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int b_n0 = 8 * (tid % (TN / 8));
    const int b_kb = tid / (TN / 8);
    const bool b_col_ok = col0 + b_n0 < N;

    const uint16_t *a_src[A_CHUNKS];
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        const int q = tid + 256 * i;
        int64_t row = row0 + q / CH;
        if (row > M - 1) row = M - 1;
        a_src[i] = A + row * lda + (q % CH) * 8;
    }
    const uint16_t *b_src = B + col0 + b_n0;

    floatx16 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.0f;

    uint4 ra[A_CHUNKS];
    uint4 rb[8];

    auto load = [&](int kt) {
        const int64_t kbase = (int64_t)kt * BK;
        if (kbase + BK <= kk) {
#pragma unroll
            for (int i = 0; i < A_CHUNKS; ++i) ra[i] = *(const uint4 *)(a_src[i] + kbase);
            int32_t ks[8];
            const int64_t j0 = kbase + b_kb * 8;
            if (I) {
                const int4 x0 = *(const int4 *)(I + j0), x1 = *(const int4 *)(I + j0 + 4);
                ks[0] = x0.x; ks[1] = x0.y; ks[2] = x0.z; ks[3] = x0.w;
                ks[4] = x1.x; ks[5] = x1.y; ks[6] = x1.z; ks[7] = x1.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) ks[i] = (int32_t)(j0 + i);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                rb[i] = b_col_ok ? *(const uint4 *)(b_src + (int64_t)ks[i] * ldb) : make_uint4(0, 0, 0, 0);
        } else {
            // last, partial slab: columns / rows at or past kk read as zero
#pragma unroll
            for (int i = 0; i < A_CHUNKS; ++i) {
                const int q = tid + 256 * i;
                const int64_t j = kbase + (q % CH) * 8;
                if (j + 8 <= kk) ra[i] = *(const uint4 *)(a_src[i] + kbase);
                else if (j < kk) ra[i] = keep_first(*(const uint4 *)(a_src[i] + kbase), (int)(kk - j));
                else ra[i] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t j = kbase + b_kb * 8 + i;
                if (j < kk && b_col_ok) {
                    const int64_t k = I ? (int64_t)I[j] : j;
                    rb[i] = *(const uint4 *)(b_src + k * ldb);
                } else {
                    rb[i] = make_uint4(0, 0, 0, 0);
                }
            }
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int q = tid + 256 * i;
            st_a<BK>(As[buf], q / CH, q % CH, ra[i]);
        }
        st_unit_t<BK>(Bs[buf], b_n0, b_kb, rb);
    };

    const int nkt = (int)((kk + BK - 1) / BK);
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nkt) load(kt + 1);
        mfma_slab<BK, FM, FN>(As[cur], Bs[cur], wm * WM, wn * WN, lane, acc);
        if (kt + 1 < nkt) store(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: fp32 accumulators -> Y (bf16 round-to-nearest-even or fp32)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int64_t col = col0 + wn * WN + fn * 32 + acc_col(lane);
            if (col >= N) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = row0 + wm * WM + fm * 32 + acc_row(lane, v);
                if (row >= row_end) continue;
                if (ydt == 1)
                    ((uint16_t *)Y)[row * ldy + col] = (uint16_t)f32_to_bf16(acc[fm][fn][v]);
                else
                    ((float *)Y)[row * ldy + col] = acc[fm][fn][v];
            }
        }
    }
}

template <int TM, int TN, int BK, int WM, int WN>
static hipError_t launch_shape(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                               const int32_t *idx, int64_t ldidx, int64_t M, int64_t N, int64_t kk,
                               int64_t gr, void *Y, int ydt, int64_t ldy, hipStream_t s)
{
    const int64_t G = (M + gr - 1) / gr;
    const int64_t rows_per_group = gr < M ? gr : M;
    const int tpg = (int)((rows_per_group + TM - 1) / TM);
    const int m_tiles = (int)(G * tpg);
    const int n_tiles = (int)((N + TN - 1) / TN);
    const int total = m_tiles * n_tiles;
    const int per = (total + 7) / 8;
    hipLaunchKernelGGL((k_gemm<TM, TN, BK, WM, WN>), dim3((unsigned)(8 * per)), dim3(256), 0, s, A, lda, B,
                       ldb, idx, ldidx, M, N, kk, gr, Y, ydt, ldy, tpg, m_tiles, n_tiles);
    return hipGetLastError();
}

// tiles from which the two-per-CU kernels run: two per CU of the 256 CUs of an
// MI355X (with fewer, a CU holds one workgroup and k_gemm_dl is faster)
constexpr int64_t kTwoPerCuMinTiles = 512;

hipError_t launch_gemm(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                       const int32_t *idx, int64_t ldidx, int64_t M, int64_t N, int64_t kk,
                       int64_t group_rows, void *Y, int ydt, int64_t ldy, hipStream_t s)
{
    const int64_t rows = group_rows < M ? group_rows : M;
    const int64_t kslab = (kk + 63) / 64 * 64;
    // two 128 x 256 workgroups per CU when there are at least two tiles per
    // CU (bf16 output; A byte offsets fit 32 bits): with an index list the
    // kept B rows go straight into registers (k_gemm_wb, which also needs a
    // B row stride under 2^23 elements for its 24-bit offset multiply), the
    // dense product streams B through LDS (k_gemm_wt); each measured the
    // faster on its case
    if (rows > 64 && lda >= kslab && (!idx || ldidx >= kslab) && ydt == 1 && M * lda * 2 < (int64_t(1) << 32)) {
        constexpr int TN = 256;
        const int64_t G = (M + group_rows - 1) / group_rows;
        const int tpg = (int)((rows + 127) / 128);
        const int m_tiles = (int)(G * tpg);
        const int n_tiles = (int)((N + TN - 1) / TN);
        if ((int64_t)m_tiles * n_tiles >= kTwoPerCuMinTiles) {
            const int per = (m_tiles * n_tiles + 7) / 8;
            if (idx && ldb * 2 < (int64_t(1) << 24)) {
                // the largest B row whose byte offset row * ldb * 2 + 2N fits 32 bits
                int64_t lim = ((int64_t(1) << 32) - 1 - 2 * N) / (2 * ldb);
                if (lim > (int64_t(1) << 24) - 1) lim = (int64_t(1) << 24) - 1;
                hipLaunchKernelGGL((k_gemm_wb<4>), dim3((unsigned)(8 * per)), dim3(256), 0, s, A, lda, B, ldb, idx,
                                   ldidx, M, N, kk, group_rows, (uint16_t *)Y, ldy, tpg, m_tiles, n_tiles,
                                   (uint32_t)lim);
            } else if (idx) {
                hipLaunchKernelGGL((k_gemm_wt<TN, 32, 3, true>), dim3((unsigned)(8 * per)), dim3(256), 0, s, A, lda,
                                   B, ldb, idx, ldidx, M, N, kk, group_rows, Y, ydt, ldy, tpg, m_tiles, n_tiles);
            } else {
                hipLaunchKernelGGL((k_gemm_wt<TN, 32, 3, false>), dim3((unsigned)(8 * per)), dim3(256), 0, s, A, lda,
                                   B, ldb, idx, ldidx, M, N, kk, group_rows, Y, ydt, ldy, tpg, m_tiles, n_tiles);
            }
            return hipGetLastError();
        }
    }
    // DMA pipeline: every A row and index row must be readable up to the slab end
    if (rows > 64 && lda >= kslab && (!idx || ldidx >= kslab)) {
        constexpr int NW = RMM_DL_WAVES, WMS = RMM_DL_WM;
        using S = DlShape<NW, WMS>;
        const int64_t G = (M + group_rows - 1) / group_rows;
        const int tpg = (int)((rows + S::TM - 1) / S::TM);
        const int m_tiles = (int)(G * tpg);
        const int n_tiles = (int)((N + S::TN - 1) / S::TN);
        const int per = (m_tiles * n_tiles + 7) / 8;
        if (idx)
            hipLaunchKernelGGL((k_gemm_dl<NW, WMS, true>), dim3((unsigned)(8 * per)), dim3(64 * NW), 0, s, A, lda, B,
                               ldb, idx, ldidx, M, N, kk, group_rows, Y, ydt, ldy, tpg, m_tiles, n_tiles);
        else
            hipLaunchKernelGGL((k_gemm_dl<NW, WMS, false>), dim3((unsigned)(8 * per)), dim3(64 * NW), 0, s, A, lda, B,
                               ldb, idx, ldidx, M, N, kk, group_rows, Y, ydt, ldy, tpg, m_tiles, n_tiles);
        return hipGetLastError();
    }
    if (rows <= 64 && lda >= kslab && (!idx || ldidx >= kslab)) {
        using S = SkShape;
        const int64_t G = (M + group_rows - 1) / group_rows;
        const int m_tiles = (int)G;
        const int n_tiles = (int)((N + S::TN - 1) / S::TN);
        const int per = (m_tiles * n_tiles + 7) / 8;
        if (idx)
            hipLaunchKernelGGL((k_gemm_sk<true>), dim3((unsigned)(8 * per)), dim3(64 * S::NW), 0, s, A, lda, B, ldb,
                               idx, ldidx, M, N, kk, group_rows, Y, ydt, ldy, 1, m_tiles, n_tiles);
        else
            hipLaunchKernelGGL((k_gemm_sk<false>), dim3((unsigned)(8 * per)), dim3(64 * S::NW), 0, s, A, lda, B, ldb,
                               idx, ldidx, M, N, kk, group_rows, Y, ydt, ldy, 1, m_tiles, n_tiles);
        return hipGetLastError();
    }
    if (rows <= 64)
        return launch_shape<64, 64, 256, 32, 32>(A, lda, B, ldb, idx, ldidx, M, N, kk, group_rows, Y, ydt, ldy, s);
    return launch_shape<128, 256, 64, 64, 128>(A, lda, B, ldb, idx, ldidx, M, N, kk, group_rows, Y, ydt, ldy, s);
}

}  // namespace rmm
