// rmm_gemm_sk.h -- reduced GEMM for groups of at most 64 rows (decode shapes),
// a deep global->LDS DMA stream (gfx950).  Included by rmm_gemm.hip after
// rmm_gemm_dl.h (shares its DMA helpers and the A-tile swizzle).
//
// Same product as the other GEMM kernels: Y[rows_g, :] = Apanel[rows_g, 0:kk]
// * B[I_g, :], kept rows of B fetched in place by index.  With 64 rows the
// product has about 64 FLOP per byte of B, far below the MFMA/HBM ridge, so
// the kernel is built to keep HBM busy: every workgroup streams the kept rows
// of a 128-column strip of B through a (D+1)-stage LDS ring, D slabs of B in
// flight, and the MFMAs only have to keep up.  D = 3 (48 KiB of B per
// workgroup, about 11 MB over the chip) measured faster than 2, 4 or 5.
//
// Tile 64 x 128 x 64, 4 waves side by side along N (wave w owns columns
// 32w..32w+31 and all 64 rows: 2 x 1 fragments of v_mfma_f32_32x32x16_bf16),
// so each A fragment and each B fragment is read from LDS once per slab.
// A tile: k-contiguous rows of 128 B, chunk c of row r at slot c ^ swz(r).
// B tile: rows of 256 B (one 64-bank line), chunk c of row k at slot
// c ^ 4(k mod 4): the 4 rows x 4 chunks touched by 32 lanes of one transposed
// read land in 16 distinct slots.
//
// Pipeline (D slabs ahead, NSTAGE = D + 1 ring stages, index ring 2D):
//   prologue  IDX(0..D-1), wait; then IDX(p+D), AB(p) for p = 0..D-1
//   step i    wait for AB(i); barrier; LDS reads (rows of slab i+D, all
//             fragments of slab i); IDX(i+2D), AB(i+D); MFMAs on slab i
// AB(x) needs the index slab x, issued before AB(x-D); waiting for AB(x-D)
// therefore also covers it.  Every step issues the same operations (slabs
// past the end reload valid memory: the last A slab and row 0 of B), so the
// count of operations newer than AB(i) is always (D-1) * (1 + AB_OPS).
// Stage (i+D) mod (D+1) held slab i-1, whose readers all passed step i's
// barrier.  A columns at or past kk in the last slab are cleared in registers.
#pragma once
#include "rmm_gemm_dl.h"

namespace rmm {

#ifndef RMM_SK_DEPTH
#define RMM_SK_DEPTH 3
#endif

struct SkShape {
    static constexpr int TM = 64, TN = 128, BK = 64, NW = 4;
    static constexpr int WN = 32, FM = 2, KS = BK / 16;
    static constexpr int D = RMM_SK_DEPTH, NSTAGE = D + 1, IDX_RING = 2 * D;
    static constexpr int A_ELEMS = TM * BK;                   // 8 KiB
    static constexpr int B_ELEMS = BK * TN;                   // 16 KiB
    static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
    static constexpr int A_SHARE = A_ELEMS * 2 / 1024 / NW;   // 1 KiB DMA blocks per wave per slab: 2
    static constexpr int B_SHARE = B_ELEMS * 2 / 1024 / NW;   // 4
};

__device__ __forceinline__ int swz_sk(int k) { return (k & 3) << 2; }

template <bool IDX>
__global__ void __launch_bounds__(64 * SkShape::NW)
k_gemm_sk(const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
          const int32_t *__restrict__ idx, int64_t ldidx, int64_t M, int64_t N, int64_t kk, int64_t gr,
          void *__restrict__ Y, int ydt, int64_t ldy, int tiles_per_group, int m_tiles, int n_tiles)
{
    using S = SkShape;
    constexpr int TM = S::TM, TN = S::TN, BK = S::BK, WN = S::WN, FM = S::FM, KS = S::KS, D = S::D;
    constexpr int AB_OPS = S::A_SHARE + S::B_SHARE;
    constexpr int STEADY = (D - 1) * ((IDX ? 1 : 0) + AB_OPS);
    __shared__ __attribute__((aligned(1024))) uint16_t smem[S::NSTAGE * S::STAGE_ELEMS];
    __shared__ __attribute__((aligned(256))) int32_t iring[S::NW][S::IDX_RING][BK];

    const int total = m_tiles * n_tiles;
    const int per = (total + 7) / 8;
    const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (t >= total) return;   // whole workgroup: no barrier is ever reached
    const int nt = t / m_tiles, mt = t % m_tiles;
    const int64_t g = mt / tiles_per_group;
    const int64_t row0 = g * gr + (int64_t)(mt % tiles_per_group) * TM;
    const int64_t row_end = (g * gr + gr < M) ? g * gr + gr : M;
    const int64_t col0 = (int64_t)nt * TN;
    const int32_t *I = IDX ? idx + g * ldidx : nullptr;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nkt = (int)((kk + BK - 1) / BK);

    // ---- per-lane DMA sources: A blocks [2w, 2w+2) (8 rows x 128 B each),
    // B blocks [4w, 4w+4) (4 rows x 256 B each)
    const uint16_t *a_src[S::A_SHARE];
#pragma unroll
    for (int i = 0; i < S::A_SHARE; ++i) {
        const int r = (wave * S::A_SHARE + i) * 8 + (lane >> 3);
        int64_t row = row0 + r;
        if (row > M - 1) row = M - 1;
        a_src[i] = A + row * lda + (((lane & 7) ^ swz(r)) << 3);
    }
    const uint16_t *b_src[S::B_SHARE];
#pragma unroll
    for (int i = 0; i < S::B_SHARE; ++i) {
        const int k = (wave * S::B_SHARE + i) * 4 + (lane >> 4);
        const int64_t c = col0 + (((lane & 15) ^ swz_sk(k)) << 3);
        b_src[i] = B + ((c < N) ? c : 0);   // columns past N: any valid chunk, never stored
    }
    const uint32_t smem0 = lds_addr(smem);
    const uint32_t iring0 = lds_addr(&iring[wave][0][0]);

    auto issue_idx = [&](int kt) {
        if constexpr (IDX) {
            const int64_t j = (int64_t)(kt < nkt ? kt : 0) * BK + lane;
            dma4(I + j, iring0 + (kt % S::IDX_RING) * BK * 4);
        }
    };
    // B row indices of slab kt (this wave's DMA lanes), from the index ring
    auto load_rows = [&](int kt, int32_t (&kr)[S::B_SHARE]) {
#pragma unroll
        for (int i = 0; i < S::B_SHARE; ++i) {
            const int jr = (wave * S::B_SHARE + i) * 4 + (lane >> 4);
            if constexpr (IDX) kr[i] = iring[wave][kt % S::IDX_RING][jr];
            else kr[i] = kt * BK + jr;
        }
    };
    // this wave's share of slab kt (past the end: the last A slab, B row 0)
    // into ring stage kt % NSTAGE
    auto issue_ab = [&](int kt, const int32_t (&kr)[S::B_SHARE]) {
        const int64_t kbase = (int64_t)kt * BK;
        const int64_t abase = (int64_t)(kt < nkt ? kt : nkt - 1) * BK;
        const uint16_t *brow[S::B_SHARE];
#pragma unroll
        for (int i = 0; i < S::B_SHARE; ++i) {
            const int jr = (wave * S::B_SHARE + i) * 4 + (lane >> 4);
            const int64_t krow = (kbase + jr < kk) ? kr[i] : 0;   // past kk: row 0
            brow[i] = b_src[i] + krow * ldb;
        }
        const uint32_t sa = smem0 + (kt % S::NSTAGE) * S::STAGE_ELEMS * 2;
        const uint32_t sb = sa + S::A_ELEMS * 2;
#pragma unroll
        for (int i = 0; i < S::A_SHARE; ++i) dma16(a_src[i] + abase, sa + (wave * S::A_SHARE + i) * 1024);
#pragma unroll
        for (int i = 0; i < S::B_SHARE; ++i) dma16_nt(brow[i], sb + (wave * S::B_SHARE + i) * 1024);
    };

    floatx16 acc[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[fm][v] = 0.0f;

    // per-lane byte offset of the transposed B reads within a stage's B tile
    const int blk = lane >> 4, li = lane & 15, s_ = li >> 2, q = li & 3;
    int b_off;
    {
        const int nb = wave * WN + (blk & 1) * 16;
        const int c = (nb >> 3) + (q >> 1);
        const int k = (blk >> 1) * 8 + s_;
        b_off = k * TN * 2 + ((c ^ swz_sk(k)) << 4) + (q & 1) * 8;
    }

    // ---- prologue
#pragma unroll
    for (int p = 0; p < D; ++p) issue_idx(p);
    vmwait<0>();
#pragma unroll
    for (int p = 0; p < D; ++p) {
        issue_idx(p + D);
        int32_t kr[S::B_SHARE];
        load_rows(p, kr);
        issue_ab(p, kr);
    }

    // Each step reads the row indices of slab kt+D and every fragment of slab
    // kt from LDS in one batch, issues the DMA of slab kt+D while those reads
    // are in flight, and only then runs the MFMAs: one LDS round trip per slab
    // instead of one per 16-deep k-step.
    for (int kt = 0; kt < nkt; ++kt) {
        vmwait<STEADY>();   // this wave's share of slab kt landed
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // every wave's share of slab kt landed; stage (kt+D) % NSTAGE (slab
        // kt-1) has no reader left
        int32_t kr[S::B_SHARE];
        load_rows(kt + D, kr);
        const uint16_t *sa = smem + (kt % S::NSTAGE) * S::STAGE_ELEMS;
        const char *sb = (const char *)(sa + S::A_ELEMS);
        u32x4 af[KS][FM];
        shortx4 blo[KS], bhi[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = 2 * ks + (lane >> 5);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int r = fm * 32 + (lane & 31);
                af[ks][fm] = *(const u32x4 *)(sa + r * BK + ((c ^ swz(r)) << 3));
            }
            const char *p = sb + b_off + ks * 16 * TN * 2;
            blo[ks] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p));
            bhi[ks] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p + 4 * TN * 2));
        }
        issue_idx(kt + 2 * D);
        issue_ab(kt + D, kr);
        if ((int64_t)(kt + 1) * BK > kk) {   // last slab: clear A columns at or past kk
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int64_t k0 = (int64_t)kt * BK + ks * 16 + 8 * (lane >> 5);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t m = (k0 + 2 * j < kk ? 0x0000ffffu : 0u) | (k0 + 2 * j + 1 < kk ? 0xffff0000u : 0u);
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm) af[ks][fm][j] &= m;
                }
            }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 bfr = __builtin_bit_cast(bf16x8, __builtin_shufflevector(blo[ks], bhi[ks], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                acc[fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[ks][fm]), bfr,
                                                                  acc[fm], 0, 0, 0);
        }
    }
    vmwait<0>();   // the trailing reloads: no DMA may land after the workgroup ends

    if (ydt == 1) {
        // bf16 output: the 64 x 128 tile staged in LDS (the ring is free once
        // every wave has passed the barrier below), written as whole 16-byte
        // row chunks with streaming stores (N % 8 == 0: a chunk never crosses N)
        constexpr int PITCH = TN * 2 + 16;   // bytes per staged row; +16 spreads rows over the banks
        static_assert(TM * PITCH <= S::NSTAGE * S::STAGE_ELEMS * 2, "staged tile fits the ring");
        char *st = (char *)smem;
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = fm * 32 + acc_row(lane, v), c = wave * WN + acc_col(lane);
                *(uint16_t *)(st + r * PITCH + 2 * c) = (uint16_t)f32_to_bf16(acc[fm][v]);
            }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        for (int e = threadIdx.x; e < TM * (TN / 8); e += 64 * S::NW) {
            const int r = e / (TN / 8), ch = e % (TN / 8);
            const int64_t row = row0 + r, cl = col0 + 8 * ch;
            if (row < row_end && cl < N)
                __builtin_nontemporal_store(*(const u32x4 *)(st + r * PITCH + 16 * ch),
                                            (u32x4 *)((uint16_t *)Y + row * ldy + cl));
        }
        return;
    }
    const int64_t col = col0 + wave * WN + acc_col(lane);
    if (col < N) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = row0 + fm * 32 + acc_row(lane, v);
                if (row >= row_end) continue;
                ((float *)Y)[row * ldy + col] = acc[fm][v];
            }
        }
    }
}

}  // namespace rmm
