// rmm_gemm_dl.h -- prefill-shape reduced GEMM with a global->LDS DMA pipeline
// (gfx950).  Included by rmm_gemm.hip.
//
// Same product as k_gemm (Y[rows_g, :] = Apanel[rows_g, 0:kk] * B[I_g, :]),
// organised the way gfx950 wants it:
//   * operands go from global memory straight into LDS with 16-byte
//     global_load_lds_dwordx4 DMA loads (lane l of a wave writes bytes
//     [16l, 16l+16) of a 1 KiB LDS block): no VGPR staging and no VALU work on
//     the load path, so a 3-deep ring of 64-deep slabs is in flight;
//   * the A tile is kept k-contiguous (an MFMA A fragment is one
//     ds_read_b128); the B tile stays n-contiguous as in memory and the MFMA
//     B fragments come from ds_read_b64_tr_b16, whose 16-lane blocks return a
//     4(k) x 16(n) sub-block transposed (lane i of the block gets column i,
//     four consecutive k);
//   * the kept-row index list is DMA-loaded into a small per-wave LDS ring one
//     slab ahead of the B loads that use it, so dropped rows of B are never
//     fetched and no load result ever waits in a register.
// The DMA loads are issued from inline assembly (they have no register
// outputs) and every wait is an explicit s_waitcnt whose count follows from
// the fixed issue order, so the compiler's conservative LDS-DMA alias waits
// never serialise the ring.
// Bank-conflict-free layouts come from choosing, per lane, which 16-byte
// global chunk it fetches: A row r stores chunk c at slot c ^ swz(r); B row k
// stores chunk c at slot c ^ swz_bt(k) (see below).
//
// Tile 128 x 256 x 64, v_mfma_f32_32x32x16_bf16.
#pragma once
#include "rmm_tile.h"

namespace rmm {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// NW waves arranged WMS (along M) x NW/WMS (along N).  Every wave reads the A
// rows and B columns of its own sub-tile from LDS, so WMS = 1 reads each B
// element (the half-rate transposed reads) once per slab and A NW times.
template <int NW, int WMS>
struct DlShape {
    static constexpr int TM = 128, TN = 256, BK = 64;
    static constexpr int WAVES_M = WMS, WAVES_N = NW / WMS;
    static constexpr int WM = TM / WAVES_M, WN = TN / WAVES_N, FM = WM / 32, FN = WN / 32;
    static constexpr int NSTAGE = 3;
    static constexpr int A_ELEMS = TM * BK;          // 16 KiB
    static constexpr int B_ELEMS = BK * TN;          // 32 KiB
    static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
    static constexpr int A_LOADS = A_ELEMS * 2 / 1024 / NW;  // 1 KiB DMA blocks per wave per slab
    static constexpr int B_LOADS = B_ELEMS * 2 / 1024 / NW;
    static constexpr int IDX_RING = 4;                       // slabs of indices per wave
};

// B row k stores 16-byte chunk c at slot c ^ swz_bt(k).  The XOR values
// {0, 6, 10, 12} make the 4 rows x 2 chunks one 16-lane block of a transposed
// read touches distinct modulo 8 slots (32 banks), and the 4 rows x 4 chunks
// of two blocks distinct modulo 16 slots (64 banks).
__device__ __forceinline__ int swz_bt(int k) { return (0xcA60 >> (4 * (k & 3))) & 0xf; }

template <int N>
__device__ __forceinline__ void vmwait() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// DMA: every lane copies 16 (or 4) bytes from its global address to
// LDS[m0 + 16*lane] (or 4*lane).  m0 is the wave-uniform LDS base.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
// the same with the non-temporal policy, for operand rows a launch reads exactly once
// (the decode GEMMs' kept B rows): they stream past the caches instead of evicting
// what is reused
__device__ __forceinline__ void dma16_nt(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

template <int NW, int WMS, bool IDX>
__global__ void __launch_bounds__(64 * NW)
k_gemm_dl(const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
          const int32_t *__restrict__ idx, int64_t ldidx, int64_t M, int64_t N, int64_t kk, int64_t gr,
          void *__restrict__ Y, int ydt, int64_t ldy, int tiles_per_group, int m_tiles, int n_tiles)
{
    using S = DlShape<NW, WMS>;
    constexpr int TM = S::TM, TN = S::TN, BK = S::BK, WM = S::WM, WN = S::WN, FM = S::FM, FN = S::FN;
    constexpr int AB = S::A_LOADS + S::B_LOADS;   // DMA loads per wave per slab
    constexpr int NT = 64 * NW;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[S::NSTAGE * S::STAGE_ELEMS];
    __shared__ __attribute__((aligned(256))) int32_t iring[NW][S::IDX_RING][BK];

    const int total = m_tiles * n_tiles;
    const int per = (total + 7) / 8;
    const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (t >= total) return;
    const int nt = t / m_tiles, mt = t % m_tiles;
    const int64_t g = mt / tiles_per_group;
    const int64_t row0 = g * gr + (int64_t)(mt % tiles_per_group) * TM;
    const int64_t row_end = (g * gr + gr < M) ? g * gr + gr : M;
    const int64_t col0 = (int64_t)nt * TN;
    const int32_t *I = IDX ? idx + g * ldidx : nullptr;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / S::WAVES_N, wn = wave % S::WAVES_N;
    const int h = lane >> 5;              // which of the two B rows of a DMA block
    const int nkt = (int)((kk + BK - 1) / BK);

    // ---- per-lane global sources of the DMA loads (slab offsets added per slab)
    const uint16_t *a_src[S::A_LOADS];
#pragma unroll
    for (int i = 0; i < S::A_LOADS; ++i) {
        const int r = (wave * S::A_LOADS + i) * 8 + (lane >> 3);
        int64_t row = row0 + r;
        if (row > M - 1) row = M - 1;
        a_src[i] = A + row * lda + (((lane & 7) ^ swz(r)) << 3);
    }
    const uint16_t *b_src[S::B_LOADS];
#pragma unroll
    for (int i = 0; i < S::B_LOADS; ++i) {
        const int k = (wave * S::B_LOADS + i) * 2 + h;
        int64_t c = col0 + (((lane & 31) ^ swz_bt(k)) << 3);
        b_src[i] = B + ((c < N) ? c : 0);   // columns past N: any valid chunk, never stored
    }
    const uint32_t smem0 = lds_addr(smem);
    const uint32_t iring0 = lds_addr(&iring[wave][0][0]);

    // index entries of slab kt into ring slot kt % 4 (slabs past the end
    // re-read slab 0, always in bounds and never used)
    auto issue_idx = [&](int kt) {
        if constexpr (IDX) {
            const int64_t j = (int64_t)(kt < nkt ? kt : 0) * BK + lane;
            dma4(I + j, iring0 + (kt % S::IDX_RING) * BK * 4);
        }
    };
    // global addresses of slab kt's B rows, read from the index ring into
    // registers (all ring reads before any DMA, so they share one LDS wait)
    const uint16_t *b_row[S::B_LOADS];
    auto prep_b = [&](int kt) {
        const int64_t kbase = (int64_t)kt * BK;
        int32_t kr[S::B_LOADS];
#pragma unroll
        for (int i = 0; i < S::B_LOADS; ++i) {
            const int jr = (wave * S::B_LOADS + i) * 2 + h;  // row of the slab
            if constexpr (IDX) kr[i] = iring[wave][kt % S::IDX_RING][jr];
            else kr[i] = (int32_t)(kbase + jr);
        }
#pragma unroll
        for (int i = 0; i < S::B_LOADS; ++i) {
            const int jr = (wave * S::B_LOADS + i) * 2 + h;
            const int64_t krow = (kbase + jr < kk) ? kr[i] : 0;   // past kk: row 0 (A is zero there)
            b_row[i] = b_src[i] + krow * ldb;
        }
    };
    // the A and B tiles of slab kt into ring stage kt % 3 (B rows from prep_b(kt))
    auto issue_ab = [&](int kt) {
        const int64_t kbase = (int64_t)kt * BK;
        const uint32_t sa = smem0 + (kt % S::NSTAGE) * S::STAGE_ELEMS * 2;
        const uint32_t sb = sa + S::A_ELEMS * 2;
#pragma unroll
        for (int i = 0; i < S::A_LOADS; ++i) dma16(a_src[i] + kbase, sa + (wave * S::A_LOADS + i) * 1024);
#pragma unroll
        for (int i = 0; i < S::B_LOADS; ++i) dma16(b_row[i], sb + (wave * S::B_LOADS + i) * 1024);
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.0f;

    // per-lane byte offsets of the transposed B reads within a stage's B tile
    const int blk = lane >> 4, li = lane & 15, s_ = li >> 2, q = li & 3;
    int b_off[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int nb = wn * WN + fn * 32 + (blk & 1) * 16;
        const int c = (nb >> 3) + (q >> 1);
        const int k = (blk >> 1) * 8 + s_;
        b_off[fn] = k * TN * 2 + ((c ^ swz_bt(k)) << 4) + (q & 1) * 8;
    }

    // ---- prologue.  Iteration j issues IDX(j+4) then AB(j+2), so this wave's
    // loads are always ordered ..., IDX(kt+2), AB(kt), IDX(kt+3), AB(kt+1), ...
    // (IDX only with an index list; AB is A_LOADS + B_LOADS loads, IDX one):
    // when AB(kt) has landed, the index slab AB(kt+2) needs landed before it.
    issue_idx(0);
    issue_idx(1);
    vmwait<0>();
    issue_idx(2);
    prep_b(0);
    issue_ab(0);
    issue_idx(3);
    if (nkt > 1) {
        prep_b(1);
        issue_ab(1);
    }

    for (int kt = 0; kt < nkt; ++kt) {
        // slab kt must be in LDS; IDX(kt+3) and AB(kt+1) may stay in flight
        if constexpr (IDX) {
            if (kt + 1 < nkt) vmwait<AB + 1>(); else vmwait<1>();
        } else {
            if (kt + 1 < nkt) vmwait<AB>(); else vmwait<0>();
        }
        // slab kt landed, so did the index slab kt+2 (issued before it)
        if (kt + 2 < nkt) prep_b(kt + 2);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // every wave's slab kt landed, and stage (kt+2)%3 (slab kt-1) is free;
        // index slot (kt+4)%4 held slab kt's indices, read two iterations ago
        issue_idx(kt + 4);
        if (kt + 2 < nkt) issue_ab(kt + 2);
        uint16_t *sa = smem + (kt % S::NSTAGE) * S::STAGE_ELEMS;
        const char *sb = (const char *)(sa + S::A_ELEMS);
        if ((int64_t)(kt + 1) * BK > kk) {
            // partial last slab: clear A columns >= kk (B rows there are row 0, finite)
            for (int e = threadIdx.x; e < TM * BK; e += NT) {
                const int r = e / BK, col = e % BK;
                const int c = col >> 3, pos = ((c ^ swz(r)) << 3) + (col & 7);
                if ((int64_t)kt * BK + col >= kk) sa[r * BK + pos] = 0;
            }
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int c = 2 * ks + (lane >> 5);
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int r = wm * WM + fm * 32 + (lane & 31);
                af[fm] = *(const bf16x8 *)(sa + r * BK + ((c ^ swz(r)) << 3));
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const char *p = sb + b_off[fn] + ks * 16 * TN * 2;
                shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p));
                shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p + 4 * TN * 2));
                bfr[fn] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
        }
    }
    vmwait<0>();   // the trailing index loads

    if (ydt == 1) {
        // bf16 output: stage the tile in LDS (the ring is free once every wave
        // has passed the barrier below), then write whole 16-byte row chunks
        // (N % 8 == 0, so a chunk never crosses N)
        constexpr int PITCH = TN * 2 + 16;   // bytes per staged row; +16 spreads rows over the banks
        static_assert(TM * PITCH <= S::NSTAGE * S::STAGE_ELEMS * 2, "staged tile fits the ring");
        char *st = (char *)smem;
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = wm * WM + fm * 32 + acc_row(lane, v), c = wn * WN + fn * 32 + acc_col(lane);
                    *(uint16_t *)(st + r * PITCH + 2 * c) = (uint16_t)f32_to_bf16(acc[fm][fn][v]);
                }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        for (int e = threadIdx.x; e < TM * (TN / 8); e += NT) {
            const int r = e / (TN / 8), ch = e % (TN / 8);
            const int64_t row = row0 + r, col = col0 + 8 * ch;
            if (row < row_end && col < N)   // streaming stores: Y is not read back by this launch
                __builtin_nontemporal_store(*(const u32x4 *)(st + r * PITCH + 16 * ch),
                                            (u32x4 *)((uint16_t *)Y + row * ldy + col));
        }
        return;
    }

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

}  // namespace rmm
