// rmm_gemm_wt.h -- prefill-shape reduced GEMM, two workgroups per CU (gfx950).
// Included by rmm_gemm.hip after rmm_gemm_dl.h (shares its DMA helpers).
//
// Same product as the other GEMM kernels: Y[rows_g, :] = Apanel[rows_g, 0:kk]
// * B[I_g, :], the kept rows of B fetched in place by index.  A selection
// group has 128 rows, so a tile is 128 x 256.  Four waves sit side by side
// along N, each owning all 128 rows of 64 columns: per 16-deep k-step a wave
// reads 4 A fragments (ds_read_b128) and 2 B fragments (two ds_read_b64_tr_b16
// each) and issues 8 v_mfma_f32_32x32x16_bf16, so every B element is read from
// LDS once per workgroup (the eight-wave k_gemm_dl reads it twice).
//
// One workgroup is 4 waves with a 3-stage ring of 32-deep slabs (78 KiB of
// LDS) and at most 256 registers per lane, so two workgroups share a CU and
// each SIMD runs one wave of each.  A workgroup waits at its one barrier per
// slab whenever its waves drift apart (measured: a third of the loop with one
// workgroup per CU); with two, the other workgroup's MFMAs fill that time.
// The launcher takes this kernel when there are at least two tiles per CU
// (the MLP down-projection: 32 groups x 16 strips) for the dense product, and
// with an index list only when B's row stride is too large for k_gemm_wb's
// 24-bit offset multiply (k_gemm_wb, B straight into registers, is faster
// with an index list and slower dense); k_gemm_dl with fewer tiles.
//
// The loop is software-pipelined: fragments of k-step s+1 are read into a
// second register set before the MFMAs of step s are issued.  The slab
// boundary (DMA wait and barrier) sits inside the last k-step of a slab, after
// that step's fragments have landed: every wave is then done reading the
// slab, its ring stage is refilled at once, and the next slab's first
// fragments are in flight before the last MFMAs of this slab are issued.  The
// last slab is peeled off so the boundary is unconditional (the compiler's
// waits before the last k-step's MFMAs then cover only that step's own reads).
//
// Pipeline (NS ring stages of BK-deep slabs; IDX(s) = DMA of the kept row
// indices of slabs s .. s+ICH-1 into a per-wave LDS ring, issued only where s
// is a multiple of ICH; AB(s) = the DMA loads of slab s's A and B tiles):
//   prologue   IDX(0 .. NS-1), wait; then IDX(p + NS), AB(p) for p < NS
//   slab j     read the ring for AB(j+NS)'s rows (their index chunk landed
//              with AB(j)), then the k-steps of slab j
//   boundary j wait for AB(j+1); barrier; the first fragments of slab j+1;
//              IDX(j + 2NS), AB(j + NS) into the stage slab j left
// AB(s) is issued NS-1 slabs before it is used.  While every AB(j+2 ..
// j+NS-1) has been issued, at least (NS-2) AB groups are newer than AB(j+1)
// (an index chunk among them only makes the wait stricter), so one constant
// wait count holds; near the end (nothing past the last slab is loaded) the
// wait is for everything.
//
// Layouts (16-byte chunks, XOR-swizzled so every access pattern is free of
// bank conflicts):
//   A stage: TM rows of BK bf16, chunk c of row r at slot c ^ swz_wa(r)
//   B stage: BK rows of TN bf16, chunk c of row k at slot c ^ swz_bt(k)
#pragma once
#include "rmm_gemm_dl.h"

namespace rmm {

// DMA with a wave-uniform 64-bit base and a 32-bit per-lane byte offset: every
// lane copies 16 bytes from base + voff to LDS[m0 + 16*lane]
__device__ __forceinline__ void dma16s(const void *base, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}

template <int BK>
__device__ __forceinline__ int swz_wa(int r)
{
    if constexpr (BK == 32) return (r >> 2) & 3;   // 64-byte rows: 4 rows per 256-byte bank line
    else return (r ^ (r >> 3)) & 7;                 // 128-byte rows
}

template <int TN_, int BK_, int NS_>
struct WtShape {
    static constexpr int TM = 128, TN = TN_, BK = BK_, NS = NS_, NW = 4;
    static constexpr int WN = TN / NW, FM = TM / 32, FN = WN / 32, KS = BK / 16;
    static constexpr int CA = BK / 8;                       // 16-byte chunks per A row
    static constexpr int CB = TN / 8;                       // 16-byte chunks per B row
    static constexpr int A_BYTES = TM * BK * 2, B_BYTES = BK * TN * 2, STAGE = A_BYTES + B_BYTES;
    static constexpr int A_DMA = A_BYTES / 1024 / NW;       // 1 KiB DMA blocks per wave per slab
    static constexpr int B_DMA = B_BYTES / 1024 / NW;
    static constexpr int A_ROWS = 1024 / (BK * 2);          // A rows per DMA block
    static constexpr int B_ROWS = 1024 / (TN * 2);          // B rows per DMA block
    static constexpr int ICH = 256 / BK;                    // slabs per index chunk (one 16-byte DMA per lane)
    static_assert(KS % 2 == 0, "two register sets alternate over an even number of k-steps");
    static_assert(2 * NS <= ICH, "an index chunk is issued before its first slab's rows are read");
    static_assert(B_ROWS == 2 && A_DMA >= 1 && B_DMA >= 1, "DMA blocks divide the tiles, two B rows each");
    
};

template <int TN, int BK, int NS, bool IDX>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_gemm_wt(const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
          const int32_t *__restrict__ idx, int64_t ldidx, int64_t M, int64_t N, int64_t kk, int64_t gr,
          void *__restrict__ Y, int ydt, int64_t ldy, int tiles_per_group, int m_tiles, int n_tiles)
{
    using S = WtShape<TN, BK, NS>;
    constexpr int TM = S::TM, WN = S::WN, FM = S::FM, FN = S::FN, KS = S::KS;
    constexpr int AB_OPS = S::A_DMA + S::B_DMA;
    constexpr int STEADY = (NS - 2) * AB_OPS;   // index chunks not counted: waiting for more is safe
    __shared__ __attribute__((aligned(1024))) char smem[NS * S::STAGE];
    __shared__ __attribute__((aligned(1024))) int32_t iring[S::NW][2][256];

    // ---- tile (XCD-aware: workgroup w runs on XCD w % 8, which takes a
    // contiguous range of tiles, N strip major, so an XCD's L2 holds one strip
    // of B for every group)
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

    // ---- per-lane DMA sources.  A: byte offsets from the slab's column base
    // (the launcher guarantees M * lda * 2 < 2^32); B: two rows per DMA block,
    // 64-bit per-lane column sources
    uint32_t a_voff[S::A_DMA];
#pragma unroll
    for (int i = 0; i < S::A_DMA; ++i) {
        const int r = (wave * S::A_DMA + i) * S::A_ROWS + lane / S::CA;
        int64_t row = row0 + r;
        if (row > M - 1) row = M - 1;   // rows past M: any valid row, never stored
        a_voff[i] = (uint32_t)(row * lda * 2) + (uint32_t)(((lane % S::CA) ^ swz_wa<BK>(r)) << 4);
    }
    const uint16_t *b_src[S::B_DMA];
#pragma unroll
    for (int i = 0; i < S::B_DMA; ++i) {
        const int k = (wave * S::B_DMA + i) * S::B_ROWS + lane / S::CB;
        const int64_t c = col0 + (((lane % S::CB) ^ swz_bt(k)) << 3);
        b_src[i] = B + ((c < N) ? c : 0);   // columns past N: any valid chunk, never stored
    }
    const uint32_t smem0 = lds_addr(smem);
    const uint32_t iring0 = lds_addr(&iring[wave][0][0]);

    // The kept-row indices of ICH slabs (256 entries) arrive by one 16-byte
    // DMA per lane into a two-chunk ring per wave.  (One 4-byte DMA per slab
    // cost as much as a 1 KiB one: this loop is bound by the DMA instructions a
    // CU issues, about 34 cycles each, and it was the seventh of seven per
    // slab.)  Chunk c is issued with the index slab s = ICH c, i.e. in the
    // same step as, and before, AB(s - NS), which every wave has waited for
    // before it reads row indices of slab s; chunk c + 2 reuses the slot after
    // chunk c's last read.  Lanes past the index row re-read its last four
    // entries (ldidx % 4 == 0): only entries below kk are ever used.
    auto issue_idx = [&](int s) {
        if constexpr (IDX) {
            if (s % S::ICH == 0 && s < nkt) {
                const int c = s / S::ICH;
                int64_t off = (int64_t)c * 256 + 4 * lane;
                if (off > ldidx - 4) off = ldidx - 4;
                dma16(I + off, iring0 + (c & 1) * 1024);
            }
        }
    };
    // sources of slab s's B rows for this wave's DMA blocks (rows past kk read
    // row 0 of B, finite, multiplied by the zero A columns there).  In two
    // halves: the index-ring reads (issued a k-step early, so their latency
    // hides under MFMAs), then the addresses
    int32_t kr[S::B_DMA];
    auto load_rows = [&](int s) {
        const int64_t kbase = (int64_t)s * BK;
#pragma unroll
        for (int i = 0; i < S::B_DMA; ++i) {
            const int jr = (wave * S::B_DMA + i) * S::B_ROWS + lane / S::CB;
            if constexpr (IDX) kr[i] = iring[wave][(s / S::ICH) & 1][(s % S::ICH) * BK + jr];
            else kr[i] = (int32_t)(kbase + jr);
        }
    };
    const uint16_t *b_row[S::B_DMA];
    auto prep_b = [&](int s) {
        const int64_t kbase = (int64_t)s * BK;
#pragma unroll
        for (int i = 0; i < S::B_DMA; ++i) {
            const int jr = (wave * S::B_DMA + i) * S::B_ROWS + lane / S::CB;
            const int64_t krow = (kbase + jr < kk) ? kr[i] : 0;
            b_row[i] = b_src[i] + krow * ldb;
        }
    };
    auto issue_ab = [&](int s) {
        const uint32_t sa = smem0 + (s % NS) * S::STAGE;
        const uint32_t sb = sa + S::A_BYTES;
        const uint16_t *abase = A + (int64_t)s * BK;
#pragma unroll
        for (int i = 0; i < S::A_DMA; ++i) dma16s(abase, a_voff[i], sa + (wave * S::A_DMA + i) * 1024);
#pragma unroll
        for (int i = 0; i < S::B_DMA; ++i) dma16(b_row[i], sb + (wave * S::B_DMA + i) * 1024);
    };

    // per-lane byte offsets of the fragment reads within a stage
    int a_off[FM][KS];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int r = fm * 32 + (lane & 31), c = 2 * ks + (lane >> 5);
            a_off[fm][ks] = r * BK * 2 + ((c ^ swz_wa<BK>(r)) << 4);
        }
    const int blk = lane >> 4, li = lane & 15, s_ = li >> 2, q = li & 3;
    int b_off[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int nb = wave * WN + fn * 32 + (blk & 1) * 16;
        const int c = (nb >> 3) + (q >> 1);
        const int k = (blk >> 1) * 8 + s_;
        b_off[fn] = S::A_BYTES + k * TN * 2 + ((c ^ swz_bt(k)) << 4) + (q & 1) * 8;
    }

    floatx16 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.0f;

    bf16x8 af[2][FM], bfr[2][FN];
    // fragments of k-step ks of slab s into register set `set`
    auto read_frags = [&](int s, int ks, int set) {
        const char *st = smem + (s % NS) * S::STAGE;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) af[set][fm] = *(const bf16x8 *)(st + a_off[fm][ks]);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const char *p = st + b_off[fn] + ks * 16 * TN * 2;
            shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p));
            shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p + 4 * TN * 2));
            bfr[set][fn] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    auto mfmas = [&](int set) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[set][fm], bfr[set][fn], acc[fm][fn], 0, 0, 0);
    };
    // the last slab may be partial: clear its A columns >= kk (every wave
    // clears its own rows' chunks after the slab has landed, before the
    // barrier that publishes it)
    auto clear_tail = [&](int s) {
        if ((int64_t)(s + 1) * BK <= kk) return;
        char *st = smem + (s % NS) * S::STAGE;
        for (int e = lane; e < (TM / 4) * BK; e += 64) {
            const int r = wave * (TM / 4) + e / BK, col = e % BK;
            const int c = col >> 3, pos = ((c ^ swz_wa<BK>(r)) << 3) + (col & 7);
            if ((int64_t)s * BK + col >= kk) ((uint16_t *)st)[r * BK + pos] = 0;
        }
    };

    // ---- prologue
#pragma unroll
    for (int p = 0; p < NS; ++p) issue_idx(p);
    vmwait<0>();
#pragma unroll
    for (int p = 0; p < NS; ++p) {
        issue_idx(p + NS);
        if (p < nkt) {
            load_rows(p);
            prep_b(p);
            issue_ab(p);
        }
    }
    // slab 0 in LDS for every wave
    if (nkt >= NS) vmwait<(NS - 1) * AB_OPS>();
    else vmwait<0>();
    clear_tail(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    read_frags(0, 0, 0);

    // slabs followed by another one: the boundary is unconditional, so the
    // compiler's waits before the last k-step's MFMAs cover only that step's
    // own fragments
    for (int j = 0; j + 1 < nkt; ++j) {
        // the kept rows of AB(j+NS): its index chunk landed with AB(j).  Read
        // on every step, also past the end (an in-bounds ring slot whose
        // values are not used): with the reads under a branch, the compiler's
        // merged wait before this slab's second MFMA covered them too, one LDS
        // round trip per slab (1.06 against 0.96 us a slab at kk = K)
        const bool more = j + NS < nkt;
        load_rows(j + NS);
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
            read_frags(j, ks + 1, (ks & 1) ^ 1);
            mfmas(ks & 1);
        }
        // the B row addresses of AB(j+NS) (a 64-bit product per row), formed
        // while those MFMAs run rather than between the wait and the barrier
        // below, where every wave of both workgroups on the CU waits for them
        if (more) prep_b(j + NS);
        // boundary j: slab j+1 landed for this wave
        if (j + NS < nkt + 1) vmwait<STEADY>();
        else vmwait<0>();
        clear_tail(j + 1);
        // every wave is done reading slab j and has slab j+1
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        read_frags(j + 1, 0, 0);   // KS is even: k-step KS-1 used set 1
        if (more) {
            issue_idx(j + 2 * NS);
            issue_ab(j + NS);
        }
        mfmas(1);
    }
    // the last slab
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) read_frags(nkt - 1, ks + 1, (ks & 1) ^ 1);
        mfmas(ks & 1);
    }
    vmwait<0>();   // trailing index loads

    // bf16 output (the only output type of this kernel; the launcher sends
    // binary32 outputs to k_gemm_dl), staged in LDS in two halves of 64 rows
    // (the ring is free once every wave has passed the barrier), written as
    // whole 16-byte row chunks (N % 8 == 0, so a chunk never crosses N)
    (void)ydt;
    constexpr int PITCH = TN * 2 + 16;
    static_assert(64 * PITCH <= NS * S::STAGE, "half a tile fits the ring");
    char *st = smem;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int fm = 2 * h; fm < 2 * h + 2; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = (fm - 2 * h) * 32 + acc_row(lane, v), c = wave * WN + fn * 32 + acc_col(lane);
                    *(uint16_t *)(st + r * PITCH + 2 * c) = (uint16_t)f32_to_bf16(acc[fm][fn][v]);
                }
                // one accumulator block at a time: converting all of them at
                // once would need more registers than the wave has
                __builtin_amdgcn_sched_barrier(0);
            }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        for (int e = threadIdx.x; e < 64 * S::CB; e += 256) {
            const int r = e / S::CB, ch = e % S::CB;
            const int64_t row = row0 + 64 * h + r, col = col0 + 8 * ch;
            if (row < row_end && col < N)   // streaming stores: Y is not read back by this launch
                __builtin_nontemporal_store(*(const u32x4 *)(st + r * PITCH + 16 * ch),
                                            (u32x4 *)((uint16_t *)Y + row * ldy + col));
        }
    }
}

}  // namespace rmm
