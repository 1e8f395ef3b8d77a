// rmm_gemm_wb.h -- prefill-shape reduced GEMM with an index list, two
// workgroups per CU, the kept rows of B loaded straight into registers
// (gfx950).  Included by rmm_gemm.hip after rmm_gemm_wt.h (shares its DMA
// helpers and A layout).
//
// Same product as the other GEMM kernels: Y[rows_g, :] = Apanel[rows_g, 0:kk]
// * B[I_g, :], the kept rows of B fetched in place by index ("Reduced Matrix
// Multiplication..." technical summary, Metodologia > Mecanismo Central).  A
// selection group has 128 rows, so a tile is 128 x 256: four waves side by
// side along N, each owning all 128 rows of 64 columns, 8
// v_mfma_f32_32x32x16_bf16 per 16-deep k-step.
//
// Where the operands travel.  The A panel slab is shared by the four waves:
// it goes to LDS by DMA (global_load_lds_dwordx4) and every wave reads its
// fragments with ds_read_b128.  Each B element, by contrast, is used by one
// wave only, so B skips LDS: lane l (half h = l / 32, m = l % 32) loads with
// 4-byte buffer loads the column pair (2m, 2m+1) of the wave's 64 columns
// from the 8 kept rows k = 8h .. 8h+7 of each k-step, and two v_perm_b32 per
// row pair form the MFMA B fragments of the even and of the odd columns (an
// MFMA B fragment is 8 consecutive k of one column in a lane).  The output
// columns of fragment 0 are then the wave's even columns and those of
// fragment 1 its odd ones, which the epilogue undoes.  Every output element
// sees the same MFMA sequence as with a transposing LDS read of B, so the
// results are bit-identical to the other prefill kernels.  Against the DMA
// pipeline of k_gemm_wt (B rows through LDS, two rows per DMA block, their
// addresses formed per row) the kept-row path costs a ring read and 8 offset
// mads per k-step in each lane and no LDS traffic; measured 3 to 4% faster
// with an index list, 2 to 3% slower on the dense product (rows 0 .. kk-1),
// which therefore keeps k_gemm_wt.
//
// Pipelines.  A: an NS-stage LDS ring of 32-deep slabs, one barrier per slab,
// slab s + NS issued into the stage slab s leaves; the fragments of a
// slab's second k-step are read before its first k-step's MFMAs, and those
// of the next slab's first k-step right after the barrier, before the second
// k-step's MFMAs.  B: the loads of slab s + 1 are issued while slab s is
// multiplied, into two register sets that alternate with the slab (the slab
// loop is unrolled by two, so each set is a fixed set of registers).  The
// loads are straight-line code (past the last slab they read row 0), so the
// compiler's own waits for them are exact; the waits for the A DMAs are
// explicit, counted from the fixed issue order.  Kept-row indices arrive in
// 256-entry chunks by DMA into a per-wave LDS ring.
//
// Offsets.  A kept row's byte offset row * ldb * 2 + column is formed in 32
// bits (v_mad_u32_u24) from a base in scalar registers.  A kept row past the
// 32-bit range (B of 4 GiB or more) is flagged when its index chunk lands
// (once per 8 slabs, outside the k-steps, which it would crowd out of
// registers): its wrapped offset still lies inside B, and the wave then
// recomputes its 128 x 64 part with 64-bit addresses, A fragments read from
// global memory.
#pragma once
#include "rmm_gemm_wt.h"

namespace rmm {

template <int V>
struct IntTag {
    static constexpr int value = V;
};

template <int NS_>
struct WbShape {
    static constexpr int TM = 128, TN = 256, BK = 32, NS = NS_, NW = 4;
    static constexpr int WN = 64, FM = 4, KS = 2;
    static constexpr int DS = 1;                       // slabs of B loaded ahead
    static constexpr int CA = BK / 8;                  // 16-byte chunks per A row
    static constexpr int A_BYTES = TM * BK * 2;        // one A stage
    static constexpr int A_DMA = A_BYTES / 1024 / NW;  // 1 KiB DMA blocks per wave per slab
    static constexpr int A_ROWS = 1024 / (BK * 2);     // A rows per DMA block
    static constexpr int ICH = 256 / BK;               // slabs per index chunk
    static constexpr int BLOADS = KS * 8;              // B loads per lane per slab
    static_assert(DS + NS <= ICH, "an index chunk is issued before the A DMAs that must land before its rows are read");
    static_assert(A_DMA == 2, "the wait counts assume two A blocks per wave per slab");
};

// Vector-memory operations this wave has issued after the A DMAs of slab
// j + 1 when it waits for them at the end of slab j (j = -1: the prologue's
// wait for slab 0).  Index chunks are not counted: a count below the true one
// only waits longer.
template <int NS>
__device__ __forceinline__ int wb_ops_after(int j, int nkt)
{
    using S = WbShape<NS>;
    const int s = j + 1;
    const int ib = s - NS;                       // the boundary that issued A(s); < 0: the prologue
    const int a_hi = min(j - 1 + NS, nkt - 1);   // the last slab whose A has been issued
    int n = S::A_DMA * max(0, a_hi - s);
    int first = ib + 1;                          // the first slab that issued B loads after A(s)
    if (ib < 0) {
        n += S::BLOADS * S::DS;                  // the prologue's B loads
        first = 0;
    }
    return n + S::BLOADS * max(0, j - first + 1);
}

// s_waitcnt vmcnt with the largest immediate not above n
__device__ __forceinline__ void vmwait_le(int n)
{
    if (n >= 52) vmwait<52>();
    else if (n >= 48) vmwait<48>();
    else if (n >= 36) vmwait<36>();
    else if (n >= 32) vmwait<32>();
    else if (n >= 20) vmwait<20>();
    else if (n >= 16) vmwait<16>();
    else if (n >= 4) vmwait<4>();
    else vmwait<0>();
}

// row_lim: the largest row whose 32-bit byte offset holds (row * ldb * 2 + 2N
// < 2^32, row < 2^24); the launcher requires ldb * 2 < 2^24
template <int NS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_gemm_wb(const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
          const int32_t *__restrict__ idx, int64_t ldidx, int64_t M, int64_t N, int64_t kk, int64_t gr,
          uint16_t *__restrict__ Y, int64_t ldy, int tiles_per_group, int m_tiles, int n_tiles, uint32_t row_lim)
{
    using S = WbShape<NS>;
    constexpr int TM = S::TM, BK = S::BK, FM = S::FM, KS = S::KS, DS = S::DS;
    __shared__ __attribute__((aligned(1024))) char smem[NS * S::A_BYTES];
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
    const int64_t col0 = (int64_t)nt * S::TN;
    const int32_t *I = idx + g * ldidx;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nkt = (int)((kk + BK - 1) / BK);
    const int hh = lane >> 5, mm = lane & 31;

    // A DMA sources: byte offsets from the slab's column base (the launcher
    // guarantees M * lda * 2 < 2^32); rows past M read row M-1, never stored
    uint32_t a_voff[S::A_DMA];
#pragma unroll
    for (int i = 0; i < S::A_DMA; ++i) {
        const int r = (wave * S::A_DMA + i) * S::A_ROWS + lane / S::CA;
        int64_t row = row0 + r;
        if (row > M - 1) row = M - 1;
        a_voff[i] = (uint32_t)(row * lda * 2) + (uint32_t)(((lane % S::CA) ^ swz_wa<BK>(r)) << 4);
    }
    // this lane's column pair of B (N % 8 == 0: a pair never straddles N;
    // pairs past N read columns 0 and 1 and are never stored)
    int64_t cpair = col0 + wave * S::WN + 2 * mm;
    if (cpair >= N) cpair = 0;
    const uint32_t cb = (uint32_t)(cpair * 2);
    const uint32_t ldb2 = (uint32_t)(ldb * 2);
    const __amdgpu_buffer_rsrc_t brsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)B, (short)0, (int)0xffffffff, 0x00020000);
    const uint32_t smem0 = lds_addr(smem);
    const uint32_t iring0 = lds_addr(&iring[wave][0][0]);

    // index chunk c (slabs ICH c .. ICH c + ICH - 1): one 16-byte DMA per lane
    // into slot c & 1 of this wave's ring; lanes past the index row re-read
    // its last four entries (ldidx % 4 == 0), which are never used
    auto issue_idx_chunk = [&](int c) {
        int64_t off = (int64_t)c * 256 + 4 * lane;
        if (off > ldidx - 4) off = ldidx - 4;
        dma16(I + off, iring0 + (c & 1) * 1024);
    };
    auto issue_a = [&](int s) {
        const uint32_t sa = smem0 + (s % NS) * S::A_BYTES;
        const uint16_t *abase = A + (int64_t)s * BK;
#pragma unroll
        for (int i = 0; i < S::A_DMA; ++i) dma16s(abase, a_voff[i], sa + (wave * S::A_DMA + i) * 1024);
    };
    // B of k-step ks of slab s: the lane's column pair in the kept rows
    // k = 8 hh .. 8 hh + 7 of the step; rows at or past kk read row 0
    // (finite: their A columns are zero)
    auto issue_b = [&](int s, int ks, uint32_t (&dst)[8], bool tail) {
        const int kp0 = s * BK + ks * 16 + 8 * hh;
        const int32_t *rp = &iring[wave][(s / S::ICH) & 1][(s % S::ICH) * BK + ks * 16 + 8 * hh];
        const int4 r0 = *(const int4 *)rp, r1 = *(const int4 *)(rp + 4);
        uint32_t rows[8] = {(uint32_t)r0.x, (uint32_t)r0.y, (uint32_t)r0.z, (uint32_t)r0.w,
                            (uint32_t)r1.x, (uint32_t)r1.y, (uint32_t)r1.z, (uint32_t)r1.w};
        if (tail) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) rows[jj] = (kp0 + jj < kk) ? rows[jj] : 0u;
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            dst[jj] = __builtin_amdgcn_raw_buffer_load_b32(brsrc, (int)(__umul24(rows[jj], ldb2) + cb), 0, 0);
    };
    // whether index chunk c (landed) holds a kept row past row_lim; only its
    // entries below kk count.  Checked once per chunk, outside the k-steps.
    uint64_t far = 0;
    auto check_chunk = [&](int c) {
        const int4 v = *(const int4 *)&iring[wave][c & 1][4 * lane];
        const int64_t p = (int64_t)c * 256 + 4 * lane;
        uint32_t mx = p < kk ? (uint32_t)v.x : 0u;
        mx = max(mx, p + 1 < kk ? (uint32_t)v.y : 0u);
        mx = max(mx, p + 2 < kk ? (uint32_t)v.z : 0u);
        mx = max(mx, p + 3 < kk ? (uint32_t)v.w : 0u);
        far |= __ballot(mx > row_lim);
    };
    // MFMA B fragments of the even and the odd columns from 8 rows of pairs
    auto form_b = [&](const uint32_t (&d)[8], bf16x8 &even, bf16x8 &odd) {
        u32x4 e, o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            e[q] = __builtin_amdgcn_perm(d[2 * q + 1], d[2 * q], 0x05040100u);   // low halves: k = 2q, 2q+1
            o[q] = __builtin_amdgcn_perm(d[2 * q + 1], d[2 * q], 0x07060302u);   // high halves
        }
        even = __builtin_bit_cast(bf16x8, e);
        odd = __builtin_bit_cast(bf16x8, o);
    };

    int a_off[FM][KS];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int r = fm * 32 + (lane & 31), c = 2 * ks + (lane >> 5);
            a_off[fm][ks] = r * BK * 2 + ((c ^ swz_wa<BK>(r)) << 4);
        }

    floatx16 acc[FM][2];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.0f;

    // the last slab may be partial: clear its A columns >= kk (every wave
    // clears its own rows' chunks after the slab has landed, before the
    // barrier that publishes it)
    auto clear_tail = [&](int s) {
        if ((int64_t)(s + 1) * BK <= kk) return;
        char *st = smem + (s % NS) * S::A_BYTES;
        for (int e = lane; e < (TM / 4) * BK; e += 64) {
            const int r = wave * (TM / 4) + e / BK, col = e % BK;
            const int c = col >> 3, pos = ((c ^ swz_wa<BK>(r)) << 3) + (col & 7);
            if ((int64_t)s * BK + col >= kk) ((uint16_t *)st)[r * BK + pos] = 0;
        }
    };

    uint32_t bq[2][KS][8];          // B of the slab being multiplied and of the next, set = slab % 2
    bf16x8 afa[FM], afb[FM];        // A fragments of a slab's first and second k-step
    auto read_a = [&](int s, int ks, bf16x8 (&af)[FM]) {
        const char *st = smem + (s % NS) * S::A_BYTES;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) af[fm] = *(const bf16x8 *)(st + a_off[fm][ks]);
    };
    auto mfmas = [&](const bf16x8 (&af)[FM], const bf16x8 &be, const bf16x8 &bo) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            acc[fm][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], be, acc[fm][0], 0, 0, 0);
            acc[fm][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bo, acc[fm][1], 0, 0, 0);
        }
    };
    // slab j (afa holds its first k-step's A fragments on entry)
    auto slab_body = [&](int j, auto ctag) {
        constexpr int C = decltype(ctag)::value;
        constexpr int CN = (C + DS) % 2;
        const bool tail = (int64_t)(j + DS + 1) * BK > kk;   // slab j + DS partial or past the end
        bf16x8 be, bo;
        issue_b(j + DS, 0, bq[CN][0], tail);
        read_a(j, 1, afb);
        form_b(bq[C][0], be, bo);
        mfmas(afa, be, bo);
        issue_b(j + DS, 1, bq[CN][1], tail);
        form_b(bq[C][1], be, bo);
        if (j + 1 < nkt) {
            // boundary j: slab j+1 landed for this wave; every wave is done
            // reading slab j and has slab j+1
            vmwait_le(wb_ops_after<NS>(j, nkt));
            clear_tail(j + 1);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            // chunk c is read from slab ICH c - DS on and issued at boundary
            // ICH (c - 1), before A(ICH (c - 1) + NS), which lands first
            if (j % S::ICH == 0 && (j / S::ICH + 1) * S::ICH < nkt) issue_idx_chunk(j / S::ICH + 1);
            if ((j + 1 + DS) % S::ICH == 0 && j + 1 + DS < nkt) check_chunk((j + 1 + DS) / S::ICH);
            if (j + NS < nkt) issue_a(j + NS);
            read_a(j + 1, 0, afa);
        }
        mfmas(afb, be, bo);
    };

    // ---- prologue: index chunk 0, A of slabs 0 .. NS-1, B of slab 0
    issue_idx_chunk(0);
    vmwait<0>();
    check_chunk(0);
#pragma unroll
    for (int p = 0; p < NS; ++p)
        if (p < nkt) issue_a(p);
    issue_b(0, 0, bq[0][0], (int64_t)BK > kk);
    issue_b(0, 1, bq[0][1], (int64_t)BK > kk);
    vmwait_le(wb_ops_after<NS>(-1, nkt));
    clear_tail(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    read_a(0, 0, afa);

    int j = 0;
    for (; j + 2 <= nkt; j += 2) {
        slab_body(j, IntTag<0>{});
        slab_body(j + 1, IntTag<1>{});
    }
    if (j < nkt) slab_body(j, IntTag<0>{});
    vmwait<0>();

    // ---- a kept B row past the 32-bit offsets (B of 4 GiB or more): this
    // wave recomputes its 128 x 64 part with 64-bit addresses, A fragments
    // from global memory (columns at or past kk as zero)
    if (__builtin_expect(far != 0, 0)) {
        // per-lane values recomputed here from the lane id (none of them stays
        // live across the main loop); cb, the column pair's byte offset, is
        const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        const int h2 = ln >> 5, m2 = ln & 31;
        const char *Bb = (const char *)B + cb;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < 2; ++fn)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.0f;
        for (int step = 0; step < KS * nkt; ++step) {
            const int64_t k0 = 16 * (int64_t)step + 8 * h2;
            uint32_t d[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int64_t k = k0 + jj;
                const int64_t row = k < kk ? (int64_t)I[k] : 0;
                d[jj] = *(const uint32_t *)(Bb + row * ldb * 2);
            }
            bf16x8 be, bo;
            form_b(d, be, bo);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                int64_t row = row0 + fm * 32 + m2;
                if (row > M - 1) row = M - 1;
                u32x4 a = *(const u32x4 *)(A + row * lda + k0);   // k0 + 8 <= lda (lda >= slab end)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (k0 + 2 * q >= kk) a[q] = 0u;
                    else if (k0 + 2 * q + 1 >= kk) a[q] &= 0xffffu;
                }
                const bf16x8 af = __builtin_bit_cast(bf16x8, a);
                acc[fm][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, be, acc[fm][0], 0, 0, 0);
                acc[fm][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bo, acc[fm][1], 0, 0, 0);
            }
        }
    }

    // ---- bf16 output (the only output type of this kernel; the launcher
    // sends binary32 outputs to k_gemm_dl), staged in LDS 32 rows at a time
    // (the ring is free once every wave has passed the barrier), the even and
    // odd columns of a lane packed into one 4-byte write, then written as
    // whole 16-byte row chunks (N % 8 == 0, so a chunk never crosses N)
    constexpr int PITCH = S::TN * 2 + 16;
    static_assert(32 * PITCH <= NS * S::A_BYTES, "a quarter tile fits the ring");
    char *st = smem;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = acc_row(lane, v), c = wave * S::WN + 2 * acc_col(lane);
            *(uint32_t *)(st + r * PITCH + 2 * c) = f32_to_bf16(acc[fm][0][v]) | (f32_to_bf16(acc[fm][1][v]) << 16);
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        for (int e = threadIdx.x; e < 32 * (S::TN / 8); e += 256) {
            const int r = e / (S::TN / 8), ch = e % (S::TN / 8);
            const int64_t row = row0 + 32 * fm + r, col = col0 + 8 * ch;
            if (row < row_end && col < N)   // streaming stores: Y is not read back by this launch
                __builtin_nontemporal_store(*(const u32x4 *)(st + r * PITCH + 16 * ch),
                                            (u32x4 *)(Y + row * ldy + col));
        }
    }
}

}  // namespace rmm
