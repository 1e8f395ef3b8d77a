// rmm_pv.hip -- P.V reduced along the key (token) dimension on MFMA (gfx950).
//
// "Reduced Matrix Multiplication..." technical summary, Metodologia > Escopo
// de Aplicacao: the reduction also applies to the token dimension of PV.  For
// head h and query block g:
//     O[h, q0:q0+128, :] = sum over kept keys k of P[h, q, k] * V[h, k, :]
// P is stored key-major (Pt[h][k][q] = P[h][q][k]): the 128 probabilities a
// block needs from key k are one contiguous 256-byte segment, and V[h][k][:]
// is another.  Both are fetched in place by kept-key index (no gather pass,
// dropped keys are never read), straight from global memory into LDS by
// 16-byte DMA, through a (D+1)-stage ring with D slabs of 32 or 64 keys in
// flight.
//
// Both operands arrive key-major, i.e. k-major rows of 256 B, and both MFMA
// fragments (A: 32 queries x 16 keys, B: 16 keys x 32 d) come from the
// transposing ds_read_b64_tr_b16: a 16-lane block reads 4 keys x 16
// consecutive queries (or d) and lane i receives column i's four keys.  Rows
// of 256 B are one 64-bank line; chunk c of key row k is stored at slot
// c ^ 4(k mod 4), which puts the 4 rows x 4 chunks one 32-lane read touches
// on 16 distinct slots.
//
// One workgroup per (head, block): a 128 x 128 output tile, 4 waves of 64 x
// 64 (2 x 2 fragments of v_mfma_f32_32x32x16_bf16).  Blocks are dispatched
// last-block first: with a causal mask the late blocks carry the most keys.
// With no index list the kept set is the whole causal prefix (r = 1).
//
// Pipeline (as the decode GEMM): prologue IDX(0..D-1), wait, then IDX(p+D),
// AB(p) for p < D; step i waits for AB(i), barrier, issues IDX(i+2D) and
// AB(i+D) (slabs past the end reload key 0 of the prefix: valid memory whose
// P values are cleared in registers), then runs slab i.  Every step issues the
// same operations, so (D-1) * (1 + AB_OPS) operations are always newer than
// AB(i) when it is waited for.
#include "rmm_tile.h"

namespace rmm {

namespace {

constexpr int kPvD = 3;                 // slabs in flight
constexpr int kPvStages = kPvD + 1;
constexpr int kPvIdxRing = 2 * kPvD;
constexpr int kPvIdxSlot = 64;          // kept-key indices one 4-byte DMA brings (64 lanes)

__device__ __forceinline__ int swz_pv(int k) { return (k & 3) << 2; }

template <int N>
__device__ __forceinline__ void pv_vmwait() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

__device__ __forceinline__ uint32_t pv_lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// every lane copies 16 (or 4) bytes from its global address to LDS[m0 + 16*lane]
// (or 4*lane); m0 is the wave-uniform LDS base
__device__ __forceinline__ void pv_dma16(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
// the same with the non-temporal policy, for P rows: each is read once, and keeping them
// out of the caches leaves room for the V rows that other query blocks of the head reuse
__device__ __forceinline__ void pv_dma16_nt(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void pv_dma4(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// one MFMA operand fragment (32 columns x 16 keys) by two transposing reads
__device__ __forceinline__ bf16x8 tr_frag(const char *p)
{
    const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p));
    const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p + 4 * 256));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace

// BK keys per slab: 64 (128 KiB of ring, one workgroup per CU) or 32 (64 KiB,
// two per CU, so one workgroup's index wait, pipeline fill and epilogue
// overlap the other's streaming).  Measured at H = 32 (same box, identical
// outputs): L = 4096 r = 0.5 75.4 against 83.5 us, r = 1 129 against 131-135;
// L = 16384 r = 0.5 915 against 924-930, r = 1 1740 against 1680 us -- the
// short workgroups gain, the longest lose to the second barrier per 64 keys.
template <bool IDX, int BK>
__global__ void __launch_bounds__(256, 64 / BK)
k_pv_gemm(const uint16_t *__restrict__ Pt, const uint16_t *__restrict__ V, int64_t H, int64_t L,
          int64_t Gq, int64_t qb, int causal, double r, const int32_t *__restrict__ idx, int64_t ldidx,
          void *__restrict__ O, int odt)
{
    constexpr int D = kPvD, FM = 2, FN = 2;
    constexpr int kPvTile = 128 * BK;          // elements of one operand tile (BK key rows)
    constexpr int A_SHARE = BK / 16, B_SHARE = BK / 16;   // 1 KiB DMA blocks per wave per slab (P, V)
    constexpr int AB_OPS = A_SHARE + B_SHARE;
    constexpr int STEADY = (D - 1) * ((IDX ? 1 : 0) + AB_OPS);
    // the bf16 epilogue stages the 128 x 128 output tile (34 KiB) in the ring
    static_assert(kPvStages * 2 * kPvTile * 2 >= 128 * (128 * 2 + 16), "ring too small for the epilogue");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[kPvStages * 2 * kPvTile];
    __shared__ __attribute__((aligned(256))) int32_t iring[4][kPvIdxRing][kPvIdxSlot];

    const int64_t b = blockIdx.x;
    const int64_t g = Gq - 1 - b / H;
    const int64_t h = b % H;
    const int64_t q0 = g * qb;
    const int64_t Kg = causal ? ((qb * (g + 1) < L) ? qb * (g + 1) : L) : L;
    const int64_t kk = IDX ? kk_rule(r, Kg) : Kg;
    const int32_t *I = IDX ? idx + (h * Gq + g) * ldidx : nullptr;
    const int64_t nq = (L - q0 < qb) ? (L - q0) : qb;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int nkt = (int)((kk + BK - 1) / BK);

    // ---- per-lane DMA sources.  Block j (0..15) of an operand tile holds key
    // rows 4j .. 4j+3; lane l fills slot l & 15 of row 4j + (l >> 4) with the
    // chunk that belongs there.  Query chunks past L (a short last block) read
    // chunk 0 instead: valid memory, never stored.
    const uint16_t *p_src[A_SHARE];
    const uint16_t *v_src[B_SHARE];
#pragma unroll
    for (int i = 0; i < A_SHARE; ++i) {
        const int k = (wave * A_SHARE + i) * 4 + (lane >> 4);
        const int c = (lane & 15) ^ swz_pv(k);
        p_src[i] = Pt + h * L * L + q0 + ((8 * c < nq) ? 8 * c : 0);
        v_src[i] = V + h * L * 128 + 8 * c;
    }
    const uint32_t smem0 = pv_lds_addr(smem);
    const uint32_t iring0 = pv_lds_addr(&iring[wave][0][0]);

    // the slab's BK indices (with BK = 32 lanes 32-63 repeat lanes 0-31, so no
    // lane reads past the slab's end of the padded index row)
    auto issue_idx = [&](int kt) {
        if constexpr (IDX) {
            const int64_t j = (int64_t)(kt < nkt ? kt : 0) * BK + (lane & (BK - 1));
            pv_dma4(I + j, iring0 + (kt % kPvIdxRing) * kPvIdxSlot * 4);
        }
    };
    auto issue_ab = [&](int kt) {
        const int64_t kbase = (int64_t)kt * BK;
        int32_t kr[A_SHARE];
#pragma unroll
        for (int i = 0; i < A_SHARE; ++i) {
            const int jr = (wave * A_SHARE + i) * 4 + (lane >> 4);
            if constexpr (IDX) kr[i] = iring[wave][kt % kPvIdxRing][jr];
            else kr[i] = (int32_t)(kbase + jr);
        }
        const uint32_t sp = smem0 + (kt % kPvStages) * 2 * kPvTile * 2;
        const uint32_t sv = sp + kPvTile * 2;
#pragma unroll
        for (int i = 0; i < A_SHARE; ++i) {
            const int jr = (wave * A_SHARE + i) * 4 + (lane >> 4);
            const int64_t key = (kbase + jr < kk) ? kr[i] : 0;   // past kk: key 0, P cleared in registers
            pv_dma16_nt(p_src[i] + key * L, sp + (wave * A_SHARE + i) * 1024);
            pv_dma16(v_src[i] + key * 128, sv + (wave * A_SHARE + i) * 1024);
        }
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.0f;

    // per-lane byte offsets of the transposed reads within a 128-column tile
    const int blk = lane >> 4, li = lane & 15, s_ = li >> 2, q = li & 3;
    int a_off[FM], b_off[FN];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int k = (blk >> 1) * 8 + s_;
        const int ca = ((wm * 64 + f * 32 + (blk & 1) * 16) >> 3) + (q >> 1);
        const int cb = ((wn * 64 + f * 32 + (blk & 1) * 16) >> 3) + (q >> 1);
        a_off[f] = k * 256 + ((ca ^ swz_pv(k)) << 4) + (q & 1) * 8;
        b_off[f] = k * 256 + ((cb ^ swz_pv(k)) << 4) + (q & 1) * 8;
    }

#pragma unroll
    for (int p = 0; p < D; ++p) issue_idx(p);
    pv_vmwait<0>();
#pragma unroll
    for (int p = 0; p < D; ++p) {
        issue_idx(p + D);
        issue_ab(p);
    }

    for (int kt = 0; kt < nkt; ++kt) {
        pv_vmwait<STEADY>();   // this wave's share of slab kt landed
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        issue_idx(kt + 2 * D);
        issue_ab(kt + D);
        const char *sp = (const char *)(smem + (kt % kPvStages) * 2 * kPvTile);
        const char *sv = sp + kPvTile * 2;
        const bool tail = (int64_t)(kt + 1) * BK > kk;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                af[f] = tr_frag(sp + a_off[f] + ks * 16 * 256);
                bfr[f] = tr_frag(sv + b_off[f] + ks * 16 * 256);
            }
            if (tail) {
                const int64_t k0 = (int64_t)kt * BK + ks * 16 + 8 * (lane >> 5);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (k0 + e >= kk)
#pragma unroll
                        for (int f = 0; f < FM; ++f) af[f][e] = (__bf16)0.0f;
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
        }
    }
    pv_vmwait<0>();   // the trailing reloads: no DMA may land after the workgroup ends

    if (odt == 1) {
        // bf16 output: stage the 128 x 128 tile in LDS (the ring is free once
        // every wave has passed the barrier below), then write 16-byte row chunks
        constexpr int PITCH = 128 * 2 + 16;
        char *st = (char *)smem;
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = wm * 64 + fm * 32 + acc_row(lane, v), c = wn * 64 + fn * 32 + acc_col(lane);
                    *(uint16_t *)(st + r * PITCH + 2 * c) = (uint16_t)f32_to_bf16(acc[fm][fn][v]);
                }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        for (int e = threadIdx.x; e < 128 * 16; e += 256) {
            const int r = e >> 4, ch = e & 15;
            if (r < nq)
                *(uint4 *)((uint16_t *)O + (h * L + q0 + r) * 128 + 8 * ch) = *(const uint4 *)(st + r * PITCH + 16 * ch);
        }
        return;
    }

#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int col = wn * 64 + fn * 32 + acc_col(lane);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * 64 + fm * 32 + acc_row(lane, v);
                if (row >= nq) continue;
                const int64_t o = (h * L + q0 + row) * 128 + col;
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
    // 32-key slabs while the largest block keeps at most 8192 keys
    const int64_t kk_max = idx ? kk_rule(r, L) : L;
    const dim3 grid((unsigned)(H * Gq)), block(256);
    if (kk_max <= 8192) {
        if (idx)
            hipLaunchKernelGGL((k_pv_gemm<true, 32>), grid, block, 0, s, Pt, V, H, L, Gq, qblock, causal, r, idx,
                               ldidx, O, odt);
        else
            hipLaunchKernelGGL((k_pv_gemm<false, 32>), grid, block, 0, s, Pt, V, H, L, Gq, qblock, causal, r, idx,
                               ldidx, O, odt);
    } else {
        if (idx)
            hipLaunchKernelGGL((k_pv_gemm<true, 64>), grid, block, 0, s, Pt, V, H, L, Gq, qblock, causal, r, idx,
                               ldidx, O, odt);
        else
            hipLaunchKernelGGL((k_pv_gemm<false, 64>), grid, block, 0, s, Pt, V, H, L, Gq, qblock, causal, r, idx,
                               ldidx, O, odt);
    }
    return hipGetLastError();
}

}  // namespace rmm
