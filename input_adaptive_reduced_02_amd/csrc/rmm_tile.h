// rmm_tile.h -- LDS tile layout and the MFMA inner step shared by the reduced
// GEMM and the P.V kernel (gfx950, 64-wide wavefronts, 4 waves per workgroup).
//
// Both MFMA operands must hold 8 consecutive contraction indices per lane
// (v_mfma_f32_32x32x16_bf16: lane l supplies row/column l%32 at contraction
// offsets 8*(l/32) .. +7).  Tiles are therefore kept in LDS contraction-major:
//   As[m][k]  (TM rows of BK bf16)   and   Bs[n][k]  (TN rows of BK bf16).
// A rows come from memory already k-contiguous.  B arrives n-contiguous (row
// k of B, or a key row of P / V); each thread loads an 8x8 block (8 rows x 16
// bytes), transposes it in registers (transpose8x8) and writes 8 k-contiguous
// 16-byte chunks.
//
// Bank conflicts: a row is BK*2 bytes, a multiple of 128, so without care all
// rows start on the same bank.  The 16-byte chunk c of row x is stored at
// chunk position c ^ swz(x), swz(x) = (x ^ (x >> 3)) & 7.  The three access
// patterns then touch 8 distinct 16-byte bank groups per 8 lanes:
//   MFMA operand reads: 8 consecutive rows (8-aligned), same c -> x & 7 varies;
//   row-contiguous writes: 8 consecutive chunks of one row -> c varies;
//   transposed writes: rows 8 apart (x>>3 varies, x & 7 fixed), same c.
#pragma once
#include "rmm_internal.h"

namespace rmm {

__device__ __forceinline__ int swz(int x) { return (x ^ (x >> 3)) & 7; }

// Zero the halves at positions >= valid (0..8) of an 8 x bf16 vector.
__device__ __forceinline__ uint4 keep_first(uint4 v, int valid)
{
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 2 * i;
        if (e >= valid) w[i] = 0;
        else if (e + 1 >= valid) w[i] &= 0xffffu;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// One BK-deep slab of MFMAs for a wave tile of (32*FM) x (32*FN).
template <int BK, int FM, int FN>
__device__ __forceinline__ void mfma_slab(const uint16_t *__restrict__ As, const uint16_t *__restrict__ Bs,
                                          int arow0, int bcol0, int lane, floatx16 (&acc)[FM][FN])
{
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        const int c = 2 * ks + (lane >> 5);
        bf16x8 af[FM], bfr[FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int r = arow0 + fm * 32 + (lane & 31);
            af[fm] = *(const bf16x8 *)(As + r * BK + ((c ^ swz(r)) << 3));
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = bcol0 + fn * 32 + (lane & 31);
            bfr[fn] = *(const bf16x8 *)(Bs + n * BK + ((c ^ swz(n)) << 3));
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
    }
}

// Store one k-contiguous chunk (row r, chunk c), or one 8x8 unit loaded
// n-contiguous (rows n0..n0+7 of the tile after transposing, chunk kb).
template <int BK>
__device__ __forceinline__ void st_a(uint16_t *As, int r, int c, uint4 v)
{
    *(uint4 *)(As + r * BK + ((c ^ swz(r)) << 3)) = v;
}

template <int BK>
__device__ __forceinline__ void st_unit_t(uint16_t *Bs, int n0, int kb, const uint4 (&rows)[8])
{
    uint4 tr[8];
    transpose8x8(rows, tr);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int n = n0 + e;
        *(uint4 *)(Bs + n * BK + ((kb ^ swz(n)) << 3)) = tr[e];
    }
}

// Row/column of accumulator element v (0..15) of lane `lane` in a 32x32 block.
__device__ __forceinline__ int acc_row(int lane, int v) { return (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

}  // namespace rmm
