// rmm_q8.hip -- the RMM hot path on int8 weights (gfx950): the quantiser, the
// row norms of the dequantised weight, and the reduced GEMM over kept int8
// weight rows.
//
// The pages ("Reduced Matrix Multiplication (RMM) para Inferencia de LLM",
// section "Resultados Experimentais", item "Compatibilidade") state that the
// method works on INT8-quantised weights and fix no scheme.  This library
// uses symmetric absmax quantisation with one binary32 scale per output
// column n:
//   s_n = max_k |B[k,n]| / 127,  q[k,n] = round-half-even(B[k,n] / s_n),
// both divisions correctly rounded binary32 (they decide integers), codes in
// [-127, 127]; an all-zero column has s_n = 0 and q = 0.  The method then runs
// on the dequantised weight s_n * q[k,n]: its row norms score the slices, and
// the product is
//   Y[m,n] = s_n * sum_j Apanel[m,j] * q[row(g,j), n].
//
// Why it pays: a kept weight row costs N bytes of HBM instead of 2N, and the
// decode-shape product is bound by exactly those bytes.
#include "rmm_gemm_dl.h"

namespace rmm {

// ------------------------------------------------------------------ quantiser
// Column absmax as binary32 bit patterns (for non-negative floats the bit
// pattern orders like the value, so an unsigned atomic max is the float max).
__global__ void __launch_bounds__(256) k_q8_clear(uint32_t *__restrict__ bits, int64_t N)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < N) bits[i] = 0u;
}

// Grid (ceil(N/8/256), splits): a lane owns 8 columns (one 16-byte load per
// row, consecutive lanes on consecutive 16-byte chunks) over a band of rows.
__global__ void __launch_bounds__(256)
k_q8_amax(const uint16_t *__restrict__ B, int64_t K, int64_t N, int64_t ldb, int64_t band,
          uint32_t *__restrict__ bits)
{
    const int64_t c = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (c >= N) return;
    const int64_t k0 = (int64_t)blockIdx.y * band;
    const int64_t k1 = (k0 + band < K) ? k0 + band : K;
    uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 8
    for (int64_t k = k0; k < k1; ++k) {
        const u32x4 v = *(const u32x4 *)(B + k * ldb + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = (v[i] << 16) & 0x7fffffffu, hi = v[i] & 0x7fff0000u;
            m[2 * i] = m[2 * i] > lo ? m[2 * i] : lo;
            m[2 * i + 1] = m[2 * i + 1] > hi ? m[2 * i + 1] : hi;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (m[e]) atomicMax(bits + c + e, m[e]);
}

// In place: absmax bits -> s_n = absmax / 127 (binary32, correctly rounded).
__global__ void __launch_bounds__(256) k_q8_scale(uint32_t *__restrict__ bits, int64_t N)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < N) ((float *)bits)[i] = __uint_as_float(bits[i]) / 127.0f;
}

__device__ __forceinline__ uint32_t q8_code(float w, float s)
{
    if (s == 0.0f) return 0u;
    float t = __builtin_rintf(w / s);   // correctly rounded quotient, ties to even
    t = t > 127.0f ? 127.0f : (t < -127.0f ? -127.0f : t);
    return (uint32_t)(int32_t)t & 0xffu;
}

// A lane turns 16 consecutive bf16 weights of one row into 16 codes.
__global__ void __launch_bounds__(256)
k_q8_quant(const uint16_t *__restrict__ B, int64_t K, int64_t N, int64_t ldb,
           const float *__restrict__ scale, int8_t *__restrict__ q, int64_t ldq)
{
    const int64_t chunks = N / 16;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= K * chunks) return;
    const int64_t k = t / chunks, c = (t % chunks) * 16;
    const u32x4 v0 = *(const u32x4 *)(B + k * ldb + c);
    const u32x4 v1 = *(const u32x4 *)(B + k * ldb + c + 8);
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w0 = i < 2 ? v0[2 * i] : v1[2 * i - 4];
        const uint32_t w1 = i < 2 ? v0[2 * i + 1] : v1[2 * i - 3];
        const int64_t n = c + 4 * i;
        out[i] = q8_code(bf16_lo(w0), scale[n]) | q8_code(bf16_hi(w0), scale[n + 1]) << 8 |
                 q8_code(bf16_lo(w1), scale[n + 2]) << 16 | q8_code(bf16_hi(w1), scale[n + 3]) << 24;
    }
    *(u32x4 *)(q + k * ldq + c) = out;
}

// ------------------------------------------------------------------ row norms
// b[k] = ||(s_n q[k,n])_n||_2 in binary64.  One lane per row, ascending n,
// each term s_n * q (exact) squared and added with one rounding each (the
// build disables contraction), so the sum is the same sequence of roundings
// as the plain left-to-right loop.
__global__ void __launch_bounds__(256)
k_rownorms_q8(const int8_t *__restrict__ q, int64_t ldq, const float *__restrict__ scale, int64_t K,
              int64_t N, double *__restrict__ out)
{
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= K) return;
    const int8_t *row = q + k * ldq;
    double acc = 0.0;
    for (int64_t n = 0; n < N; n += 16) {
        const u32x4 v = *(const u32x4 *)(row + n);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const double x = (double)scale[n + i] * (double)(int8_t)(v[i >> 2] >> (8 * (i & 3)));
            const double sq = x * x;
            acc = acc + sq;
        }
    }
    out[k] = __builtin_sqrt(acc);
}

// ------------------------------------------------------------------ GEMM
// Tile 64 x 128 x 64, 4 waves side by side along N (wave w owns columns
// 32w..32w+31 and all 64 rows: 2 x 1 fragments of v_mfma_f32_32x32x16_bf16).
//
// A tile: the bf16 panel, k-contiguous rows of 128 B, chunk c of row r at
// slot c ^ swz(r) (as the other GEMMs).  B tile: 64 kept int8 rows of 128 B
// (8 chunks of 16 columns), chunk c of row k at slot c ^ swz_q8(k).
//
// B fragments come from ds_read_b64_tr_b8: in each 16-lane block, lane
// 2b + h addresses bytes [8h, 8h+8) of row b of an 8 x 16 byte block, and
// lane 8h + c receives byte c of each of the 8 rows: column 8h + c, 8
// consecutive k -- the k-run of a bf16 MFMA B fragment.  Lanes 0-31 read k
// 0-7 of the 16-deep step and lanes 32-63 k 8-15; blocks 0/2 cover columns
// 0-15 and blocks 1/3 columns 16-31 of the wave's strip.  The 8 codes are
// widened to bf16 exactly (|q| <= 127 needs 7 significant bits).
//
// Pipeline as the bf16 decode kernel: D slabs ahead, NSTAGE = D + 1 ring
// stages, index ring 2D; every step issues the same operations (slabs past
// the end reload valid memory), so the count of memory operations newer than
// AB(i) is always (D-1) * (1 + AB_OPS).  With half the bytes per B row, D = 6
// keeps as many weight bytes in flight per CU as the bf16 kernel's D = 3.
#ifndef RMM_Q8_DEPTH
#define RMM_Q8_DEPTH 6
#endif

struct Q8Shape {
    static constexpr int TM = 64, TN = 128, BK = 64, NW = 4;
    static constexpr int WN = 32, FM = 2, KS = BK / 16;
    static constexpr int D = RMM_Q8_DEPTH, NSTAGE = D + 1, IDX_RING = 2 * D;
    static constexpr int A_BYTES = TM * BK * 2;            // 8 KiB
    static constexpr int B_BYTES = BK * TN;                // 8 KiB
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int A_SHARE = A_BYTES / 1024 / NW;    // 1 KiB DMA blocks per wave per slab: 2
    static constexpr int B_SHARE = B_BYTES / 1024 / NW;    // 2
};

// Rows k..k+7 (k a multiple of 8) of one transposed read each give 32 lanes
// one 32-byte chunk pair; shifting the pair by (k >> 1) & 3 puts the 8 rows
// of 128 B into the 8 distinct 32-byte bank groups of a 256-byte bank line.
__device__ __forceinline__ int swz_q8(int k) { return ((k >> 1) & 3) << 1; }

typedef int intx2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) intx2 lds_intx2;

// two int8 codes (bytes sh/8 and sh/8+1 of x) -> two bf16 in one word, exact
__device__ __forceinline__ uint32_t q8_pair_bf16(uint32_t x, int sh)
{
    const float a = (float)(int8_t)(x >> sh);
    const float b = (float)(int8_t)(x >> (sh + 8));
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

template <bool IDX>
__global__ void __launch_bounds__(64 * Q8Shape::NW)
k_gemm_q8(const uint16_t *__restrict__ A, int64_t lda, const int8_t *__restrict__ Bq, int64_t ldq,
          const float *__restrict__ scale, const int32_t *__restrict__ idx, int64_t ldidx, int64_t M,
          int64_t N, int64_t kk, int64_t gr, void *__restrict__ Y, int ydt, int64_t ldy,
          int tiles_per_group, int m_tiles, int n_tiles)
{
    using S = Q8Shape;
    constexpr int TM = S::TM, TN = S::TN, BK = S::BK, WN = S::WN, FM = S::FM, KS = S::KS, D = S::D;
    constexpr int AB_OPS = S::A_SHARE + S::B_SHARE;
    constexpr int STEADY = (D - 1) * ((IDX ? 1 : 0) + AB_OPS);
    __shared__ __attribute__((aligned(1024))) char smem[S::NSTAGE * S::STAGE_BYTES];
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
    // B blocks [2w, 2w+2) (8 rows x 128 B each)
    // A chunks starting at or past kk read column 0 instead (their values are
    // cleared in registers), so A needs only lda >= kk; index loads past kk
    // read entry kk-1 (unused), so idx needs only ldidx >= kk.
    const uint16_t *a_row[S::A_SHARE];
    int a_col[S::A_SHARE];
#pragma unroll
    for (int i = 0; i < S::A_SHARE; ++i) {
        const int r = (wave * S::A_SHARE + i) * 8 + (lane >> 3);
        int64_t row = row0 + r;
        if (row > M - 1) row = M - 1;
        a_row[i] = A + row * lda;
        a_col[i] = ((lane & 7) ^ swz(r)) << 3;
    }
    const int8_t *b_src[S::B_SHARE];
#pragma unroll
    for (int i = 0; i < S::B_SHARE; ++i) {
        const int k = (wave * S::B_SHARE + i) * 8 + (lane >> 3);
        const int64_t c = col0 + (((lane & 7) ^ swz_q8(k)) << 4);
        b_src[i] = Bq + ((c < N) ? c : 0);   // columns past N: any valid chunk, never stored
    }
    const uint32_t smem0 = lds_addr(smem);
    const uint32_t iring0 = lds_addr(&iring[wave][0][0]);

    auto issue_idx = [&](int kt) {
        if constexpr (IDX) {
            int64_t j = (int64_t)(kt < nkt ? kt : 0) * BK + lane;
            if (j > kk - 1) j = kk - 1;
            dma4(I + j, iring0 + (kt % S::IDX_RING) * BK * 4);
        }
    };
    // this wave's share of slab kt (past the end: the last A slab, B row 0)
    // into ring stage kt % NSTAGE; B row indices read before any DMA
    auto issue_ab = [&](int kt) {
        const int64_t kbase = (int64_t)kt * BK;
        const int64_t abase = (int64_t)(kt < nkt ? kt : nkt - 1) * BK;
        int32_t kr[S::B_SHARE];
#pragma unroll
        for (int i = 0; i < S::B_SHARE; ++i) {
            const int jr = (wave * S::B_SHARE + i) * 8 + (lane >> 3);
            if constexpr (IDX) kr[i] = iring[wave][kt % S::IDX_RING][jr];
            else kr[i] = (int32_t)(kbase + jr);
        }
        const int8_t *brow[S::B_SHARE];
#pragma unroll
        for (int i = 0; i < S::B_SHARE; ++i) {
            const int jr = (wave * S::B_SHARE + i) * 8 + (lane >> 3);
            const int64_t krow = (kbase + jr < kk) ? kr[i] : 0;   // past kk: row 0
            brow[i] = b_src[i] + krow * ldq;
        }
        const uint32_t sa = smem0 + (kt % S::NSTAGE) * S::STAGE_BYTES;
        const uint32_t sb = sa + S::A_BYTES;
#pragma unroll
        for (int i = 0; i < S::A_SHARE; ++i) {
            const int64_t ac = abase + a_col[i];
            dma16(a_row[i] + (ac < kk ? ac : 0), sa + (wave * S::A_SHARE + i) * 1024);
        }
#pragma unroll
        for (int i = 0; i < S::B_SHARE; ++i) dma16(brow[i], sb + (wave * S::B_SHARE + i) * 1024);
    };

    floatx16 acc[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[fm][v] = 0.0f;

    // per-lane byte offset of the transposed byte reads within a stage's B tile
    int b_off;
    {
        const int blk = lane >> 4, b = (lane & 15) >> 1, h = lane & 1;
        const int k = (blk >> 1) * 8 + b;
        const int c = 2 * wave + (blk & 1);
        b_off = k * TN + ((c ^ swz_q8(k)) << 4) + h * 8;
    }

    // ---- prologue
#pragma unroll
    for (int p = 0; p < D; ++p) issue_idx(p);
    vmwait<0>();
#pragma unroll
    for (int p = 0; p < D; ++p) {
        issue_idx(p + D);
        issue_ab(p);
    }

    for (int kt = 0; kt < nkt; ++kt) {
        vmwait<STEADY>();   // this wave's share of slab kt landed
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // every wave's share of slab kt landed; stage (kt+D) % NSTAGE (slab
        // kt-1) has no reader left
        issue_idx(kt + 2 * D);
        issue_ab(kt + D);
        const char *st = smem + (kt % S::NSTAGE) * S::STAGE_BYTES;
        const uint16_t *sa = (const uint16_t *)st;
        const char *sb = st + S::A_BYTES;
        const bool tail = (int64_t)(kt + 1) * BK > kk;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = 2 * ks + (lane >> 5);
            bf16x8 af[FM];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int r = fm * 32 + (lane & 31);
                af[fm] = *(const bf16x8 *)(sa + r * BK + ((c ^ swz(r)) << 3));
            }
            if (tail) {
                const int64_t k0 = (int64_t)kt * BK + ks * 16 + 8 * (lane >> 5);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (k0 + e >= kk)
#pragma unroll
                        for (int fm = 0; fm < FM; ++fm) af[fm][e] = (__bf16)0.0f;
            }
            const intx2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2 *)(sb + b_off + ks * 16 * TN));
            u32x4 w;
            w[0] = q8_pair_bf16((uint32_t)raw[0], 0);
            w[1] = q8_pair_bf16((uint32_t)raw[0], 16);
            w[2] = q8_pair_bf16((uint32_t)raw[1], 0);
            w[3] = q8_pair_bf16((uint32_t)raw[1], 16);
            const bf16x8 bfr = __builtin_bit_cast(bf16x8, w);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                acc[fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr, acc[fm], 0, 0, 0);
        }
    }
    vmwait<0>();   // the trailing reloads: no DMA may land after the workgroup ends

    const int64_t col = col0 + wave * WN + acc_col(lane);
    if (col < N) {
        const float sc = scale[col];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = row0 + fm * 32 + acc_row(lane, v);
                if (row >= row_end) continue;
                const float y = acc[fm][v] * sc;
                if (ydt == 1)
                    ((uint16_t *)Y)[row * ldy + col] = (uint16_t)f32_to_bf16(y);
                else
                    ((float *)Y)[row * ldy + col] = y;
            }
        }
    }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_quantize_q8(const uint16_t *B, int64_t K, int64_t N, int64_t ldb, int8_t *q,
                              int64_t ldq, float *scale, hipStream_t s)
{
    uint32_t *bits = (uint32_t *)scale;
    const unsigned nb = (unsigned)((N + 255) / 256);
    hipLaunchKernelGGL(k_q8_clear, dim3(nb), dim3(256), 0, s, bits, N);
    // bands of rows so that about 64k lanes share the column reduction
    const int64_t col_blocks = (N / 8 + 255) / 256;
    int64_t splits = (65536 / 256 + col_blocks - 1) / col_blocks;
    if (splits > K) splits = K;
    if (splits > 65535) splits = 65535;
    const int64_t band = (K + splits - 1) / splits;
    splits = (K + band - 1) / band;
    hipLaunchKernelGGL(k_q8_amax, dim3((unsigned)col_blocks, (unsigned)splits), dim3(256), 0, s, B, K, N,
                       ldb, band, bits);
    hipLaunchKernelGGL(k_q8_scale, dim3(nb), dim3(256), 0, s, bits, N);
    const int64_t lanes = K * (N / 16);
    hipLaunchKernelGGL(k_q8_quant, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s, B, K, N, ldb,
                       (const float *)scale, q, ldq);
    return hipGetLastError();
}

hipError_t launch_rownorms_q8(const int8_t *q, int64_t ldq, const float *scale, int64_t K, int64_t N,
                              double *out, hipStream_t s)
{
    hipLaunchKernelGGL(k_rownorms_q8, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s, q, ldq, scale, K,
                       N, out);
    return hipGetLastError();
}

hipError_t launch_gemm_q8(const uint16_t *A, int64_t lda, const int8_t *Bq, int64_t ldq,
                          const float *scale, const int32_t *idx, int64_t ldidx, int64_t M, int64_t N,
                          int64_t kk, int64_t group_rows, void *Y, int ydt, int64_t ldy, hipStream_t s)
{
    using S = Q8Shape;
    const int64_t G = (M + group_rows - 1) / group_rows;
    const int tiles_per_group = (int)((group_rows + S::TM - 1) / S::TM);
    const int m_tiles = (int)(G * tiles_per_group);
    const int n_tiles = (int)((N + S::TN - 1) / S::TN);
    const int total = m_tiles * n_tiles;
    const dim3 grid((unsigned)(8 * ((total + 7) / 8))), block(64 * S::NW);
    if (idx)
        hipLaunchKernelGGL(k_gemm_q8<true>, grid, block, 0, s, A, lda, Bq, ldq, scale, idx, ldidx, M, N, kk,
                           group_rows, Y, ydt, ldy, tiles_per_group, m_tiles, n_tiles);
    else
        hipLaunchKernelGGL(k_gemm_q8<false>, grid, block, 0, s, A, lda, Bq, ldq, scale, idx, ldidx, M, N, kk,
                           group_rows, Y, ydt, ldy, tiles_per_group, m_tiles, n_tiles);
    return hipGetLastError();
}

}  // namespace rmm
