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
// Tile 64 x 128 (rows x columns), 4 waves, no barrier in the main loop.
// The kept rows are cut into slabs of 32; wave w takes a contiguous quarter
// of the slabs and multiplies each into its own full 64 x 128 fp32
// accumulator (2 x 4 fragments of v_mfma_f32_32x32x16_bf16).  Every wave
// streams its slabs through a private LDS ring with its own DMA loads and
// its own s_waitcnt, so the waves never wait for one another (a slab shared
// by all waves would make every step wait for the slowest wave's loads); each
// A and B byte of a slab is read from LDS once.  The four partial tiles are
// summed through LDS once, at the end.
//
// A tile of a slab: the bf16 panel, 64 rows of 64 B (4 chunks of 8 k), chunk
// c of row r at slot c ^ ((r >> 2) & 3): the 16 rows of one 16-lane phase of
// a fragment read fall in 16 distinct 16-byte bank groups.  B tile: 32 kept
// int8 rows of 128 B (8 chunks of 16 columns), chunk c of row k at slot
// c ^ swz_q8(k).
//
// B fragments come from ds_read_b64_tr_b8: in each 16-lane block, lane
// 2b + h addresses bytes [8h, 8h+8) of row b of an 8 x 16 byte block, and
// lane 8h + c receives byte c of each of the 8 rows: column 8h + c, 8
// consecutive k -- the k-run of a bf16 MFMA B fragment.  Lanes 0-31 read k
// 0-7 of a 16-deep step and lanes 32-63 k 8-15; blocks 0/2 cover columns
// 0-15 and blocks 1/3 columns 16-31 of a 32-column fragment.  The 8 codes
// are widened to bf16 exactly (|q| <= 127 needs 7 significant bits).
//
// Per-wave pipeline: NS ring stages, D = NS - 1 slabs of DMA ahead, index
// ring 2D.  Step i waits for the wave's slab i, reads its fragments and the
// row indices of slab i+D, issues the DMA of slab i+D (into the stage slab
// i-1 used, whose fragments the MFMAs of step i-1 consumed) and the index
// DMA of slab i+2D, and runs the MFMAs of slab i.  Every step issues the same
// memory operations (slabs past the wave's last reload valid memory: the last
// A slab and row 0 of B), so the count of operations newer than slab i's is
// always (D-1) * OPS.
#ifndef RMM_Q8_STAGES
#define RMM_Q8_STAGES 3
#endif
#ifndef RMM_Q8_TN
#define RMM_Q8_TN 256
#endif

struct Q8Shape {
    static constexpr int TM = 64, TN = RMM_Q8_TN, BK = 32, NW = 4;
    static constexpr int B_ROWS_PER_BLOCK = 1024 / TN, B_CHUNKS = TN / 16;
    static constexpr int FM = TM / 32, FN = TN / 32, KS = BK / 16;
    static constexpr int NS = RMM_Q8_STAGES, D = NS - 1, IDX_RING = 2 * D;
    static constexpr int A_BYTES = TM * BK * 2;                  // 4 KiB
    static constexpr int B_BYTES = BK * TN;                      // 4 KiB
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int A_BLOCKS = A_BYTES / 1024, B_BLOCKS = B_BYTES / 1024;   // 1 KiB DMA blocks
    static constexpr int WAVE_BYTES = NS * STAGE_BYTES;          // one wave's ring
    static constexpr int PART_PITCH = TN;                        // fp32 partial tiles, 32 rows each
    static constexpr int RED_COLS = TN / NW;                     // columns each wave sums and stores
    static_assert(NW * 32 * TN * 4 <= NW * WAVE_BYTES, "partial tiles must fit the rings");
    static_assert(2 * (TN / NW / 2) * 64 * NW == TM * TN, "a part's sums fill its workspace tile");
};

__device__ __forceinline__ int swz_a32(int r) { return (r >> 2) & 3; }

// Rows k..k+7 (k a multiple of 8) of one transposed read each give 32 lanes
// one 32-byte chunk pair.  Rows of 128 B: shifting the pair by (k >> 1) & 3
// puts the 8 rows into the 8 distinct 32-byte bank groups of a 256-byte bank
// line; rows of 256 B: shifting it by k & 7 does.
__device__ __forceinline__ int swz_q8(int k)
{
    return Q8Shape::TN == 128 ? ((k >> 1) & 3) << 1 : (k & 7) << 1;
}

typedef int intx2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) intx2 lds_intx2;

// two int8 codes (bytes sh/8 and sh/8+1 of x) -> two bf16 in one word, exact
__device__ __forceinline__ uint32_t q8_pair_bf16(uint32_t x, int sh)
{
    const float a = (float)(int8_t)(x >> sh);
    const float b = (float)(int8_t)(x >> (sh + 8));
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

__device__ __forceinline__ bf16x8 q8_frag(intx2 raw)
{
    u32x4 w;
    w[0] = q8_pair_bf16((uint32_t)raw[0], 0);
    w[1] = q8_pair_bf16((uint32_t)raw[0], 16);
    w[2] = q8_pair_bf16((uint32_t)raw[1], 0);
    w[3] = q8_pair_bf16((uint32_t)raw[1], 16);
    return __builtin_bit_cast(bf16x8, w);
}

// fp32 partial tile in LDS: row r, column c at r * 128 + (c ^ ((r & 4) << 3)),
// so the two row groups of one accumulator write (rows r and r + 4) fall in
// different halves of the 64 banks
__device__ __forceinline__ int part_at(int r, int c) { return r * Q8Shape::PART_PITCH + (c ^ ((r & 4) << 3)); }

template <bool IDX>
__global__ void __launch_bounds__(64 * Q8Shape::NW)
k_gemm_q8(const uint16_t *__restrict__ A, int64_t lda, const int8_t *__restrict__ Bq, int64_t ldq,
          const float *__restrict__ scale, const int32_t *__restrict__ idx, int64_t ldidx, int64_t M,
          int64_t N, int64_t kk, int64_t gr, void *__restrict__ Y, int ydt, int64_t ldy,
          int tiles_per_group, int m_tiles, int n_tiles, int ksplit, float *__restrict__ part_ws,
          unsigned int *__restrict__ arrivals)
{
    using S = Q8Shape;
    constexpr int TM = S::TM, TN = S::TN, BK = S::BK, FM = S::FM, FN = S::FN, KS = S::KS;
    constexpr int D = S::D, NS = S::NS;
    constexpr int OPS = (IDX ? 1 : 0) + S::A_BLOCKS + S::B_BLOCKS;
    constexpr int STEADY = (D - 1) * OPS;
    __shared__ __attribute__((aligned(1024))) char smem[S::NW * S::WAVE_BYTES];
    __shared__ __attribute__((aligned(256))) int32_t iring[S::NW][S::IDX_RING][64];

    // work item t = tile * ksplit + part; the parts of one tile are
    // consecutive items, so they run on the same XCD
    const int total = m_tiles * n_tiles * ksplit;
    const int per = (total + 7) / 8;
    const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (t >= total) return;   // whole workgroup: no barrier is ever reached
    const int tile = t / ksplit, kpart = t % ksplit;
    const int nt = tile / m_tiles, mt = tile % m_tiles;
    const int64_t g = mt / tiles_per_group;
    const int64_t row0 = g * gr + (int64_t)(mt % tiles_per_group) * TM;
    const int64_t row_end = (g * gr + gr < M) ? g * gr + gr : M;
    const int64_t col0 = (int64_t)nt * TN;
    const int32_t *I = IDX ? idx + g * ldidx : nullptr;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nkt = (int)((kk + BK - 1) / BK);
    const int pslabs = (nkt + ksplit - 1) / ksplit;      // this workgroup's slabs: [p0, p1)
    const int p0 = min(nkt, kpart * pslabs), p1 = min(nkt, p0 + pslabs);
    const int quarter = (p1 - p0 + S::NW - 1) / S::NW;
    const int s0 = min(p1, p0 + wave * quarter);         // this wave's slabs: [s0, s0 + n)
    const int n = min(p1, s0 + quarter) - s0;

    // ---- per-lane DMA sources.  A block b: rows 16b + lane/4, 16-byte slot
    // lane % 4; B block b: kept rows 8b + lane/8, slot lane % 8.  A chunks
    // starting at or past kk read column 0 instead (their values are cleared
    // in registers), so A needs only lda >= kk; index loads past kk read
    // entry kk-1 (unused), so idx needs only ldidx >= kk.
    const uint16_t *a_row[S::A_BLOCKS];
    int a_col[S::A_BLOCKS];
#pragma unroll
    for (int b = 0; b < S::A_BLOCKS; ++b) {
        const int r = b * 16 + (lane >> 2);
        int64_t row = row0 + r;
        if (row > M - 1) row = M - 1;
        a_row[b] = A + row * lda;
        a_col[b] = ((lane & 3) ^ swz_a32(r)) << 3;
    }
    const int8_t *b_src[S::B_BLOCKS];
#pragma unroll
    for (int b = 0; b < S::B_BLOCKS; ++b) {
        const int k = b * S::B_ROWS_PER_BLOCK + lane / S::B_CHUNKS;
        const int64_t c = col0 + (((lane % S::B_CHUNKS) ^ swz_q8(k)) << 4);
        b_src[b] = Bq + ((c < N) ? c : 0);   // columns past N: any valid chunk, never stored
    }
    const uint32_t ring0 = lds_addr(smem) + wave * S::WAVE_BYTES;
    const char *ring = smem + wave * S::WAVE_BYTES;
    const uint32_t iring0 = lds_addr(&iring[wave][0][0]);

    // the wave's i-th slab is slab s0 + i; past the wave's last slab: reloads
    auto issue_idx = [&](int i) {
        if constexpr (IDX) {
            const int s = s0 + i;
            int64_t j = (int64_t)(i < n ? s : 0) * BK + (lane & 31);
            if (j > kk - 1) j = kk - 1;
            dma4(I + j, iring0 + (i % S::IDX_RING) * 256);
        }
    };
    auto load_rows = [&](int i, int32_t (&kr)[S::B_BLOCKS]) {
#pragma unroll
        for (int b = 0; b < S::B_BLOCKS; ++b) {
            const int jr = b * S::B_ROWS_PER_BLOCK + lane / S::B_CHUNKS;
            if constexpr (IDX) kr[b] = iring[wave][i % S::IDX_RING][jr];
            else kr[b] = (s0 + i) * BK + jr;
        }
    };
    auto issue_ab = [&](int i, const int32_t (&kr)[S::B_BLOCKS]) {
        const int s = s0 + i;
        const int64_t kbase = (int64_t)s * BK;
        const int64_t abase = (int64_t)(s < nkt ? s : nkt - 1) * BK;
        const uint32_t sa = ring0 + (i % NS) * S::STAGE_BYTES;
        const uint32_t sb = sa + S::A_BYTES;
#pragma unroll
        for (int b = 0; b < S::A_BLOCKS; ++b) {
            const int64_t ac = abase + a_col[b];
            dma16(a_row[b] + (ac < kk ? ac : 0), sa + b * 1024);
        }
#pragma unroll
        for (int b = 0; b < S::B_BLOCKS; ++b) {
            const int jr = b * S::B_ROWS_PER_BLOCK + lane / S::B_CHUNKS;
            const int64_t krow = (i < n && kbase + jr < kk) ? kr[b] : 0;   // past the end: row 0
            dma16_nt(b_src[b] + krow * ldq, sb + b * 1024);
        }
    };

    // per-lane offsets of the fragments within a stage (k-step 0; k-step 1 at
    // + 32 bytes for A, + 16 * TN for B)
    int a_off[FM][KS];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int r = fm * 32 + (lane & 31);
            a_off[fm][ks] = r * BK * 2 + (((2 * ks + (lane >> 5)) ^ swz_a32(r)) << 4);
        }
    int b_off[FN];
    {
        const int blk = lane >> 4, b = (lane & 15) >> 1, h = lane & 1;
        const int k = (blk >> 1) * 8 + b;   // (k + 16) has the same swizzle
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            b_off[fn] = S::A_BYTES + k * TN + (((2 * fn + (blk & 1)) ^ swz_q8(k)) << 4) + h * 8;
    }

    floatx16 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.0f;

    // ---- prologue
#pragma unroll
    for (int p = 0; p < D; ++p) issue_idx(p);
    vmwait<0>();
#pragma unroll
    for (int p = 0; p < D; ++p) {
        issue_idx(p + D);
        int32_t kr[S::B_BLOCKS];
        load_rows(p, kr);
        issue_ab(p, kr);
    }

    for (int i = 0; i < n; ++i) {
        vmwait<STEADY>();   // the wave's slab i landed (and the indices of slab i+D)
        int32_t kr[S::B_BLOCKS];
        load_rows(i + D, kr);
        const char *st = ring + (i % NS) * S::STAGE_BYTES;
        u32x4 af[KS][FM];
        intx2 bf[KS][FN];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) af[ks][fm] = *(const u32x4 *)(st + a_off[fm][ks]);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                bf[ks][fn] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2 *)(st + b_off[fn] + ks * 16 * TN));
        }
        issue_idx(i + 2 * D);
        issue_ab(i + D, kr);
        const int64_t kslab = (int64_t)(s0 + i) * BK;
        if (kslab + BK > kk) {   // the last slab: clear A columns at or past kk
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int64_t k0 = kslab + ks * 16 + 8 * (lane >> 5);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t m = (k0 + 2 * q < kk ? 0x0000ffffu : 0u) | (k0 + 2 * q + 1 < kk ? 0xffff0000u : 0u);
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm) af[ks][fm][q] &= m;
                }
            }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const bf16x8 b = q8_frag(bf[ks][fn]);
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[ks][fm]), b,
                                                                          acc[fm][fn], 0, 0, 0);
            }
    }
    vmwait<0>();   // the trailing reloads: no DMA may land after the rings are reused
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // ---- sum the four wave partials through LDS, 32 rows at a time (wave
    // w's partial in region w): a lane ends with one row and RED_COLS / 2
    // columns of the workgroup's sum
    constexpr int RC = S::RED_COLS, LC = RC / 2;
    float *part = (float *)smem;
    const int rr = lane >> 1, cc = wave * RC + (lane & 1) * LC;
    float y[FM][LC];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        float *mine = part + wave * 32 * S::PART_PITCH;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                mine[part_at(acc_row(lane, v), fn * 32 + acc_col(lane))] = acc[fm][fn][v];
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int e = 0; e < LC; ++e) y[fm][e] = 0.0f;
#pragma unroll
        for (int p = 0; p < S::NW; ++p) {
            const float *src = part + p * 32 * S::PART_PITCH + part_at(rr, cc);
#pragma unroll
            for (int q = 0; q < LC / 4; ++q) {
                const float4 v = *(const float4 *)(src + 4 * q);
                y[fm][4 * q] += v.x;
                y[fm][4 * q + 1] += v.y;
                y[fm][4 * q + 2] += v.z;
                y[fm][4 * q + 3] += v.w;
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // partials read before the next pass
    }

    // ---- split over workgroups: the two parts of a tile meet in global
    // memory (thread-major: element e of thread x at e * threads + x, so
    // every store and load of a wave is one 256-byte run).  Each part stores
    // its sum with agent-coherent stores, waits for them to complete, then
    // adds 1 to the tile's arrival counter; the part that finds 1 there
    // arrives second, sets the counter back to 0, reads the other sum with
    // agent-coherent loads and adds the two in part order (the first part
    // simply ends).  Every counter is thus 0 after any completed call, so a
    // workspace zero-filled once serves later calls of any shape, also
    // launches replayed from a graph.
    // Ordering: the partial sums are relaxed atomic stores and loads at agent
    // scope (global_store/load with sc1, performed at the device-coherent
    // level, not in an XCD's own L2), and s_waitcnt vmcnt(0) before the
    // counter update waits for every one of them to be acknowledged; the
    // second part issues its loads only after its counter update returned.
    // Release/acquire at agent scope would add a write-back and an
    // invalidation of the whole L2 around every handoff (measured 2.2x slower
    // for the kernel), for words that already bypass it.
    if (ksplit == 2) {
        float *mine_ws = part_ws + ((int64_t)tile * 2 + kpart) * (TM * TN);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int e = 0; e < LC; ++e)
                __hip_atomic_store(mine_ws + (fm * LC + e) * (64 * S::NW) + threadIdx.x, y[fm][e], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // every store of this wave completed
        __syncthreads();                                     // ... and of every wave
        __shared__ int second;
        if (threadIdx.x == 0) {
            const unsigned int old =
                __hip_atomic_fetch_add(arrivals + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            second = old == 1u;
            if (second)   // both parts have arrived: nothing else touches this counter in this call
                __hip_atomic_store(arrivals + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!second) return;
        const float *other = part_ws + ((int64_t)tile * 2 + (1 - kpart)) * (TM * TN);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int e = 0; e < LC; ++e) {
                const float o = __hip_atomic_load(other + (fm * LC + e) * (64 * S::NW) + threadIdx.x,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                float &x = y[fm][e];
                x = kpart == 0 ? x + o : o + x;
            }
    }

    // ---- column scale and store, in pieces of 8 columns (N % 16 == 0: a
    // piece is all inside or all past N)
    const int64_t col = col0 + cc;
    float sc[LC];
#pragma unroll
    for (int e = 0; e < LC; ++e) sc[e] = (col + e < N) ? scale[col + e] : 0.0f;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int64_t row = row0 + fm * 32 + rr;
        if (row >= row_end) continue;
        if (ydt == 1) {
#pragma unroll
            for (int q = 0; q < LC / 8; ++q) {
                if (col + 8 * q >= N) break;
                u32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 8 * q + 2 * e;
                    o[e] = f32_to_bf16(y[fm][c] * sc[c]) | (f32_to_bf16(y[fm][c + 1] * sc[c + 1]) << 16);
                }
                *(u32x4 *)((uint16_t *)Y + row * ldy + col + 8 * q) = o;
            }
        } else {
#pragma unroll
            for (int q = 0; q < LC / 8; ++q) {
                if (col + 8 * q >= N) break;
                float4 *dst = (float4 *)((float *)Y + row * ldy + col + 8 * q);
                const int c = 8 * q;
                dst[0] = make_float4(y[fm][c] * sc[c], y[fm][c + 1] * sc[c + 1], y[fm][c + 2] * sc[c + 2],
                                     y[fm][c + 3] * sc[c + 3]);
                dst[1] = make_float4(y[fm][c + 4] * sc[c + 4], y[fm][c + 5] * sc[c + 5], y[fm][c + 6] * sc[c + 6],
                                     y[fm][c + 7] * sc[c + 7]);
            }
        }
    }
}

// ------------------------------------------------------------------ GEMM, short kept lists
// k_gemm_q8s: for groups of at most 64 rows and at most 4096 kept rows.  One
// workgroup per 64 x 128 tile; its 4 waves sit side by side along N (wave w:
// columns 32w .. 32w+31, all 64 rows) and share one stream of 64-deep slabs
// through a 4-stage DMA ring (3 slabs in flight), so there are no partial
// sums to reduce and no split to hand off.  A short loop is where those fixed
// costs of k_gemm_q8 weigh most: decode shape (64 x 8192 @ 8192 x 28672, same
// box) 24.5 against 30.4 us at kk = 2458, 37.8 against 39.6 us at kk = 4096;
// past that the per-slab widening and MFMAs no longer hide under the stream
// (51.6 against 49.9 us at kk = 5735).  The two kernels add the same exact
// products in different fp32 orders.
struct Q8sShape {
    static constexpr int TM = 64, TN = 128, BK = 64, NW = 4, WN = 32, FM = 2, KS = BK / 16;
    static constexpr int D = 3, NSTAGE = D + 1, IDX_RING = 2 * D;
    static constexpr int A_BYTES = TM * BK * 2, B_BYTES = BK * TN, STAGE = A_BYTES + B_BYTES;   // 8 + 8 KiB
    static constexpr int A_SHARE = A_BYTES / 1024 / NW, B_SHARE = B_BYTES / 1024 / NW;       // 2, 2
};

// B rows of 128 bytes: chunk pair shifted by (k >> 1) & 3 (as swz_q8 for 128-byte rows)
__device__ __forceinline__ int swz_q8s(int k) { return ((k >> 1) & 3) << 1; }

template <bool IDX>
__global__ void __launch_bounds__(256)
k_gemm_q8s(const uint16_t *__restrict__ A, int64_t lda, const int8_t *__restrict__ Bq, int64_t ldq,
           const float *__restrict__ scale, const int32_t *__restrict__ idx, int64_t ldidx, int64_t M, int64_t N,
           int64_t kk, int64_t gr, void *__restrict__ Y, int ydt, int64_t ldy, int m_tiles, int n_tiles)
{
    using S = Q8sShape;
    constexpr int BK = S::BK, TN = S::TN, WN = S::WN, FM = S::FM, KS = S::KS, D = S::D;
    constexpr int AB_OPS = S::A_SHARE + S::B_SHARE;
    constexpr int STEADY = (D - 1) * ((IDX ? 1 : 0) + AB_OPS);   // operations always newer than AB(i)
    __shared__ __attribute__((aligned(1024))) char smem[S::NSTAGE * S::STAGE];
    __shared__ __attribute__((aligned(256))) int32_t iring[S::NW][S::IDX_RING][BK];

    // consecutive workgroups on consecutive XCDs take tiles 'per' apart
    const int total = m_tiles * n_tiles;
    const int per = (total + 7) / 8;
    const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (t >= total) return;
    const int nt = t / m_tiles, g = t % m_tiles;      // one row tile per group (gr <= 64)
    const int64_t row0 = (int64_t)g * gr;
    const int64_t row_end = (row0 + gr < M) ? row0 + gr : M;
    const int64_t col0 = (int64_t)nt * TN;
    const int32_t *I = IDX ? idx + g * ldidx : nullptr;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nkt = (int)((kk + BK - 1) / BK);

    // per-lane DMA sources: A rows (rows past M copy row M-1; rows of the next
    // group are loaded and never stored), B column chunks (past N: chunk 0)
    const uint16_t *a_src[S::A_SHARE];
#pragma unroll
    for (int i = 0; i < S::A_SHARE; ++i) {
        const int r = (wave * S::A_SHARE + i) * 8 + (lane >> 3);
        int64_t row = row0 + r;
        if (row > M - 1) row = M - 1;
        a_src[i] = A + row * lda + (((lane & 7) ^ swz(r)) << 3);
    }
    const int8_t *b_src[S::B_SHARE];
#pragma unroll
    for (int i = 0; i < S::B_SHARE; ++i) {
        const int k = (wave * S::B_SHARE + i) * 8 + (lane >> 3);
        const int64_t c = col0 + (((lane & 7) ^ swz_q8s(k)) << 4);
        b_src[i] = Bq + ((c < N) ? c : 0);
    }
    const uint32_t smem0 = lds_addr(smem);
    const uint32_t iring0 = lds_addr(&iring[wave][0][0]);
    // the slab's 64 kept-row indices (slabs past the end reload slab 0's)
    auto issue_idx = [&](int kt) {
        if constexpr (IDX) {
            const int64_t j = (int64_t)(kt < nkt ? kt : 0) * BK + lane;
            dma4(I + j, iring0 + (kt % S::IDX_RING) * BK * 4);
        }
    };
    auto load_rows = [&](int kt, int32_t (&kr)[S::B_SHARE]) {
#pragma unroll
        for (int i = 0; i < S::B_SHARE; ++i) {
            const int jr = (wave * S::B_SHARE + i) * 8 + (lane >> 3);
            if constexpr (IDX) kr[i] = iring[wave][kt % S::IDX_RING][jr];
            else kr[i] = kt * BK + jr;
        }
    };
    // A and B of slab kt (past the end: the last A slab and B row 0, valid
    // memory whose products are cleared in registers)
    auto issue_ab = [&](int kt, const int32_t (&kr)[S::B_SHARE]) {
        const int64_t kbase = (int64_t)kt * BK;
        const int64_t abase = (int64_t)(kt < nkt ? kt : nkt - 1) * BK;
        const uint32_t sa = smem0 + (kt % S::NSTAGE) * S::STAGE;
        const uint32_t sb = sa + S::A_BYTES;
#pragma unroll
        for (int i = 0; i < S::A_SHARE; ++i) dma16(a_src[i] + abase, sa + (wave * S::A_SHARE + i) * 1024);
#pragma unroll
        for (int i = 0; i < S::B_SHARE; ++i) {
            const int jr = (wave * S::B_SHARE + i) * 8 + (lane >> 3);
            const int64_t krow = (kbase + jr < kk) ? kr[i] : 0;
            dma16_nt(b_src[i] + krow * ldq, sb + (wave * S::B_SHARE + i) * 1024);
        }
    };
    // this lane's byte offset of its transposed B read within a stage
    int b_off;
    {
        const int blk = lane >> 4, b = (lane & 15) >> 1, h = lane & 1;
        const int k = (blk >> 1) * 8 + b;
        b_off = S::A_BYTES + k * TN + (((2 * wave + (blk & 1)) ^ swz_q8s(k)) << 4) + h * 8;
    }
    floatx16 acc[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[fm][v] = 0.0f;

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
    for (int kt = 0; kt < nkt; ++kt) {
        vmwait<STEADY>();   // this wave's share of slab kt landed
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        int32_t kr[S::B_SHARE];
        load_rows(kt + D, kr);
        const char *st = smem + (kt % S::NSTAGE) * S::STAGE;
        const uint16_t *sa = (const uint16_t *)st;
        u32x4 af[KS][FM];
        intx2 bf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = 2 * ks + (lane >> 5);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int r = fm * 32 + (lane & 31);
                af[ks][fm] = *(const u32x4 *)(sa + r * BK + ((c ^ swz(r)) << 3));
            }
            bf[ks] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2 *)(st + b_off + ks * 16 * TN));
        }
        issue_idx(kt + 2 * D);
        issue_ab(kt + D, kr);
        if ((int64_t)(kt + 1) * BK > kk) {   // partial last slab: clear A columns >= kk
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
            const bf16x8 b = q8_frag(bf[ks]);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                acc[fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[ks][fm]), b, acc[fm],
                                                                  0, 0, 0);
        }
    }
    vmwait<0>();   // the trailing reloads: no DMA may land after the workgroup ends

    const int colw = wave * WN + acc_col(lane);
    const float sc = (col0 + colw < N) ? scale[col0 + colw] : 0.0f;
    if (ydt == 1) {
        // bf16 output: stage the 64 x 128 tile in LDS (the ring is free once
        // every wave has passed the barrier below), then 16-byte row chunks
        constexpr int PITCH = TN * 2 + 16;
        char *stg = smem;
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = fm * 32 + acc_row(lane, v);
                *(uint16_t *)(stg + r * PITCH + 2 * colw) = (uint16_t)f32_to_bf16(acc[fm][v] * sc);
            }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        for (int e = threadIdx.x; e < S::TM * (TN / 8); e += 256) {
            const int r = e / (TN / 8), ch = e % (TN / 8);
            const int64_t row = row0 + r, cl = col0 + 8 * ch;
            if (row < row_end && cl < N)
                __builtin_nontemporal_store(*(const u32x4 *)(stg + r * PITCH + 16 * ch),
                                            (u32x4 *)((uint16_t *)Y + row * ldy + cl));
        }
        return;
    }
    const int64_t col = col0 + colw;
    if (col < N) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = row0 + fm * 32 + acc_row(lane, v);
                if (row < row_end) ((float *)Y)[row * ldy + col] = acc[fm][v] * sc;
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

// Tiles of 64 x 256; when there are at most 128 tiles (fewer than half the
// CUs) every tile is split into two halves of its kept rows, each on its own
// workgroup, which meet through the workspace (two fp32 partial tiles and a
// 4-byte arrival counter per tile).
int q8_ksplit(int64_t M, int64_t N, int64_t group_rows)
{
    using S = Q8Shape;
    const int64_t G = (M + group_rows - 1) / group_rows;
    const int64_t tiles = G * ((group_rows + S::TM - 1) / S::TM) * ((N + S::TN - 1) / S::TN);
    return tiles <= 128 ? 2 : 1;
}

// Workspace of a split call: the tiles' 4-byte arrival counters at its start
// (256-byte aligned block), the two fp32 partial tiles per tile at its end.
// With the counters at a fixed place and the partials right-aligned, the
// counters of any shape that fits a workspace never lie where an earlier
// call of another shape left partial sums.
static size_t q8_counter_bytes(int64_t tiles) { return ((size_t)tiles * 4 + 255) / 256 * 256; }
static size_t q8_partial_bytes(int64_t tiles) { return (size_t)tiles * 2 * Q8Shape::TM * Q8Shape::TN * sizeof(float); }

size_t gemm_q8_workspace_bytes(int64_t M, int64_t N, int64_t group_rows)
{
    using S = Q8Shape;
    if (q8_ksplit(M, N, group_rows) == 1) return 0;
    const int64_t G = (M + group_rows - 1) / group_rows;
    const int64_t tiles = G * ((group_rows + S::TM - 1) / S::TM) * ((N + S::TN - 1) / S::TN);
    return q8_counter_bytes(tiles) + q8_partial_bytes(tiles);
}

hipError_t launch_gemm_q8(const uint16_t *A, int64_t lda, const int8_t *Bq, int64_t ldq,
                          const float *scale, const int32_t *idx, int64_t ldidx, int64_t M, int64_t N,
                          int64_t kk, int64_t group_rows, void *Y, int ydt, int64_t ldy, void *ws, size_t ws_bytes,
                          hipStream_t s)
{
    using S = Q8Shape;
    const int64_t G = (M + group_rows - 1) / group_rows;
    const int tiles_per_group = (int)((group_rows + S::TM - 1) / S::TM);
    const int m_tiles = (int)(G * tiles_per_group);
    const int n_tiles = (int)((N + S::TN - 1) / S::TN);
    const int ksplit = q8_ksplit(M, N, group_rows);
    const int total = m_tiles * n_tiles * ksplit;
    float *part_ws = nullptr;
    unsigned int *arrivals = nullptr;
    if (ksplit == 2) {   // ws_bytes >= q8_counter_bytes + q8_partial_bytes (checked by the caller)
        arrivals = (unsigned int *)ws;
        const size_t off = (ws_bytes - q8_partial_bytes((int64_t)m_tiles * n_tiles)) / 256 * 256;
        part_ws = (float *)((char *)ws + off);
    }
    // short kept lists of small groups: one shared slab stream per 64 x 128
    // tile (its loads read whole 64-deep slabs of the panel and the index row)
    if (group_rows <= 64 && kk <= 4096 && lda >= pad_up(kk) && (!idx || ldidx >= pad_up(kk))) {
        using T = Q8sShape;
        const int mt = (int)G, ntl = (int)((N + T::TN - 1) / T::TN);
        const dim3 g8((unsigned)(8 * ((mt * ntl + 7) / 8))), b8(64 * T::NW);
        if (idx)
            hipLaunchKernelGGL(k_gemm_q8s<true>, g8, b8, 0, s, A, lda, Bq, ldq, scale, idx, ldidx, M, N, kk,
                               group_rows, Y, ydt, ldy, mt, ntl);
        else
            hipLaunchKernelGGL(k_gemm_q8s<false>, g8, b8, 0, s, A, lda, Bq, ldq, scale, idx, ldidx, M, N, kk,
                               group_rows, Y, ydt, ldy, mt, ntl);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)(8 * ((total + 7) / 8))), block(64 * S::NW);
    if (idx)
        hipLaunchKernelGGL(k_gemm_q8<true>, grid, block, 0, s, A, lda, Bq, ldq, scale, idx, ldidx, M, N, kk,
                           group_rows, Y, ydt, ldy, tiles_per_group, m_tiles, n_tiles, ksplit, part_ws, arrivals);
    else
        hipLaunchKernelGGL(k_gemm_q8<false>, grid, block, 0, s, A, lda, Bq, ldq, scale, idx, ldidx, M, N, kk,
                           group_rows, Y, ydt, ldy, tiles_per_group, m_tiles, n_tiles, ksplit, part_ws, arrivals);
    return hipGetLastError();
}

}  // namespace rmm
