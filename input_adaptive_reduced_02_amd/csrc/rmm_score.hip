// rmm_score.hip -- scoring kernels of the RMM hot path (gfx950).
//
// The score of contraction slice k for a group of rows is the activation
// column norm ||A[rows, k]||_2 ("Reduced Matrix Multiplication..." technical
// summary, Metodologia > Estrategia de Selecao), multiplied in this library
// by the weight row norm ||B[k, :]||_2.  For P.V the score of key k for a
// query block is the block's column mass of P times ||V[k, :]||_2 (reduction
// of the token dimension of PV, Metodologia > Escopo de Aplicacao).
//
// All three kernels are HBM-bound streams.  Each lane owns whole sums and
// adds its terms in ascending index order in binary64 (squares of bf16 and
// binary32 values are exact in binary64, and fma(x, x, acc) rounds once, the
// same as acc + x*x with an exact product), then takes a correctly rounded
// sqrt and rounds the score once to binary32.  Coalescing comes from
// neighbouring lanes owning neighbouring columns (colscore) or from wide
// per-lane loads of contiguous rows (rownorms, pv_score).
#include "rmm_internal.h"

namespace rmm {

// ------------------------------------------------------------------ B row norms
// One lane per row; the row is read in 16-byte vectors, summed left to right.
template <int DT>
__global__ void __launch_bounds__(256)
k_rownorms(const void *__restrict__ Bv, int64_t K, int64_t N, int64_t ldb, double *__restrict__ out)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= K) return;
    double acc = 0.0;
    if (DT == 1) {
        const uint16_t *row = (const uint16_t *)Bv + k * ldb;
        int64_t n = 0;
        for (; n + 32 <= N; n += 32) {
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *(const uint4 *)(row + n + 8 * u);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    double lo = bf16_lo(w[i]), hi = bf16_hi(w[i]);
                    acc = __builtin_fma(lo, lo, acc);
                    acc = __builtin_fma(hi, hi, acc);
                }
            }
        }
        for (; n < N; ++n) {
            double x = bf16_to_f32(row[n]);
            acc = __builtin_fma(x, x, acc);
        }
    } else {
        const float *row = (const float *)Bv + k * ldb;
        int64_t n = 0;
        for (; n + 4 <= N; n += 4) {
            float4 v = *(const float4 *)(row + n);
            double x0 = v.x, x1 = v.y, x2 = v.z, x3 = v.w;
            acc = __builtin_fma(x0, x0, acc);
            acc = __builtin_fma(x1, x1, acc);
            acc = __builtin_fma(x2, x2, acc);
            acc = __builtin_fma(x3, x3, acc);
        }
        for (; n < N; ++n) {
            double x = row[n];
            acc = __builtin_fma(x, x, acc);
        }
    }
    out[k] = __builtin_sqrt(acc);
}

hipError_t launch_rownorms(const void *B, int dt, int64_t K, int64_t N, int64_t ldb, double *out,
                           hipStream_t s)
{
    dim3 grid((unsigned)((K + 255) / 256));
    if (dt == 1)
        hipLaunchKernelGGL(k_rownorms<1>, grid, dim3(256), 0, s, B, K, N, ldb, out);
    else
        hipLaunchKernelGGL(k_rownorms<0>, grid, dim3(256), 0, s, B, K, N, ldb, out);
    return hipGetLastError();
}

// ------------------------------------------------------------------ column scores
// Grid (ceil(K / 128), G), 128 lanes per workgroup; each lane owns one column
// of one group and walks the group's rows top to bottom, the loads of up to
// kColUnroll rows in flight (consecutive lanes read consecutive columns, so
// every row load of a wave is one coalesced 128- or 256-byte segment).
constexpr int kColUnroll = 64;
constexpr int kColThreads = 128;

template <int DT>
__device__ __forceinline__ double load_elem(const void *p, int64_t i)
{
    if (DT == 1) return (double)bf16_to_f32(((const uint16_t *)p)[i]);
    return (double)((const float *)p)[i];
}

template <int DT>
__global__ void __launch_bounds__(kColThreads)
k_colscore(const void *__restrict__ Av, int64_t M, int64_t K, int64_t lda,
           const double *__restrict__ bnorm, int64_t gr, float *__restrict__ scores)
{
    const int64_t g = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * kColThreads + threadIdx.x;
    if (c >= K) return;
    const int64_t r0 = g * gr;
    const int64_t rows = (M - r0 < gr) ? (M - r0) : gr;
    const char *p = (const char *)Av + (r0 * lda + c) * (DT == 1 ? 2 : 4);
    const int64_t ld = lda * (DT == 1 ? 2 : 4);   // row stride in bytes
    double a = 0.0;
    int64_t m = 0;
    for (; m + kColUnroll <= rows; m += kColUnroll) {
        double x[kColUnroll];
#pragma unroll
        for (int u = 0; u < kColUnroll; ++u) x[u] = load_elem<DT>(p + (m + u) * ld, 0);
#pragma unroll
        for (int u = 0; u < kColUnroll; ++u) a = __builtin_fma(x[u], x[u], a);
    }
    for (; m < rows; ++m) {
        const double x = load_elem<DT>(p + m * ld, 0);
        a = __builtin_fma(x, x, a);
    }
    const double b = bnorm ? bnorm[c] : 1.0;
    scores[g * K + c] = (float)(__builtin_sqrt(a) * b);
}

hipError_t launch_colscore(const void *A, int dt, int64_t M, int64_t K, int64_t lda,
                           const double *bnorm, int64_t group_rows, float *scores, hipStream_t s)
{
    const int64_t G = (M + group_rows - 1) / group_rows;
    dim3 grid((unsigned)((K + kColThreads - 1) / kColThreads), (unsigned)G);
    if (dt == 1)
        hipLaunchKernelGGL(k_colscore<1>, grid, dim3(kColThreads), 0, s, A, M, K, lda, bnorm, group_rows,
                           scores);
    else
        hipLaunchKernelGGL(k_colscore<0>, grid, dim3(kColThreads), 0, s, A, M, K, lda, bnorm, group_rows,
                           scores);
    return hipGetLastError();
}

// ------------------------------------------------------------------ P.V scores
// ||V[h][k][:]||_2 for every key (head dimension 128): one wave per 64 keys.
// The 64 rows (16 KiB) arrive with coalesced 16-byte loads (one 1 KiB run,
// four rows, per instruction) and pass through LDS, so that lane l then sums
// row l's squares in ascending d in binary64 (exact squares, one rounding per
// fma) -- the sequential order.  Rows are staged 272 bytes apart, so the 16
// lanes of one ds_read_b128 phase touch distinct banks.
constexpr int kVnPitch = 272;

__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ void __launch_bounds__(256)
k_pv_vnorm(const uint16_t *__restrict__ V, int64_t HL, double *__restrict__ vnorm)
{
    __shared__ __attribute__((aligned(16))) unsigned char st[4][64 * kVnPitch];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * 64;   // this wave's first key
    if (r0 >= HL) return;                                        // no workgroup barrier below
    unsigned char *s = st[wave];
    u32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        int64_t row = r0 + 4 * i + (lane >> 4);
        if (row > HL - 1) row = HL - 1;
        v[i] = *(const u32x4 *)(V + row * 128 + 8 * (lane & 15));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) *(u32x4 *)(s + (4 * i + (lane >> 4)) * kVnPitch + 16 * (lane & 15)) = v[i];
    wave_lds_fence();
    const int64_t row = r0 + lane;
    if (row >= HL) return;
    double vv = 0.0;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const u32x4 w = *(const u32x4 *)(s + lane * kVnPitch + 16 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double lo = bf16_lo(w[i]), hi = bf16_hi(w[i]);
            vv = __builtin_fma(lo, lo, vv);
            vv = __builtin_fma(hi, hi, vv);
        }
    }
    vnorm[row] = __builtin_sqrt(vv);
}

// Block masses times V norms.  Work item = (head h, query block g, 64 keys
// k0 .. k0+63 of the block's candidate keys): uniform in size whatever the
// causal prefix length.  Items of a head are numbered block by block; with a
// causal mask block g holds ceil(K_g / 64) = 2(g+1) items (all blocks but the
// last full when L is a multiple of 128), so item i of a head lies in the
// block g with g(g+1) <= i < (g+1)(g+2).
//
// Persistent waves walk the items with a grid stride, visiting them in the
// scattered order (i * perm) mod total (perm coprime to total) so that the
// items in flight at one time belong to many blocks and heads.  For an item
// the wave reads the 64 key-major segments Pt[h][k][q0 .. q0+128) (256 B
// each) with 16-byte loads that cover four whole segments per instruction;
// the segments then pass through a small LDS slice half by half (queries
// 0..63, then 64..127) so that lane l can sum segment l in binary64 -- eight
// partial sums (query mod 8), each in ascending q, added pairwise, the order
// the attention producer uses for the same scores -- and write
// (float)(mass * ||V_k||).  The loads of the next item are issued before the
// current item is summed.  They carry the non-temporal policy: every segment
// is read once (H = 32: the scoring step 140.3 -> 127.4 us at L = 4096, 1954
// -> 1818 us at L = 16384, identical scores).  Items that are not full (a short last query block
// or a prefix ending inside the 64 keys) take a plain per-lane path.
constexpr int kPvPitch = 144;   // bytes per staged half segment: 128 + 16 (rows on distinct banks)

struct PvItem {
    int64_t h, g, k0, q0, nq, Kg;
    bool full;
};

__device__ __forceinline__ PvItem pv_item(int64_t it, int64_t L, int64_t qb, int causal, int64_t G,
                                          int64_t per_head)
{
    PvItem r;
    r.h = it / per_head;
    const int64_t rem = it - r.h * per_head;
    const int64_t cpb = (L + 63) / 64;
    if (causal) {
        int64_t g = (int64_t)((__builtin_sqrtf(4.0f * (float)rem + 1.0f) - 1.0f) * 0.5f);
        while (g > 0 && g * (g + 1) > rem) --g;
        while ((g + 1) * (g + 2) <= rem) ++g;
        if (g > G - 1) g = G - 1;
        r.g = g;
        r.k0 = (rem - g * (g + 1)) * 64;
    } else {
        r.g = rem / cpb;
        r.k0 = (rem - r.g * cpb) * 64;
    }
    r.q0 = r.g * qb;
    r.nq = (L - r.q0 < qb) ? (L - r.q0) : qb;
    r.Kg = causal ? ((r.q0 + qb < L) ? r.q0 + qb : L) : L;
    r.full = r.nq == 128 && r.k0 + 64 <= r.Kg;
    return r;
}

__global__ void __launch_bounds__(256)
k_pv_mass(const uint16_t *__restrict__ Pt, int64_t H, int64_t L, int64_t qblock, int causal,
          const double *__restrict__ vnorm, float *__restrict__ scores, int64_t per_head, int64_t perm)
{
    __shared__ __attribute__((aligned(16))) unsigned char seg[4][64 * kPvPitch + 64 * 16];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t G = (L + qblock - 1) / qblock;
    const int64_t total = H * per_head;
    const int64_t stride = (int64_t)gridDim.x * 4;
    unsigned char *sw = seg[w];
    const int c = lane & 15;
    // staging destinations: lanes holding chunks 0..7 write them in the first
    // half, the others in the second; the lanes not writing a half store to
    // a private dummy slot (never read), so every store is wave-wide
    unsigned char *real = sw + (lane >> 4) * kPvPitch + 16 * (c & 7);
    unsigned char *dummy = sw + 64 * kPvPitch + 16 * lane;
    const int step0 = (c < 8) ? 4 * kPvPitch : 0, step1 = (c < 8) ? 0 : 4 * kPvPitch;
    unsigned char *d0 = (c < 8) ? real : dummy, *d1 = (c < 8) ? dummy : real;
    auto wave_sync = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    int64_t it = (int64_t)blockIdx.x * 4 + w;
    u32x4 v[16];
    PvItem cur{};
    if (it < total) {
        cur = pv_item(it * perm % total, L, qblock, causal, G, per_head);
        if (cur.full) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                v[i] = __builtin_nontemporal_load((const u32x4 *)(Pt + (cur.h * L + cur.k0 + 4 * i + (lane >> 4)) * L + cur.q0 + 8 * c));
        }
    }
    while (it < total) {
        const int64_t nx = it + stride;
        PvItem nxt{};
        if (nx < total) nxt = pv_item(nx * perm % total, L, qblock, causal, G, per_head);
        const int64_t k = cur.k0 + lane;
        double m8[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};   // partial sums, query mod 8
        if (cur.full) {
            u32x4 hi[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                *(u32x4 *)(d0 + i * step0) = v[i];
                hi[i] = v[i];
            }
            // the registers are free: start the next item's loads now
            if (nx < total && nxt.full) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    v[i] = __builtin_nontemporal_load((const u32x4 *)(Pt + (nxt.h * L + nxt.k0 + 4 * i + (lane >> 4)) * L + nxt.q0 + 8 * c));
            }
            const unsigned char *row = sw + lane * kPvPitch;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                if (half == 1) {
                    wave_sync();   // every lane has read the first half
#pragma unroll
                    for (int i = 0; i < 16; ++i) *(u32x4 *)(d1 + i * step1) = hi[i];
                }
                wave_sync();       // the slice was written by other lanes of this wave
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const u32x4 x = *(const u32x4 *)(row + 16 * j);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        m8[2 * e] += (double)bf16_lo(x[e]);
                        m8[2 * e + 1] += (double)bf16_hi(x[e]);
                    }
                }
            }
            wave_sync();           // every lane has read the slice before the next item
        } else {
            if (k < cur.Kg) {
                const uint16_t *src = Pt + (cur.h * L + k) * L + cur.q0;
                for (int64_t i = 0; i < cur.nq; ++i) m8[i & 7] += (double)bf16_to_f32(src[i]);
            }
            if (nx < total && nxt.full) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    v[i] = __builtin_nontemporal_load((const u32x4 *)(Pt + (nxt.h * L + nxt.k0 + 4 * i + (lane >> 4)) * L + nxt.q0 + 8 * c));
            }
        }
        const double mass = ((m8[0] + m8[1]) + (m8[2] + m8[3])) + ((m8[4] + m8[5]) + (m8[6] + m8[7]));
        if (k < cur.Kg) scores[(cur.h * G + cur.g) * L + k] = (float)(mass * vnorm[cur.h * L + k]);
        cur = nxt;
        it = nx;
    }
}

hipError_t launch_pv_vnorm(const uint16_t *V, int64_t H, int64_t L, int64_t D, double *vnorm, hipStream_t s)
{
    if (D != 128) return hipErrorInvalidValue;   // the callers take D == 128 only
    const int64_t HL = H * L;
    hipLaunchKernelGGL(k_pv_vnorm, dim3((unsigned)((HL + 255) / 256)), dim3(256), 0, s, V, HL, vnorm);
    return hipGetLastError();
}

hipError_t launch_pv_score(const uint16_t *Pt, const uint16_t *V, int64_t H, int64_t L, int64_t D,
                           int64_t qblock, int causal, double *vnorm, float *scores, hipStream_t s)
{
    if (hipError_t e = launch_pv_vnorm(V, H, L, D, vnorm, s)) return e;
    const int64_t G = (L + qblock - 1) / qblock;
    const int64_t cpb = (L + 63) / 64;
    // items per head: causal blocks hold 2(g+1) items, the last ceil(L/64) - 2(G-1)
    const int64_t per_head = causal ? (G - 1) * G + cpb : G * cpb;
    const int64_t total = H * per_head;
    int64_t blocks = (total + 3) / 4;
    if (blocks > 1024) blocks = 1024;   // four 4-wave workgroups per CU (41 KiB of LDS each), persistent
    // a prime coprime to the item count (item indices times it stay below 2^63)
    int64_t perm = 1;
    for (int64_t p : {1000003LL, 999983LL, 999979LL, 999961LL})
        if (total % p != 0) {
            perm = p % total;
            break;
        }
    if (perm == 0) perm = 1;
    hipLaunchKernelGGL(k_pv_mass, dim3((unsigned)blocks), dim3(256), 0, s, Pt, H, L, qblock, causal, vnorm, scores,
                       per_head, perm);
    return hipGetLastError();
}

}  // namespace rmm
