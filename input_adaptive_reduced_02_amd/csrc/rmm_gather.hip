// rmm_gather.hip -- compaction of the kept slices into bf16 panels (gfx950).
//
// Forms the columns A[:, I] of the reduced product A[:, I] B[I, :]
// ("Reduced Matrix Multiplication..." technical summary, Metodologia >
// Mecanismo Central) as a dense, zero-padded bf16 panel the GEMM streams with
// plain 16-byte loads.  Optionally packs the kept rows B[I, :] as well (single
// group only; the GEMM otherwise reads kept B rows in place by index).
//
// HBM-bound data movement.  Picking 2-byte elements straight out of global
// memory costs the load units a cache-line access per element, so whole rows
// of A are first copied into LDS with coalesced 16-byte loads (a workgroup
// stages about 8 KiB of rows, a single row up to 32 KiB), then every thread
// picks 8 kept elements of a row out of LDS by index and writes them as one
// 16-byte panel chunk.  The global traffic is exactly one read of A and one
// write of the panel.
#include "rmm_internal.h"

namespace rmm {

template <int DT>
__global__ void __launch_bounds__(256)
k_gather_a(const void *__restrict__ Av, int64_t M, int64_t lda, const int32_t *__restrict__ idx,
           int64_t ldidx, int64_t kk, int64_t gr, uint16_t *__restrict__ Ap, int64_t ldp,
           int64_t chunks_per_row)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t m = t / chunks_per_row;
    const int64_t j0 = (t % chunks_per_row) * 8;
    if (m >= M) return;
    const int32_t *I = idx + (m / gr) * ldidx;
    uint32_t h[8];
    if (j0 + 8 <= kk) {
        const int4 i0 = *(const int4 *)(I + j0);
        const int4 i1 = *(const int4 *)(I + j0 + 4);
        const int32_t ks[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
        if (DT == 1) {
            const uint16_t *row = (const uint16_t *)Av + m * lda;
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = row[ks[e]];
        } else {
            const float *row = (const float *)Av + m * lda;
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = f32_to_bf16(row[ks[e]]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t j = j0 + e;
            h[e] = 0;
            if (j < kk) {
                const int32_t k = I[j];
                if (DT == 1)
                    h[e] = ((const uint16_t *)Av)[m * lda + k];
                else
                    h[e] = f32_to_bf16(((const float *)Av)[m * lda + k]);
            }
        }
    }
    uint4 o = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    *(uint4 *)(Ap + m * ldp + j0) = o;
}

constexpr int kGatherLds = 32768;   // longest A row (bytes) staged in LDS
constexpr int kGatherIdx = 4;       // panel chunks per thread whose indices are loaded ahead

// DMA: every lane copies 16 bytes from its global address to LDS[m0 + 16*lane]
__device__ __forceinline__ void gather_dma16(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

// One workgroup per `rpw` consecutive rows.  The rows go to LDS by DMA in
// 1 KiB blocks, every block of the workgroup in flight at once (wave w issues
// blocks w, w + 4, ...; lanes past a row's last 16-byte chunk re-read the
// row's start into staging space no pick reads).  While they land, every
// thread loads the kept indices of its first panel chunks into registers.
// Then thread t writes panel chunks t, t + 256, ... of every row, picking the
// 8 kept elements of a chunk out of LDS.  A row's chunks all lie inside its
// leading dimension (lda * es is a multiple of 16 and K <= lda).
template <int DT>
__global__ void __launch_bounds__(256)
k_gather_rows(const void *__restrict__ Av, int64_t M, int64_t K, int64_t lda, const int32_t *__restrict__ idx,
              int64_t ldidx, int64_t kk, int64_t gr, uint16_t *__restrict__ Ap, int64_t ldp, int rpw,
              int row_bytes)
{
    extern __shared__ __attribute__((aligned(1024))) unsigned char stage[];
    constexpr int ES = DT == 1 ? 2 : 4;
    const int64_t m0 = (int64_t)blockIdx.x * rpw;
    const int nrow = (int)((M - m0 < rpw) ? (M - m0) : rpw);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int chunks = (int)((K * ES + 15) / 16);   // 16-byte chunks of a row holding its K elements
    const int blocks = (chunks + 63) / 64;          // 1 KiB DMA blocks per row
    const uint32_t st0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)stage;
    for (int b = wave; b < nrow * blocks; b += 4) {
        const int r = b / blocks, c = (b % blocks) * 64 + lane;
        const unsigned char *src = (const unsigned char *)Av + (m0 + r) * lda * ES;
        gather_dma16(c < chunks ? src + 16 * c : src, st0 + r * row_bytes + (b % blocks) * 1024);
    }
    // indices of this thread's first chunks of the first row's group (a
    // workgroup's rows may span two groups; the others load theirs below)
    const int64_t cpr = pad_up(kk) / 8;
    const int32_t *I0 = idx + (m0 / gr) * ldidx;
    int4 ia[kGatherIdx], ib[kGatherIdx];
#pragma unroll
    for (int q = 0; q < kGatherIdx; ++q) {
        const int64_t j0 = (int64_t)(tid + 256 * q) * 8;
        ia[q] = ib[q] = int4{0, 0, 0, 0};
        if (j0 + 8 <= kk) {
            ia[q] = *(const int4 *)(I0 + j0);
            ib[q] = *(const int4 *)(I0 + j0 + 4);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // panel chunk j0/8 of staged row `row`, its indices given (full chunks) or
    // read from I (the chunk that reaches kk)
    auto pick = [&](const unsigned char *row, const int32_t *I, int64_t j0, int4 i0, int4 i1, uint16_t *out) {
        uint32_t h[8];
        if (j0 + 8 <= kk) {
            const int32_t ks[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                h[e] = DT == 1 ? ((const uint16_t *)row)[ks[e]] : f32_to_bf16(((const float *)row)[ks[e]]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                h[e] = 0;
                if (j0 + e < kk) {
                    const int32_t k = I[j0 + e];
                    h[e] = DT == 1 ? ((const uint16_t *)row)[k] : f32_to_bf16(((const float *)row)[k]);
                }
            }
        }
        // streaming store: the panel is read next by the GEMM on other CUs
        const u32x4 o = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        __builtin_nontemporal_store(o, (u32x4 *)(out + j0));
    };
    for (int r = 0; r < nrow; ++r) {
        const int64_t m = m0 + r;
        const int32_t *I = idx + (m / gr) * ldidx;
        const bool same = (m / gr) == (m0 / gr);
        const unsigned char *row = stage + r * row_bytes;
        uint16_t *out = Ap + m * ldp;
#pragma unroll
        for (int q = 0; q < kGatherIdx; ++q) {
            const int64_t j0 = (int64_t)(tid + 256 * q) * 8;
            if (j0 >= cpr * 8) break;
            int4 i0 = ia[q], i1 = ib[q];
            if (!same && j0 + 8 <= kk) {
                i0 = *(const int4 *)(I + j0);
                i1 = *(const int4 *)(I + j0 + 4);
            }
            pick(row, I, j0, i0, i1, out);
        }
        for (int64_t c = tid + 256 * kGatherIdx; c < cpr; c += 256) {
            const int64_t j0 = c * 8;
            int4 i0 = {0, 0, 0, 0}, i1 = {0, 0, 0, 0};
            if (j0 + 8 <= kk) {
                i0 = *(const int4 *)(I + j0);
                i1 = *(const int4 *)(I + j0 + 4);
            }
            pick(row, I, j0, i0, i1, out);
        }
    }
}

// Bp[j][:] = bf16(B[idx[j]][:]) for j < kk, zero for kk <= j < kpad.
template <int DT>
__global__ void __launch_bounds__(256)
k_gather_b(const void *__restrict__ Bv, int64_t N, int64_t ldb, const int32_t *__restrict__ idx,
           int64_t kk, int64_t kpad, uint16_t *__restrict__ Bp, int64_t ldbp, int64_t chunks_per_row)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t j = t / chunks_per_row;
    const int64_t n0 = (t % chunks_per_row) * 8;
    if (j >= kpad) return;
    uint4 o = make_uint4(0, 0, 0, 0);
    if (j < kk) {
        const int64_t k = idx[j];
        if (DT == 1) {
            o = *(const uint4 *)((const uint16_t *)Bv + k * ldb + n0);
        } else {
            const float *row = (const float *)Bv + k * ldb + n0;
            const float4 a = *(const float4 *)row, b = *(const float4 *)(row + 4);
            o = make_uint4(f32_to_bf16(a.x) | (f32_to_bf16(a.y) << 16), f32_to_bf16(a.z) | (f32_to_bf16(a.w) << 16),
                           f32_to_bf16(b.x) | (f32_to_bf16(b.y) << 16), f32_to_bf16(b.z) | (f32_to_bf16(b.w) << 16));
        }
    }
    *(uint4 *)(Bp + j * ldbp + n0) = o;
}

hipError_t launch_gather(const void *A, int dt, int64_t M, int64_t K, int64_t lda, const int32_t *idx,
                         int64_t ldidx, int64_t kk, int64_t group_rows, uint16_t *Ap, int64_t ldp,
                         const void *B, int64_t N, int64_t ldb, uint16_t *Bp, int64_t ldbp,
                         hipStream_t s)
{
    const int64_t kpad = pad_up(kk);
    const int64_t cpr = kpad / 8;
    // staged row size: whole 1 KiB DMA blocks
    const int64_t row_bytes = (K * (dt == 1 ? 2 : 4) + 1023) / 1024 * 1024;
    if (row_bytes <= kGatherLds) {
        // rows per workgroup: about 8 KiB of rows, so that many small
        // workgroups overlap one another's load and write phases on a CU
        int rpw = (int)(8192 / row_bytes);
        if (rpw > 8) rpw = 8;
        if (rpw < 1) rpw = 1;
        const unsigned blocks = (unsigned)((M + rpw - 1) / rpw);
        const size_t lds = (size_t)rpw * row_bytes;
        if (dt == 1)
            hipLaunchKernelGGL(k_gather_rows<1>, dim3(blocks), dim3(256), lds, s, A, M, K, lda, idx, ldidx, kk,
                               group_rows, Ap, ldp, rpw, (int)row_bytes);
        else
            hipLaunchKernelGGL(k_gather_rows<0>, dim3(blocks), dim3(256), lds, s, A, M, K, lda, idx, ldidx, kk,
                               group_rows, Ap, ldp, rpw, (int)row_bytes);
    } else {
        const int64_t threads = M * cpr;
        dim3 grid((unsigned)((threads + 255) / 256));
        if (dt == 1)
            hipLaunchKernelGGL(k_gather_a<1>, grid, dim3(256), 0, s, A, M, lda, idx, ldidx, kk, group_rows, Ap, ldp,
                               cpr);
        else
            hipLaunchKernelGGL(k_gather_a<0>, grid, dim3(256), 0, s, A, M, lda, idx, ldidx, kk, group_rows, Ap, ldp,
                               cpr);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !Bp) return e;
    const int64_t cb = N / 8;
    dim3 gb((unsigned)((kpad * cb + 255) / 256));
    if (dt == 1)
        hipLaunchKernelGGL(k_gather_b<1>, gb, dim3(256), 0, s, B, N, ldb, idx, kk, kpad, Bp, ldbp, cb);
    else
        hipLaunchKernelGGL(k_gather_b<0>, gb, dim3(256), 0, s, B, N, ldb, idx, kk, kpad, Bp, ldbp, cb);
    return hipGetLastError();
}

}  // namespace rmm
