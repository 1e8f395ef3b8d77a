// rmm_select.hip -- per-group top-k selection of the RMM hot path (gfx950).
//
// Keeps the kk best-scored contraction slices of a group ("Reduced Matrix
// Multiplication..." technical summary, Metodologia > Estrategia de Selecao:
// keep the top ceil(rho d) scores), ties going to the lower index, and writes
// the kept indices in ascending order.
//
// One 1024-thread workgroup per group.  Scores are non-negative binary32, so
// their bit patterns, read as int32, order like the values.  Thread t holds
// the keys of the contiguous index range [t*kpt, (t+1)*kpt) in registers.
//   1. Threshold T = the kk-th largest key, found bit by bit from the top, two
//      bits per round: the three candidate prefixes are counted at once with
//      wavefront ballots and scalar popcounts, then summed over the 16 waves
//      through LDS (16 rounds, one barrier each).
//   2. Ordered compaction: per-wave exclusive counts of keys > T and == T come
//      from ballots masked to the lower lanes (mbcnt), per-wave totals from one
//      LDS exchange; every thread then knows its output position, and keys
//      == T are kept in index order until kk is reached.
// No atomics anywhere, so the output is deterministic.
#include "rmm_internal.h"

namespace rmm {

// Sum of a wave-uniform value over the workgroup's 16 waves; every thread
// gets the result.  `slot` is one of two alternating LDS rows, so consecutive
// calls need a single barrier each.
__device__ __forceinline__ uint64_t block_sum_uniform(uint64_t v, uint64_t *slot)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) slot[wave] = v;
    __syncthreads();
    uint64_t s = 0;
#pragma unroll
    for (int w = 0; w < kSelectThreads / 64; ++w) s += slot[w];
    return s;
}

template <int KPT>
__global__ void __launch_bounds__(kSelectThreads)
k_select(const float *__restrict__ scores, SelectShape sh, int32_t *__restrict__ idx, int64_t ldidx,
         float *__restrict__ thresh, double *__restrict__ bound)
{
    constexpr int NW = kSelectThreads / 64;
    __shared__ uint64_t red[2][NW];
    __shared__ uint64_t wsum[NW];
    __shared__ double fsum[NW];
    __shared__ int32_t s_last;

    const int64_t grp = blockIdx.x;
    int64_t K, kk;
    if (sh.pv) {
        const int64_t g = grp % sh.Gq;
        K = sh.causal ? ((sh.qblock * (g + 1) < sh.K) ? sh.qblock * (g + 1) : sh.K) : sh.K;
        kk = kk_rule(sh.r, K);
    } else {
        K = sh.K;
        kk = sh.kk;
    }
    const float *s = scores + grp * sh.lds;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) s_last = 0;   // written again (by the kk-th keeper) after several barriers
    const int kpt = (int)((K + kSelectThreads - 1) / kSelectThreads);
    const int64_t base = (int64_t)tid * kpt;

    int32_t key[KPT];  // -1 marks "no key here"; real keys are >= 0
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int64_t k = base + i;
        key[i] = (i < kpt && k < K) ? __float_as_int(s[k]) : -1;
    }

    // ---- 1. threshold search
    int32_t T = 0;
    int round = 0;
    for (int sh2 = 29; sh2 >= 1; sh2 -= 2, ++round) {
        const int32_t c1 = T | (1 << sh2), c2 = T | (2 << sh2), c3 = T | (3 << sh2);
        uint32_t n1 = 0, n2 = 0, n3 = 0;   // wave-uniform counts
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            n1 += __popcll(__ballot(key[i] >= c1));
            n2 += __popcll(__ballot(key[i] >= c2));
            n3 += __popcll(__ballot(key[i] >= c3));
        }
        const uint64_t tot = block_sum_uniform((uint64_t)n1 | ((uint64_t)n2 << 21) | ((uint64_t)n3 << 42),
                                               red[round & 1]);
        const int64_t t1 = tot & 0x1fffff, t2 = (tot >> 21) & 0x1fffff, t3 = tot >> 42;
        const int v = (t3 >= kk) ? 3 : (t2 >= kk) ? 2 : (t1 >= kk) ? 1 : 0;
        T |= v << sh2;
    }
    {
        const int32_t c1 = T | 1;
        uint32_t n1 = 0;
#pragma unroll
        for (int i = 0; i < KPT; ++i) n1 += __popcll(__ballot(key[i] >= c1));
        const uint64_t tot = block_sum_uniform(n1, red[round & 1]);
        if ((int64_t)tot >= kk) T = c1;
    }

    // ---- 2. ordered compaction
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes < this one
    uint32_t gt_w = 0, eq_w = 0, gt_tot_w = 0, eq_tot_w = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const uint64_t bg = __ballot(key[i] > T), be = __ballot(key[i] == T);
        gt_w += __popcll(bg & below);
        eq_w += __popcll(be & below);
        gt_tot_w += __popcll(bg);
        eq_tot_w += __popcll(be);
    }
    if (lane == 0) wsum[wave] = ((uint64_t)gt_tot_w << 32) | eq_tot_w;
    __syncthreads();
    uint64_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint64_t x = wsum[w];
        before += (w < wave) ? x : 0;
        total += x;
    }
    const int64_t gt_before = (int64_t)(before >> 32) + gt_w;
    const int64_t eq_before = (int64_t)(before & 0xffffffffu) + eq_w;
    const int64_t need_eq = kk - (int64_t)(total >> 32);  // >= 1 by the choice of T
    int64_t pos = gt_before + (eq_before < need_eq ? eq_before : need_eq);
    int64_t eq_seen = eq_before;
    int32_t *out = idx + grp * ldidx;
    double dropped = 0.0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        if (key[i] < 0) continue;
        const int32_t k = (int32_t)(base + i);
        bool keep = key[i] > T;
        if (key[i] == T) {
            keep = eq_seen < need_eq;
            ++eq_seen;
        }
        if (keep) {
            if (pos < kk) out[pos] = k;   // always true when T is the kk-th key
            if (pos == kk - 1) s_last = k;
            ++pos;
        } else {
            dropped += (double)__int_as_float(key[i]);
        }
    }
    if (tid == 0 && thresh) thresh[grp] = __int_as_float(T);
    if (bound) {
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) dropped += __shfl_xor(dropped, m, 64);
        if (lane == 0) fsum[wave] = dropped;
    }
    __syncthreads();
    const int64_t padded = pad_up(kk);
    for (int64_t j = kk + tid; j < padded; j += kSelectThreads) out[j] = s_last;
    if (bound && tid == 0) {
        double b = 0.0;
        for (int w = 0; w < NW; ++w) b += fsum[w];
        bound[grp] = b;
    }
}

hipError_t launch_select(const float *scores, const SelectShape &sh, int32_t *idx, int64_t ldidx,
                         float *thresh, double *bound, hipStream_t s)
{
    dim3 grid((unsigned)sh.groups), block(kSelectThreads);
    if (sh.K <= 4 * kSelectThreads)
        hipLaunchKernelGGL(k_select<4>, grid, block, 0, s, scores, sh, idx, ldidx, thresh, bound);
    else if (sh.K <= 16 * kSelectThreads)
        hipLaunchKernelGGL(k_select<16>, grid, block, 0, s, scores, sh, idx, ldidx, thresh, bound);
    else
        hipLaunchKernelGGL(k_select<32>, grid, block, 0, s, scores, sh, idx, ldidx, thresh, bound);
    return hipGetLastError();
}

}  // namespace rmm
