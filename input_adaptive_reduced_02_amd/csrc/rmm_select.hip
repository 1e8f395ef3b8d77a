// rmm_select.hip -- per-group top-k selection of the RMM hot path (gfx950).
//
// Keeps the kk best-scored contraction slices of a group ("Reduced Matrix
// Multiplication..." technical summary, Metodologia > Estrategia de Selecao:
// keep the top ceil(rho d) scores), ties going to the lower index, and writes
// the kept indices in ascending order.
//
// One 1024-thread workgroup per group; thread t holds the keys of the
// contiguous index range [t*kpt, (t+1)*kpt) in registers.  Scores are
// non-negative binary32, so their bit patterns, read as int32, order like the
// values.  The threshold T (the kk-th largest key) is found in two steps:
//   1. Bit-pattern histogram: with lo, hi the group's smallest and largest
//      key, key u goes to bucket (u - lo) >> b, 2^b the narrowest power-of-two
//      width for which 2048 buckets cover hi - lo.  The shift is monotone, so
//      the bucket index never decreases as u grows and equal keys share a
//      bucket: the kk-th largest key lies in the bucket where the count from
//      the top reaches kk.
//      Buckets even in the bit pattern are roughly even in log(score), so
//      outlier channels do not crowd the bulk of the scores into a few
//      buckets; the LDS atomics rarely collide and the threshold's bucket
//      holds few keys.
//   2. The bucket's keys are copied to LDS (in any order, places reserved by
//      one LDS atomic per wave and key slot) and T is found among them: up to
//      64 candidates by exact rank, up to 1024 bit by bit, two bits per round
//      (three candidate prefixes counted with wavefront ballots) starting
//      below the high bits the smallest and largest candidate share (T lies
//      between them).  Every wave does this on its own, with the candidates
//      in registers, so no barrier broadcasts T; beyond 1024 candidates all
//      16 waves share the search through LDS.
// Then the ordered compaction: each thread counts its keys > T and == T, a
// prefix sum over the wave and one LDS exchange of the wave totals place its
// kept keys; keys == T are kept in index order until kk.  Atomics only place
// the candidates in LDS, whose order T does not depend on; no atomic decides
// an output order and no floating-point sum decides anything, so the output
// is deterministic.
//
// Select + gather in one launch (NRB > 0): the group's rows are split over
// `slices` workgroups, each of which runs the whole selection of its group
// (identical, deterministic work) while its own rows of A stream into LDS
// with DMA loads (issued after the histogram, in flight during the rest of
// the selection; issued before the keys arrive they delayed them and were
// slower).  After the threshold and the ordered compaction (kept
// indices into an LDS list) every workgroup picks its rows' kept elements out
// of LDS into the bf16 panel, 8 per lane and one 16-byte store; the first
// slice also writes the index row, threshold and bound.  The panel equals the
// one the separate gather writes from the same index row.
#include "rmm_internal.h"
#include "rmm_select.h"

namespace rmm {

constexpr int kBuckets = 2048;

// Sum of a wave-uniform value over the workgroup's NW waves; every thread gets
// the result.  `slot` is one of two alternating LDS rows, so consecutive calls
// need a single barrier each.
template <int NW>
__device__ __forceinline__ uint64_t block_sum_uniform(uint64_t v, uint64_t *slot)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) slot[wave] = v;
    __syncthreads();
    uint64_t s = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += slot[w];
    return s;
}

__device__ __forceinline__ uint64_t lanes_below(int lane) { return lane == 0 ? 0ull : (~0ull >> (64 - lane)); }

// Inclusive prefix sum over the 64 lanes of a wave, in six cross-lane steps
// (a 16-ballot bit-sliced scan cost about ten times the vector instructions).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(v, d, 64);
        if (lane >= d) v += y;
    }
    return v;
}

// Exclusive prefix sum of a per-thread value over the workgroup of NW waves
// (thread order), plus the total (which must fit 32 bits).
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wtot, uint32_t &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_scan(v, lane);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t x = wtot[w];
        before += (w < wave) ? x : 0;
        total += x;
    }
    return before + incl - v;
}

// Count of candidates >= c1, c2, c3 among cand[i], i in [first, n) step
// `step`, packed 21 bits each; wave-uniform.
__device__ __forceinline__ uint64_t count3(const int32_t *cand, uint32_t first, uint32_t n, uint32_t step,
                                           int32_t c1, int32_t c2, int32_t c3)
{
    uint32_t m1 = 0, m2 = 0, m3 = 0;
    for (uint32_t b0 = 0; b0 < n; b0 += step) {
        const uint32_t i = b0 + first;
        const int32_t v = (i < n) ? cand[i] : -1;
        m1 += __popcll(__ballot(v >= c1));
        m2 += __popcll(__ballot(v >= c2));
        m3 += __popcll(__ballot(v >= c3));
    }
    return (uint64_t)m1 | ((uint64_t)m2 << 21) | ((uint64_t)m3 << 42);
}

// DMA: every lane copies 16 bytes from its global address to LDS[lds + 16*lane]
// (global_load_lds_dwordx4; no register result, so nothing waits for it until
// an explicit s_waitcnt).
__device__ __forceinline__ void sel_dma16(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ uint32_t sel_lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
// NRB = 0: selection only, one workgroup of NT threads per group (1024 for a
// few long groups: latency; 256 for many groups: several workgroups per CU and
// 4-wave barriers).  NRB > 0: selection and gather, `ga.slices` 1024-thread
// workgroups per group, each staging at most NRB 1 KiB blocks of rows per
// wave (16 * NRB KiB per workgroup).
template <int KPT, int NRB, int NT>
__global__ void __launch_bounds__(NT)
k_select(const float *__restrict__ scores, SelectShape sh, int32_t *__restrict__ idx, int64_t ldidx,
         float *__restrict__ thresh, double *__restrict__ bound, SelectGather ga)
{
    constexpr int NW = NT / 64, BPT = kBuckets / NT;   // waves; histogram buckets per thread
    static_assert(NRB == 0 || NT == kSelectThreads, "the fused gather runs 1024-thread workgroups");
    static_assert(BPT >= 2 && kBuckets % NT == 0, "a thread scans whole buckets");
    __shared__ uint32_t hist[kBuckets];
    __shared__ __attribute__((aligned(16))) int32_t cand[KPT * NT];   // later the kept list
    __shared__ __attribute__((aligned(1024))) unsigned char stage[NRB > 0 ? NRB * 16 * 1024 : 16];
    __shared__ uint64_t red[2][NW];
    __shared__ uint64_t wsum64[NW];
    __shared__ uint32_t wtot[NW];
    __shared__ int32_t imin[NW], imax[NW];
    __shared__ double fsum[NW];
    __shared__ int32_t s_bin;
    __shared__ uint32_t s_nc;
    __shared__ int64_t s_above;

    const int64_t grp = NRB > 0 ? blockIdx.x / ga.slices : blockIdx.x;
    const int slice = NRB > 0 ? (int)(blockIdx.x % ga.slices) : 0;
    const bool lead = slice == 0;   // the workgroup that writes idx, thresh and bound
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
    // keys per thread, a multiple of 4 where KPT allows (KPT is a power of
    // two >= the plain quotient), so full runs take 16-byte loads: K = 14336
    // gives 896 threads of 16 keys rather than 1024 of 14 (4-byte loads at a
    // 56-byte lane stride)
    const int kpt0 = (int)((K + NT - 1) / NT);
    const int kpt = KPT >= 4 ? (kpt0 + 3) & ~3 : kpt0;
    const int64_t base = (int64_t)tid * kpt;

    for (int i = tid; i < kBuckets; i += NT) hist[i] = 0;
    if (tid == 0) s_nc = 0;   // candidate count, first added to after two barriers
    int32_t key[KPT];           // -1 marks "no key here"; real keys are >= 0
    int32_t lo = 0x7fffffff, hi = 0;
    if (KPT % 4 == 0 && kpt == KPT && base + KPT <= K && ((uintptr_t)(s + base) & 15u) == 0) {
        // a full, aligned run of keys: 16-byte loads, every key present
#pragma unroll
        for (int i = 0; i < KPT; i += 4) {
            const u32x4 v = *(const u32x4 *)(s + base + i);
#pragma unroll
            for (int e = 0; e < 4; ++e) key[i + e] = (int32_t)v[e];
        }
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            lo = min(lo, key[i]);
            hi = max(hi, key[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int64_t k = base + i;
            key[i] = (i < kpt && k < K) ? __float_as_int(s[k]) : -1;
        }
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            if (key[i] >= 0) {
                lo = min(lo, key[i]);
                hi = max(hi, key[i]);
            }
        }
    }
    // ---- group min / max of the keys
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        lo = min(lo, __shfl_xor(lo, m, 64));
        hi = max(hi, __shfl_xor(hi, m, 64));
    }
    if (lane == 0) {
        imin[wave] = lo;
        imax[wave] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        lo = min(lo, imin[w]);
        hi = max(hi, imax[w]);
    }
    // buckets 2^bsh bit patterns wide, the narrowest power of two that covers
    // hi - lo with kBuckets of them
    const uint32_t span = hi > lo ? (uint32_t)(hi - lo) : 0u;
    const int bits = span ? 32 - __clz(span) : 0;
    const int bsh = bits > 11 ? bits - 11 : 0;
    static_assert(kBuckets == 2048, "bucket widths assume 2^11 buckets");
    auto bucket = [&](int32_t k) -> int { return (int)((uint32_t)(k - lo) >> bsh); };

    // ---- 1. bit-pattern histogram, then the bucket holding the kk-th key
#pragma unroll
    for (int i = 0; i < KPT; ++i)
        if (key[i] >= 0) atomicAdd(&hist[bucket(key[i])], 1u);
    __syncthreads();
    {
        // thread t owns buckets BPT t .. BPT t + BPT - 1 and walks them from
        // the top; exactly one bucket holds the kk-th largest key
        uint32_t h[BPT], mine = 0;
#pragma unroll
        for (int b = 0; b < BPT; ++b) {
            h[b] = hist[BPT * tid + b];
            mine += h[b];
        }
        uint32_t total;
        const uint32_t incl = block_excl_scan<NW>(mine, wtot, total) + mine;
        int64_t above = (int64_t)total - incl;   // keys in buckets above this thread's
#pragma unroll
        for (int b = BPT - 1; b >= 0; --b) {
            if (above < kk && kk <= above + h[b]) {
                s_bin = BPT * tid + b;
                s_above = above;
            }
            above += h[b];
        }
    }
    __syncthreads();
    const int bin = s_bin;
    const int64_t need = kk - s_above;   // how many of the bucket's keys are kept (>= 1)
    // The slice's rows of A into LDS, in flight during the rest of the
    // selection: no compiler-placed wait below is for these loads (the keys
    // have arrived, and the barriers wait for LDS operations only); an
    // explicit wait precedes the pick.  Row i of the slice goes to LDS byte
    // i * lda * 2: the rows are one contiguous global range, copied in 1 KiB
    // blocks (block b by wave b % 16), and lanes past its end re-read its
    // start into block space no row uses.
    int64_t srow0 = 0, sbytes = 0;
    int nrows = 0;
    if constexpr (NRB > 0) {
        const int64_t g0 = grp * ga.gr;
        const int64_t gend = (g0 + ga.gr < ga.M) ? g0 + ga.gr : ga.M;
        srow0 = g0 + (int64_t)slice * ga.rows;
        nrows = (int)((gend - srow0 < ga.rows) ? (gend - srow0 > 0 ? gend - srow0 : 0) : ga.rows);
        sbytes = (int64_t)nrows * ga.lda * 2;
        const char *src = (const char *)ga.A + srow0 * ga.lda * 2;
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        const uint32_t st0 = sel_lds_addr(stage);
#pragma unroll
        for (int i = 0; i < NRB; ++i) {
            const int b = wv + NW * i;
            const int64_t o = (int64_t)b * 1024 + 16 * lane;
            if ((int64_t)b * 1024 < sbytes) sel_dma16(o < sbytes ? src + o : src, st0 + b * 1024);
        }
    }

    // ---- 2. the bucket's keys to LDS, in any order (T depends on their
    // values only): per key slot one wave-aggregated LDS atomic reserves the
    // wave's places.  Then every wave finds T on its own (no broadcast
    // barrier), unless there are more than 1024 candidates.
    const uint64_t below = lanes_below(lane);
    // key k is in the bucket iff 0 <= k - blo < 2^bsh; an absent key (-1) wraps
    // to at least 2^31 as an unsigned difference
    const int32_t blo = lo + (bin << bsh);
    const uint32_t bw = 1u << bsh;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const bool in = (uint32_t)(key[i] - blo) < bw;
        const uint64_t m = __ballot(in);
        if (m) {
            uint32_t at = 0;
            if (lane == 0) at = atomicAdd(&s_nc, (uint32_t)__popcll(m));
            at = __shfl(at, 0, 64);
            if (in) cand[at + __popcll(m & below)] = key[i];
        }
    }
    __syncthreads();
    const uint32_t n1 = s_nc;
    int32_t T = 0;
    if (n1 <= 64) {
        // few candidates: lane i takes candidate i and counts the larger and
        // the equal ones; T is a candidate with #(> T) < need <= #(>= T)
        const int32_t mine = lane < (int)n1 ? cand[lane] : -1;
        uint32_t gt = 0, ge = 0;
        for (uint32_t i = 0; i < n1; ++i) {
            const int32_t x = cand[i];
            gt += x > mine;
            ge += x >= mine;
        }
        const uint64_t hit = __ballot(lane < (int)n1 && gt < need && need <= ge);
        T = __shfl(mine, __builtin_ctzll(hit), 64);   // whole wave active
    } else if (n1 <= 1024) {
        // candidates held in registers (16 slots of 64)
        int32_t c[16];
        int32_t lo = 0x7fffffff, hi = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t i = j * 64 + lane;
            c[j] = (i < n1) ? cand[i] : -1;
            if (c[j] >= 0) {
                lo = min(lo, c[j]);
                hi = max(hi, c[j]);
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            lo = min(lo, __shfl_xor(lo, m, 64));
            hi = max(hi, __shfl_xor(hi, m, 64));
        }
        // lo <= T <= hi, so T shares their common high bits; search the rest
        const int hb = (lo == hi) ? -1 : 31 - __clz(lo ^ hi);
        T = (hb < 0) ? lo : (lo & ~((int32_t)((2u << hb) - 1u)));
        const int nslots = (int)((n1 + 63) / 64);
        int b = hb;
        for (; b >= 1; b -= 2) {
            const int32_t c1 = T | (1 << (b - 1)), c2 = T | (2 << (b - 1)), c3 = T | (3 << (b - 1));
            uint32_t m1 = 0, m2 = 0, m3 = 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (j < nslots) {
                    m1 += __popcll(__ballot(c[j] >= c1));
                    m2 += __popcll(__ballot(c[j] >= c2));
                    m3 += __popcll(__ballot(c[j] >= c3));
                }
            }
            T |= ((m3 >= need) ? 3 : (m2 >= need) ? 2 : (m1 >= need) ? 1 : 0) << (b - 1);
        }
        if (b == 0) {
            uint32_t m1 = 0;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (j < nslots) m1 += __popcll(__ballot(c[j] >= (T | 1)));
            if (m1 >= need) T |= 1;
        }
    } else {
        int round = 0;
        for (int sh2 = 29; sh2 >= 1; sh2 -= 2, ++round) {
            const uint64_t c = block_sum_uniform<NW>(
                count3(cand, tid, n1, NT, T | (1 << sh2), T | (2 << sh2), T | (3 << sh2)), red[round & 1]);
            const int64_t t1 = c & 0x1fffff, t2 = (c >> 21) & 0x1fffff, t3 = c >> 42;
            T |= ((t3 >= need) ? 3 : (t2 >= need) ? 2 : (t1 >= need) ? 1 : 0) << sh2;
        }
        const uint64_t c = block_sum_uniform<NW>(count3(cand, tid, n1, NT, T | 1, T | 1, T | 1), red[round & 1]);
        if ((int64_t)(c & 0x1fffff) >= need) T |= 1;
    }

    // ---- 3. ordered compaction: per-thread counts of keys > T and == T
    // (packed 16 bits each: a wave holds at most 64 * 64 keys), their
    // exclusive prefix over the wave, the wave totals through LDS
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) cnt += (key[i] > T ? 1u : 0u) + (key[i] == T ? 0x10000u : 0u);
    const uint32_t cincl = wave_incl_scan(cnt, lane);
    const uint32_t gt_w = (cincl - cnt) & 0xffffu, eq_w = (cincl - cnt) >> 16;
    if (lane == 63) wsum64[wave] = ((uint64_t)(cincl & 0xffffu) << 32) | (cincl >> 16);
    __syncthreads();
    uint64_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint64_t x = wsum64[w];
        before += (w < wave) ? x : 0;
        total += x;
    }
    // group sizes fit 32 bits (K < 2^31)
    const int32_t kk32 = (int32_t)kk;
    const int32_t gt_before = (int32_t)(before >> 32) + (int32_t)gt_w;
    const int32_t eq_before = (int32_t)(before & 0xffffffffu) + (int32_t)eq_w;
    const int32_t need_eq = kk32 - (int32_t)(total >> 32);  // >= 1 by the choice of T
    int32_t pos = gt_before + min(eq_before, need_eq);
    int32_t eq_seen = eq_before;
    const int32_t kbase = (int32_t)base;
    int32_t *out = idx + grp * ldidx;
    double dropped = 0.0;
    const bool want_bound = bound != nullptr;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int32_t kv = key[i];      // -1 (absent) is neither kept nor dropped
        bool keep = kv > T;
        if (kv == T) {
            keep = eq_seen < need_eq;
            ++eq_seen;
        }
        if (keep) {
            // the kept list goes to LDS (every reader of cand passed a barrier
            // since) and leaves in one coalesced copy after the last barrier
            if (pos < kk32) cand[pos] = kbase + i;   // always true when T is the kk-th key
            ++pos;
        } else if (want_bound && kv >= 0) {
            dropped += (double)__int_as_float(kv);
        }
    }
    if (lead && tid == 0 && thresh) thresh[grp] = __int_as_float(T);
    if (bound) {
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) dropped += __shfl_xor(dropped, m, 64);
        if (lane == 0) fsum[wave] = dropped;
    }
    if constexpr (NRB > 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's row blocks
    // LDS-only barrier: the kept list and fsum are in LDS; the one
    // global store issued so far (thresh) is read by no one here, so there is
    // no need to wait for it as __syncthreads would
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int64_t padded = pad_up(kk);
    if (lead) {
        for (int64_t j = tid; j < kk; j += NT) out[j] = cand[j];
        if (padded > kk) {
            const int32_t last = cand[kk - 1];   // kk >= 1 here
            for (int64_t j = kk + tid; j < padded; j += NT) out[j] = last;
        }
        if (bound && tid == 0) {
            double b = 0.0;
            for (int w = 0; w < NW; ++w) b += fsum[w];
            bound[grp] = b;
        }
    }
    if constexpr (NRB > 0) {
        // the rows and the kept list are in LDS: panel chunk c of row i holds
        // the row's elements at kept indices 8c .. 8c+7 (zero past kk).
        // (row, chunk) items in row-major order, thread tid takes items tid,
        // tid + 1024, ..., stepped without division
        const int cpr = (int)(padded / 8);
        const int kk32 = (int)kk;
        const int di = NT / cpr, dc = NT % cpr;
        int i = tid / cpr, c = tid % cpr;
        for (; i < nrows; i += di, c += dc) {
            if (c >= cpr) {
                c -= cpr;
                if (++i >= nrows) break;
            }
            const int j0 = 8 * c;
            const uint16_t *row = (const uint16_t *)(stage + (size_t)i * (size_t)ga.lda * 2);
            uint32_t h[8];
            if (j0 + 8 <= kk32) {
                const int4 i0 = *(const int4 *)(cand + j0);
                const int4 i1 = *(const int4 *)(cand + j0 + 4);
                const int32_t ks[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
                for (int q = 0; q < 8; ++q) h[q] = row[ks[q]];
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) h[q] = (j0 + q < kk32) ? row[cand[j0 + q]] : 0u;
            }
            // streaming store: the panel is read next by other CUs, not from this L2
            const u32x4 o = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
            __builtin_nontemporal_store(o, (u32x4 *)(ga.Ap + (srow0 + i) * ga.ldp + j0));
        }
    }
}

// ------------------------------------------------------------------ one wave per group
// Used for many short groups (at most 64 * KPT <= 256 keys: the QK feature
// lists of 128 candidates).  Key i = 64 j + lane sits in register j of lane
// `lane`, so loads coalesce and the kept indices, taken in (j, lane) order,
// come out ascending.  T by a bitwise search over the keys in registers, two
// bits per round with ballot counts (a histogram and bucket scan over 2048
// buckets took 7 us for 1024 groups of 128, ranking every key against every
// other 10.9 us), then the ordered compaction with ballots (keys == T kept in
// index order until kk).
__device__ __forceinline__ int wave_min(int v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ int wave_max(int v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int KPT>
__global__ void __launch_bounds__(64)
k_select_wave(const float *__restrict__ scores, SelectShape sh, int32_t *__restrict__ idx, int64_t ldidx,
              float *__restrict__ thresh, double *__restrict__ bound)
{
    static_assert(KPT <= 4, "one wave holds at most 256 keys");
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
    const int lane = threadIdx.x;
    const uint64_t below = lanes_below(lane);

    int32_t key[KPT];   // -1: no key
    int32_t lo = 0x7fffffff, hi = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int64_t i = (int64_t)j * 64 + lane;
        key[j] = (i < K) ? __float_as_int(s[i]) : -1;
        if (key[j] >= 0) {
            lo = min(lo, key[j]);
            hi = max(hi, key[j]);
        }
    }
    lo = wave_min(lo);
    hi = wave_max(hi);

    int32_t T;
    if (lo == hi) {
        T = lo;   // every key equal
    } else {
        // T = the largest value with #(keys >= T) >= kk, i.e. the kk-th
        // largest key.  lo <= T <= hi, so T shares their common high bits;
        // the rest are found two per round, counting the keys at or above
        // three candidate prefixes with ballots (absent keys, -1, never count)
        const int hb = 31 - __clz(lo ^ hi);
        T = lo & ~((int32_t)((2u << hb) - 1u));
        int b = hb;
        for (; b >= 1; b -= 2) {
            const int32_t c1 = T | (1 << (b - 1)), c2 = T | (2 << (b - 1)), c3 = T | (3 << (b - 1));
            int64_t m1 = 0, m2 = 0, m3 = 0;
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                m1 += __popcll(__ballot(key[j] >= c1));
                m2 += __popcll(__ballot(key[j] >= c2));
                m3 += __popcll(__ballot(key[j] >= c3));
            }
            T |= ((m3 >= kk) ? 3 : (m2 >= kk) ? 2 : (m1 >= kk) ? 1 : 0) << (b - 1);
        }
        if (b == 0) {
            int64_t m1 = 0;
#pragma unroll
            for (int j = 0; j < KPT; ++j) m1 += __popcll(__ballot(key[j] >= (T | 1)));
            if (m1 >= kk) T |= 1;
        }
    }

    // ---- 3. ordered compaction
    uint32_t ngt = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) ngt += key[j] > T;
    const int64_t need_eq = kk - (int64_t)wave_sum(ngt);   // >= 1 by the choice of T
    int32_t *out = idx + grp * ldidx;
    int64_t pos = 0, eq_seen = 0;
    int32_t last = 0;
    double dropped = 0.0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool gtk = key[j] > T, eqk = key[j] == T;
        const uint64_t me = __ballot(eqk);
        const bool keep = gtk || (eqk && eq_seen + __popcll(me & below) < need_eq);
        const uint64_t mk = __ballot(keep);
        if (keep) {
            const int64_t p = pos + __popcll(mk & below);
            if (p < kk) out[p] = j * 64 + lane;
        } else if (key[j] >= 0) {
            dropped += (double)__int_as_float(key[j]);
        }
        if (mk) last = j * 64 + 63 - __clzll(mk);   // highest kept index so far
        pos += __popcll(mk);
        eq_seen += __popcll(me);
    }
    const int64_t padded = pad_up(kk);
    for (int64_t j = kk + lane; j < padded; j += 64) out[j] = last;
    if (thresh && lane == 0) thresh[grp] = __int_as_float(T);
    if (bound) {
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) dropped += __shfl_xor(dropped, m, 64);
        if (lane == 0) bound[grp] = dropped;
    }
}

hipError_t launch_select(const float *scores, const SelectShape &sh, int32_t *idx, int64_t ldidx,
                         float *thresh, double *bound, hipStream_t s)
{
    const dim3 grid((unsigned)sh.groups);
    // Many short groups (the QK feature lists: 128 candidates): one wave per
    // group, many groups per CU at once.
    if (sh.groups >= 512 && sh.K <= 256) {
        hipLaunchKernelGGL(k_select_wave<4>, grid, dim3(64), 0, s, scores, sh, idx, ldidx, thresh, bound);
        return hipGetLastError();
    }
    // Many longer groups (the P.V key lists, up to L keys): 256-thread
    // workgroups, several per CU, 4-wave barriers; a long group no longer
    // rests on one wave (L = 4096: 35 us with one wave per group).
    if (sh.groups >= 512 && sh.K <= 64 * 256) {
        const int64_t kpt = (sh.K + 255) / 256;
#define RMM_SELECT_256(N) \
    hipLaunchKernelGGL((k_select<N, 0, 256>), grid, dim3(256), 0, s, scores, sh, idx, ldidx, thresh, bound, SelectGather{})
        if (kpt <= 2) RMM_SELECT_256(2);
        else if (kpt <= 4) RMM_SELECT_256(4);
        else if (kpt <= 8) RMM_SELECT_256(8);
        else if (kpt <= 16) RMM_SELECT_256(16);
        else if (kpt <= 32) RMM_SELECT_256(32);
        else RMM_SELECT_256(64);
#undef RMM_SELECT_256
        return hipGetLastError();
    }
    // Few groups: one 1024-thread workgroup each, whose 16 waves finish a
    // group soonest -- latency.
    const int64_t kpt = (sh.K + kSelectThreads - 1) / kSelectThreads;
#define RMM_SELECT_LAUNCH(N)                                                                              \
    hipLaunchKernelGGL((k_select<N, 0, kSelectThreads>), grid, dim3(kSelectThreads), 0, s, scores, sh, idx, ldidx, \
                       thresh, bound, SelectGather{})
    if (kpt <= 2) RMM_SELECT_LAUNCH(2);
    else if (kpt <= 4) RMM_SELECT_LAUNCH(4);
    else if (kpt <= 8) RMM_SELECT_LAUNCH(8);
    else if (kpt <= 16) RMM_SELECT_LAUNCH(16);
    else RMM_SELECT_LAUNCH(32);
#undef RMM_SELECT_LAUNCH
    return hipGetLastError();
}

bool select_gather_plan(int dt, int64_t M, int64_t K, int64_t lda, int64_t group_rows, SelectGather &ga,
                        int &nrb)
{
    const int64_t G = (M + group_rows - 1) / group_rows;
    const int64_t kpt = (K + kSelectThreads - 1) / kSelectThreads;
    if (dt != 1 || kpt > 8 || G >= 512) return false;
    const int64_t rows = group_rows < M ? group_rows : M;   // rows of the largest group
    const int64_t row_bytes = lda * 2;
    const int64_t cap = 6 * 16 * 1024;                      // largest staging (NRB = 6)
    if (row_bytes > cap) return false;
    // about 256 workgroups in all, fewer rows per slice if they do not fit
    int64_t slices = 256 / G;
    if (slices < 1) slices = 1;
    if (slices > rows) slices = rows;
    int64_t per = (rows + slices - 1) / slices;
    if (per * row_bytes > cap) per = cap / row_bytes;
    slices = (rows + per - 1) / per;
    if (G * slices > 512) return false;
    const int64_t bytes = per * row_bytes;
    nrb = bytes <= 16384 ? 1 : bytes <= 32768 ? 2 : bytes <= 65536 ? 4 : 6;
    ga.M = M;
    ga.lda = lda;
    ga.gr = group_rows;
    ga.slices = (int)slices;
    ga.rows = per;
    return true;
}

hipError_t launch_select_gather(const float *scores, const SelectShape &sh, int32_t *idx, int64_t ldidx,
                                float *thresh, double *bound, const SelectGather &ga, int nrb, hipStream_t s)
{
    dim3 grid((unsigned)(sh.groups * ga.slices)), block(kSelectThreads);
    const int64_t kpt = (sh.K + kSelectThreads - 1) / kSelectThreads;
#define RMM_SG_LAUNCH(N, R) \
    hipLaunchKernelGGL((k_select<N, R, kSelectThreads>), grid, block, 0, s, scores, sh, idx, ldidx, thresh, bound, ga)
#define RMM_SG_NRB(N)                        \
    do {                                     \
        if (nrb == 1) RMM_SG_LAUNCH(N, 1);   \
        else if (nrb == 2) RMM_SG_LAUNCH(N, 2); \
        else if (nrb == 4) RMM_SG_LAUNCH(N, 4); \
        else RMM_SG_LAUNCH(N, 6);            \
    } while (0)
    if (kpt <= 1) RMM_SG_NRB(1);
    else if (kpt <= 2) RMM_SG_NRB(2);
    else if (kpt <= 4) RMM_SG_NRB(4);
    else RMM_SG_NRB(8);
#undef RMM_SG_NRB
#undef RMM_SG_LAUNCH
    return hipGetLastError();
}

}  // namespace rmm
