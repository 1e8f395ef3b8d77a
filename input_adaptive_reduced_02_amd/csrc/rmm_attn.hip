// rmm_attn.hip -- attention probabilities with the QK^T feature reduction,
// emitting the P.V key scores on the way (gfx950).
//
// "Reduced Matrix Multiplication..." technical summary, Metodologia > Escopo
// de Aplicacao: in attention the method reduces the feature (head) dimension
// of QK^T and, optionally, the token dimension of PV.  For head h and query
// block g (128 queries, candidate keys k < K_g: the causal prefix, or every
// key without the mask):
//   feature score  s_j = ||Q[block, j]||_2 * ||K[0 .. K_g-1, j]||_2   (k_qk_ktile, k_qk_qscore)
//   kept features  I   = the kk = ceil(r D) best (the shared select kernel)
//   logits         S[q, k] = sum_{j in I} Q[q, j] K[k, j] / sqrt(D)
//   probabilities  P[q, .] = softmax of row q over its keys (k <= q causal)
// k_attn_probs forms P and stores it bf16 and KEY-MAJOR (Pt[h][k][q]), the
// layout the P.V product reads; from the stored values it also forms the P.V
// key scores (sum over the block's queries of P[q, k]) * ||V[k, :]||_2, so
// the token-dimension selection needs no second pass over P.
//
// k_attn_probs, one 512-thread workgroup per (head, query block):
//   waves 0-3 (compute) hold the block's 128 queries x 128 features as MFMA
//   fragments in registers for the whole kernel, the dropped features zeroed
//   (their products are exact zeros, so the sums are the reduced logits), and
//   multiply them with key tiles of 128 keys in LDS (v_mfma_f32_32x32x16_bf16,
//   a 2 x 2 arrangement of 64 x 64 wave tiles).  Compacting the kept features
//   would save MFMA work, which does not bound this kernel (below), and costs
//   scattered 2-byte LDS writes for every key tile;
//   waves 4-7 (helpers) stage the next key tile (16-byte loads and LDS
//   writes), and in the second pass store the finished P tile to HBM and sum
//   its key rows for the P.V scores, while the compute waves work on the next
//   tile.  One barrier per tile; key tiles and P tiles are double-buffered.
//   Pass 1 (S^T = K Q^T, keys as rows): every lane keeps a running max and
//   sum of exp2 for its queries over its keys; the partials of lane pairs and
//   of the two key halves are merged at the end of the pass.
//   Pass 2 (S = Q K^T, queries as rows): recompute the tile, P =
//   exp2(S * log2(e)/sqrt(D) - M_q) with M_q = max + log2(sum) of the row,
//   rounded to bf16 (v_cvt_pk_bf16_f32); four consecutive queries of one key
//   land in one 8-byte LDS write of the key-major tile.  Masks are applied on
//   the diagonal and ragged tiles only.
// Roofline: pass 2 writes the causal half of Pt (L^2 H bytes for H heads of
// length L) and each element costs two exp2 (one per pass), so the exp2/VALU
// work and the HBM writes bound the kernel; the MFMA work (2 x 2 L^2 D H / 2
// FLOP) is a small share; key tiles come from L2 (a head's workgroups share
// an XCD).
#include "rmm_internal.h"
#include "rmm_tile.h"

namespace rmm {

constexpr int kHD = 128;                 // head dimension D
constexpr int kQB = 128;                 // queries per block
constexpr int kKT = 128;                 // keys per tile
constexpr int kPitch = 136;              // LDS row pitch in bf16 (272 bytes: rows 4 banks apart)
constexpr int kTile = 128 * kPitch;      // bf16 per LDS tile
constexpr int kAttnThreads = 512;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <bool B>
struct Flag {
    static constexpr bool value = B;
};

// two binary32 values -> packed bf16 (v_cvt_pk_bf16_f32: round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// ------------------------------------------------------------------ feature scores
// scores[h][g][j] = binary32(sqrt(qsum) * sqrt(ksum)), qsum the sum of squares
// of query column j over block g, ksum that of key column j over the block's
// keys (the causal prefix, or every key; 1 without key norms).  The sums are
// binary64 in a fixed order chosen for parallelism: within a 128-row tile,
// four partial sums of the rows r = 0, 1, 2, 3 (mod 4) in ascending r, added
// as (p0 + p1) + (p2 + p3); over the tiles of a prefix, the tile sums in
// ascending tile order.  Every square of a bf16 value is exact in binary64,
// so a sum of n of them differs from any other order's by at most about
// n 2^-53 relative -- far inside the binary32 spacing of the score (2^-24),
// so the binary32 scores agree with a plain ascending sum's to within one
// unit in the last place, and only when the sum lies that close to a rounding
// boundary.  Two kernels:
//   k_qk_ktile: one workgroup per (head, key tile): the tile's column sums.
//   k_qk_qscore: one workgroup per (head, query block): the block's query
//     column sums, the prefix of the key tile sums, the product.
// (One workgroup per head carrying the 128 key columns as L-step binary64
// chains through the whole sequence took 41.9 us at L = 4096.)
constexpr int kTileChunks = kQB * kHD / 8;   // 16-byte chunks of a 128 x 128 bf16 tile

// Sum of x*x over rows 0 .. rows-1 of column j of an LDS tile (row stride
// kHD): four partial sums (row mod 4), each in ascending row order, then
// (p0 + p1) + (p2 + p3).  The LDS reads of the next 16 rows are issued before
// the fmas of the current 16.
__device__ __forceinline__ double sumsq_tile(const uint16_t *t, int j, int rows)
{
    double p[4] = {0.0, 0.0, 0.0, 0.0};
    if (rows == kQB) {
        uint16_t x[2][16];
#pragma unroll
        for (int u = 0; u < 16; ++u) x[0][u] = t[u * kHD + j];
#pragma unroll
        for (int b = 0; b < kQB / 16; ++b) {
            if (b + 1 < kQB / 16) {
#pragma unroll
                for (int u = 0; u < 16; ++u) x[(b + 1) & 1][u] = t[((b + 1) * 16 + u) * kHD + j];
            }
            __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of these fmas
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const double v = (double)bf16_to_f32(x[b & 1][u]);
                p[u & 3] = __builtin_fma(v, v, p[u & 3]);
            }
        }
    } else {
        for (int r = 0; r < rows; ++r) {
            const double v = (double)bf16_to_f32(t[r * kHD + j]);
            p[r & 3] = __builtin_fma(v, v, p[r & 3]);
        }
    }
    return (p[0] + p[1]) + (p[2] + p[3]);
}

// 16-byte chunks lt + n*i (i < kTileChunks / n) of tile t of a [L][128] bf16
// matrix; rows past L re-read row L-1 (those rows are never summed)
template <int NCH>
__device__ __forceinline__ void tile_load(const uint16_t *M, int64_t L, int64_t t, int lt, u32x4 (&v)[NCH])
{
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = lt + (kTileChunks / NCH) * i;
        int64_t row = t * kQB + (c >> 4);
        if (row > L - 1) row = L - 1;
        v[i] = *(const u32x4 *)(M + row * kHD + 8 * (c & 15));
    }
}
template <int NCH>
__device__ __forceinline__ void tile_store(uint16_t *buf, int lt, const u32x4 (&v)[NCH])
{
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = lt + (kTileChunks / NCH) * i;
        *(u32x4 *)(buf + (c >> 4) * kHD + 8 * (c & 15)) = v[i];
    }
}

// tsum[h][t][j]: the sum of squares of key column j over key tile t of head h
__global__ void __launch_bounds__(128)
k_qk_ktile(const uint16_t *__restrict__ K, int64_t L, double *__restrict__ tsum)
{
    constexpr int NCH = kTileChunks / 128;
    __shared__ __attribute__((aligned(16))) uint16_t kt[kQB * kHD];
    const int64_t G = (L + kQB - 1) / kQB;
    const int64_t h = blockIdx.x / G, t = blockIdx.x % G;
    const int j = threadIdx.x;
    u32x4 v[NCH];
    tile_load<NCH>(K + h * L * kHD, L, t, j, v);
    tile_store<NCH>(kt, j, v);
    __syncthreads();
    tsum[(h * G + t) * kHD + j] = sumsq_tile(kt, j, (int)((L - t * kQB < kQB) ? (L - t * kQB) : kQB));
}

template <int USE_K, int CAUSAL>
__global__ void __launch_bounds__(128)
k_qk_qscore(const uint16_t *__restrict__ Q, int64_t L, const double *__restrict__ tsum,
            float *__restrict__ scores)
{
    constexpr int NCH = kTileChunks / 128;
    __shared__ __attribute__((aligned(16))) uint16_t qt[kQB * kHD];
    const int64_t G = (L + kQB - 1) / kQB;
    const int64_t h = blockIdx.x / G, g = blockIdx.x % G;
    const int j = threadIdx.x;
    u32x4 v[NCH];
    tile_load<NCH>(Q + h * L * kHD, L, g, j, v);
    double ks = 0.0;
    if (USE_K) {
        // the key tiles the block is multiplied with, added in ascending
        // order; the loads of 16 tiles are issued before their adds (and the
        // first ones while the query tile is still in flight)
        const double *ts = tsum + h * G * kHD + j;
        const int64_t tend = CAUSAL ? g + 1 : G;
        for (int64_t t0 = 0; t0 < tend; t0 += 16) {
            double x[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) x[u] = (t0 + u < tend) ? ts[(t0 + u) * kHD] : 0.0;
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (t0 + u < tend) ks += x[u];
        }
    }
    tile_store<NCH>(qt, j, v);
    __syncthreads();
    const double qa = sumsq_tile(qt, j, (int)((L - g * kQB < kQB) ? (L - g * kQB) : kQB));
    const double kn = USE_K ? __builtin_sqrt(ks) : 1.0;
    scores[(h * G + g) * kHD + j] = (float)(__builtin_sqrt(qa) * kn);
}

hipError_t launch_qk_score(const uint16_t *Q, const uint16_t *K, int64_t H, int64_t L, int causal, int use_k,
                           double *tsum, float *scores, hipStream_t s)
{
    const int64_t G = (L + kQB - 1) / kQB;
    const dim3 grid((unsigned)(H * G)), block(128);
    if (use_k) {
        hipLaunchKernelGGL(k_qk_ktile, grid, block, 0, s, K, L, tsum);
        if (hipError_t e = hipGetLastError()) return e;
    }
    if (causal && use_k) hipLaunchKernelGGL((k_qk_qscore<1, 1>), grid, block, 0, s, Q, L, tsum, scores);
    else if (use_k) hipLaunchKernelGGL((k_qk_qscore<1, 0>), grid, block, 0, s, Q, L, tsum, scores);
    else hipLaunchKernelGGL((k_qk_qscore<0, 0>), grid, block, 0, s, Q, L, tsum, scores);
    return hipGetLastError();
}

// ------------------------------------------------------------------ probabilities
__device__ __forceinline__ u32x4 load_chunk(const uint16_t *base, int64_t row, int64_t rows_valid, int w)
{
    if (row < rows_valid) return *(const u32x4 *)(base + row * kHD + 8 * w);
    return u32x4{0u, 0u, 0u, 0u};
}

// PVS: whether the P.V key scores are formed (pvs != NULL)
template <int PVS>
__global__ void __launch_bounds__(kAttnThreads)
k_attn_probs(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, int64_t H, int64_t L, int causal,
             const int32_t *__restrict__ idx, int64_t ldidx, int kk, uint16_t *__restrict__ Pt,
             const double *__restrict__ vnorm, float *__restrict__ pvs)
{
    __shared__ __attribute__((aligned(16))) uint16_t kbuf[2][kTile];
    __shared__ __attribute__((aligned(16))) uint16_t pbuf[2][kTile];
    __shared__ float2 stat[2][kQB];
    __shared__ __attribute__((aligned(16))) float mrow[4][64];   // M_q of each compute wave's queries

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t G = (L + kQB - 1) / kQB;
    // heaviest causal blocks first; consecutive workgroups take consecutive
    // heads, so with H a multiple of 8 all blocks of a head share an XCD
    const int64_t bid = blockIdx.x;
    const int64_t h = bid % H;
    const int64_t g = causal ? G - 1 - bid / H : bid / H;
    const int64_t q0 = g * kQB;
    const int nq = (int)((L - q0 < kQB) ? (L - q0) : kQB);
    const int T = causal ? (int)(g + 1) : (int)G;     // key tiles
    const uint16_t *Qh = Q + h * L * kHD;
    const uint16_t *Kh = K + h * L * kHD;
    const float c2 = 1.4426950408889634f / 11.313708498984761f;   // log2(e) / sqrt(128)

    // ---- this thread's 16-byte window (features 8w .. 8w+7 of a row) and, with
    // a feature list, the mask that zeroes its dropped features in the query
    // tile: a dropped feature then adds exact zeros to every logit, so the
    // key tiles need no change
    const int w = tid & 15;
    u32x4 keep = {~0u, ~0u, ~0u, ~0u};
    if (idx) {
        const int32_t *I = idx + (h * G + g) * ldidx;
        uint32_t m = 0;
        for (int j = 0; j < kk; ++j) {
            const int f = I[j];
            if ((f >> 3) == w) m |= 1u << (f & 7);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            keep[e] = (((m >> (2 * e)) & 1u) ? 0x0000ffffu : 0u) | (((m >> (2 * e + 1)) & 1u) ? 0xffff0000u : 0u);
    }

    // ---- prologue: query tile into pbuf[0], key tile 0 into kbuf[0]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + kAttnThreads * i, r = c >> 4;
        *(u32x4 *)&pbuf[0][r * kPitch + 8 * w] = load_chunk(Qh, q0 + r, L, w) & keep;
        *(u32x4 *)&kbuf[0][r * kPitch + 8 * w] = load_chunk(Kh, r, L, w);
    }
    constexpr int KS = kHD / 16;                       // 16-deep MFMA steps over the head dimension
    const int U = 2 * T;                               // tiles over both passes
    auto tile_of = [&](int u) { return u < T ? u : u - T; };
    const int64_t Kvalid = L;                          // keys at or past L do not exist

    if (wave < 4) {
        // ---------------------------------------------------------------- compute waves
        const int wq = wave & 1, wk = wave >> 1;       // query half, key half
        __syncthreads();                               // prologue staging done
        bf16x8 qf[2][KS];
        float m_run[2], l_run[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int r = wq * 64 + f * 32 + (lane & 31);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[f][ks] = *(const bf16x8 *)&pbuf[0][r * kPitch + 8 * (2 * ks + (lane >> 5))];
            m_run[f] = -1e30f;
            l_run[f] = 0.0f;
        }
        for (int u = 0; u < U; ++u) {
            const int t = tile_of(u);
            const int64_t k0 = (int64_t)t * kKT;
            const bool edge = (causal && t == g) || (k0 + kKT > Kvalid);
            // masks in tile-local indices: key kl is cut when kl >= klim, or
            // (causal) when kl - ql > dq, ql the block-local query
            const int klim = (int)((Kvalid - k0 < kKT) ? (Kvalid - k0) : kKT);
            const int dq = (int)(q0 - k0);
            if (u == T) {
                // end of pass 1: merge the running (max, sum) of lane pairs
                // and of the two key halves; M_q = max + log2(sum)
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    const float mo = __shfl_xor(m_run[f], 32), lo = __shfl_xor(l_run[f], 32);
                    const float mm = fmaxf(m_run[f], mo);
                    l_run[f] = l_run[f] * exp2f(m_run[f] - mm) + lo * exp2f(mo - mm);
                    m_run[f] = mm;
                    if (lane < 32) stat[wk][wq * 64 + f * 32 + lane] = make_float2(m_run[f], l_run[f]);
                }
                __syncthreads();
                {
                    const int q = wq * 64 + lane;
                    const float2 a = stat[0][q], b = stat[1][q];
                    const float mm = fmaxf(a.x, b.x);
                    const float l = a.y * exp2f(a.x - mm) + b.y * exp2f(b.x - mm);
                    mrow[wave][lane] = mm + __log2f(l);   // read back by this wave only
                }
            }
            const uint16_t *kb = kbuf[u & 1];
            // one K fragment: 8 features (chunk 2ks + lane/32) of key row r of the tile
            auto kfrag = [&](int r, int ks) {
                return *(const bf16x8 *)&kb[r * kPitch + 8 * (2 * ks + (lane >> 5))];
            };
            // Each pass is one straight block per tile kind (masked or not): the
            // MFMAs of the second half are issued after those of the first, so
            // the first half's exp2 work can run under them.
            auto pass1 = [&](auto masked) {
                constexpr bool MASKED = decltype(masked)::value;
                // S^T = K Q^T: acc[i][j] rows = keys wk*64 + i*32 + .., cols = queries wq*64 + j*32 + ..
                floatx16 acc[2][2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 kf = kfrag(wk * 64 + i * 32 + (lane & 31), ks);
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[j][ks], acc[i][j], 0, 0, 0);
                    }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        if (MASKED) {
                            // key kl = kb + c with c = i*32 + acc_row(0, v) a constant;
                            // cut when c > thr
                            const int ql = wq * 64 + j * 32 + (lane & 31);
                            const int kb0 = wk * 64 + (lane >> 5) * 4;
                            int thr = klim - kb0 - 1;
                            if (causal) thr = min(thr, dq + ql - kb0);
#pragma unroll
                            for (int v = 0; v < 16; ++v)
                                if (i * 32 + acc_row(0, v) > thr) acc[i][j][v] = -INFINITY;
                        }
                        float t4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
                        for (int v = 0; v < 16; ++v) t4[v & 3] = fmaxf(t4[v & 3], acc[i][j][v]);
                        const float tmax = fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3]));
                        const float mn = fmaxf(m_run[j], tmax * c2);
                        // v_exp_f32 straight (arguments <= 0; results below 2^-126 may flush to 0)
                        float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            s4[v & 3] += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i][j][v], c2, -mn));
                        l_run[j] = l_run[j] * exp2f(m_run[j] - mn) + ((s4[0] + s4[1]) + (s4[2] + s4[3]));
                        m_run[j] = mn;
                    }
            };
            auto pass2 = [&](auto masked) {
                constexpr bool MASKED = decltype(masked)::value;
                // S = Q K^T: acc[i][j] rows = queries wq*64 + i*32 + .., cols = keys wk*64 + j*32 + ..
                floatx16 acc[2][2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 kf = kfrag(wk * 64 + j * 32 + (lane & 31), ks);
#pragma unroll
                        for (int i = 0; i < 2; ++i)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[i][ks], kf, acc[i][j], 0, 0, 0);
                    }
                // P = exp2(S c2 - M_q), bf16
                uint16_t *pb = pbuf[u & 1];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int kl = wk * 64 + j * 32 + (lane & 31);
                    // query ql = qb + c with c = i*32 + acc_row(0, v) a constant;
                    // cut when the key is past the end, or (causal) c < thr
                    const int qb = wq * 64 + (lane >> 5) * 4;
                    const bool gone = kl >= klim;
                    const int thr = causal ? kl - qb - dq : -1;
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int v4 = 0; v4 < 4; ++v4) {
                            const int qw = i * 32 + acc_row(lane, 4 * v4);   // within the wave's 64 queries
                            const float4 mq = *(const float4 *)&mrow[wave][qw];
                            const float mv[4] = {mq.x, mq.y, mq.z, mq.w};
                            float p[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i][j][4 * v4 + e], c2, -mv[e]));
                                if (MASKED && (gone || i * 32 + acc_row(0, 4 * v4 + e) < thr)) p[e] = 0.0f;
                            }
                            const int ql = wq * 64 + qw;
                            *(uint2 *)&pb[kl * kPitch + ql] = make_uint2(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]));
                        }
                }
            };
            if (u < T) {
                if (edge) pass1(Flag<true>{});
                else pass1(Flag<false>{});
            } else {
                if (edge) pass2(Flag<true>{});
                else pass2(Flag<false>{});
            }
            __syncthreads();
        }
    } else {
        // ---------------------------------------------------------------- helper waves
        const int ht = tid - 256;
        // Key loads and P stores go through buffer resources over one tile:
        // the hardware range check (byte offset at or past num_records) makes
        // a load read zeros and drops a store, which cuts the rows past the
        // last key without per-lane compares. With L <= 32768 every offset
        // stays below 2^31. Lane ht moves bytes 16 (ht & 15) of rows
        // ht / 16 + 16 i, i = 0 .. 7.
        const uint32_t kvoff = (uint32_t)ht * 16u;
        const int qc = ht & 15;
        // lanes whose query columns lie past the block's last query get an
        // offset past any tile's num_records (0x80000000 + 7 * 32 L < 2^32)
        const uint32_t pvoff = 8 * qc < nq ? (uint32_t)((ht >> 4) * L * 2 + 16 * qc) : 0x80000000u;
        const uint32_t prow16 = (uint32_t)(16 * L * 2);
        u32x4 kreg[8];
        auto load_ktile = [&](int64_t k0) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(Kh + k0 * kHD), (short)0, (int)((L - k0) * kHD * 2), 0x00020000);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                kreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, kvoff + 4096u * i, 0, 0));
        };
        if (U > 1) load_ktile((int64_t)tile_of(1) * kKT);
        __syncthreads();                               // prologue staging done
        for (int u = 0; u <= U; ++u) {
            if (u == T) __syncthreads();               // the compute waves' statistics exchange
            if (u + 1 < U) {
                // key tile u+1 into its buffer (free since the last barrier), loads for tile u+2
                uint16_t *kb = kbuf[(u + 1) & 1];
#pragma unroll
                for (int i = 0; i < 8; ++i) *(u32x4 *)&kb[((ht + 256 * i) >> 4) * kPitch + 8 * w] = kreg[i];
                if (u + 2 < U) load_ktile((int64_t)tile_of(u + 2) * kKT);
            }
            if (u - 1 >= T) {
                // the P tile of step u-1: every helper lane stores an eighth of
                // it; with key scores, lanes 2k and 2k+1 first sum half of key
                // row k each (one helper wave per SIMD, so the summing does not
                // pile onto two of the compute waves' SIMDs)
                const uint16_t *pb = pbuf[(u - 1) & 1];
                const int64_t kp0 = (int64_t)(u - 1 - T) * kKT;
                auto store_tile = [&]() {
                    const int64_t rows = Kvalid - kp0 < kKT ? Kvalid - kp0 : kKT;
                    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                        (void *)(Pt + (h * L + kp0) * L + q0), (short)0, (int)(rows * L * 2), 0x00020000);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        // non-temporal (aux 2): P is written once and read by the next launch,
                        // so it should not displace the K and Q tiles still being reused
                        __builtin_amdgcn_raw_buffer_store_b128(
                            *(const u32x4 *)&pb[((ht >> 4) + 16 * i) * kPitch + 8 * qc],
                            rs, pvoff + prow16 * i, 0, 2);
                };
                if (PVS) {
                    // eight partial sums (query q mod 8), each in ascending q,
                    // added as ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 + p7)):
                    // lane 2k forms the first bracket, lane 2k+1 the second
                    const int kr = ht >> 1, hf = ht & 1;
                    const int64_t k = kp0 + kr;
                    double m[4] = {0.0, 0.0, 0.0, 0.0};
                    if (k < Kvalid) {
                        for (int c = 0; c < nq / 8; ++c) {
                            const u32x2 v = *(const u32x2 *)&pb[kr * kPitch + 8 * c + 4 * hf];
                            m[0] += (double)bf16_lo(v[0]);
                            m[1] += (double)bf16_hi(v[0]);
                            m[2] += (double)bf16_lo(v[1]);
                            m[3] += (double)bf16_hi(v[1]);
                        }
                    }
                    const double part = (m[0] + m[1]) + (m[2] + m[3]);
                    const double other = __shfl_xor(part, 1, 64);
                    if (hf == 0 && k < Kvalid) pvs[(h * G + g) * L + k] = (float)((part + other) * vnorm[h * L + k]);
                }
                store_tile();
            }
            if (u < U) __syncthreads();
        }
    }
}

hipError_t launch_attn_probs(const uint16_t *Q, const uint16_t *K, int64_t H, int64_t L, int causal,
                             const int32_t *idx, int64_t ldidx, int64_t kk, uint16_t *Pt, const double *vnorm,
                             float *pvs, hipStream_t s)
{
    const int64_t G = (L + kQB - 1) / kQB;
    if (pvs)
        hipLaunchKernelGGL(k_attn_probs<1>, dim3((unsigned)(H * G)), dim3(kAttnThreads), 0, s, Q, K, H, L, causal,
                           idx, ldidx, (int)kk, Pt, vnorm, pvs);
    else
        hipLaunchKernelGGL(k_attn_probs<0>, dim3((unsigned)(H * G)), dim3(kAttnThreads), 0, s, Q, K, H, L, causal,
                           idx, ldidx, (int)kk, Pt, vnorm, pvs);
    return hipGetLastError();
}

}  // namespace rmm
