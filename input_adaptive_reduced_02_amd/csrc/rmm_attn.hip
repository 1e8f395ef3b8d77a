// rmm_attn.hip -- attention probabilities with the QK^T feature reduction,
// emitting the P.V key scores on the way (gfx950).
//
// "Reduced Matrix Multiplication..." technical summary, Metodologia > Escopo
// de Aplicacao: in attention the method reduces the feature (head) dimension
// of QK^T and, optionally, the token dimension of PV.  For head h and query
// block g (128 queries, candidate keys k < K_g: the causal prefix, or every
// key without the mask):
//   feature score  s_j = ||Q[block, j]||_2 * ||K[0 .. K_g-1, j]||_2   (k_qk_score)
//   kept features  I   = the kk = ceil(r D) best (the shared select kernel)
//   logits         S[q, k] = sum_{j in I} Q[q, j] K[k, j] / sqrt(D)
//   probabilities  P[q, .] = softmax of row q over its keys (k <= q causal)
// k_attn_probs forms P and stores it bf16 and KEY-MAJOR (Pt[h][k][q]), the
// layout the P.V product reads; from the stored values it also forms the P.V
// key scores (sum over the block's queries of P[q, k]) * ||V[k, :]||_2, so
// the token-dimension selection needs no second pass over P.
//
// k_attn_probs, one 512-thread workgroup per (head, query block):
//   waves 0-3 (compute) hold the block's 128 queries x KP kept features as
//   MFMA fragments in registers for the whole kernel and multiply them with
//   key tiles of 128 keys x KP features in LDS (v_mfma_f32_32x32x16_bf16, a
//   2 x 2 arrangement of 64 x 64 wave tiles);
//   waves 4-7 (helpers) stage the next key tile (16-byte loads; with a
//   feature list, each kept feature is written to its slot so tiles are
//   compact), and in the second pass store the finished P tile to HBM and sum
//   its key rows for the P.V scores, while the compute waves work on the next
//   tile.  One barrier per tile; key tiles and P tiles are double-buffered.
//   Pass 1 (S^T = K Q^T, keys as rows): every lane keeps a running max and
//   sum of exp2 for its queries over its keys; the partials of lane pairs and
//   of the two key halves are merged at the end of the pass.
//   Pass 2 (S = Q K^T, queries as rows): recompute the tile, P =
//   exp2(S * log2(e)/sqrt(D) - M_q) with M_q = max + log2(sum) of the row,
//   rounded to bf16; four consecutive queries of one key land in one 8-byte
//   LDS write of the key-major tile.
// Roofline: pass 2 writes the causal half of Pt (L^2 H bytes at L per head)
// and both passes recompute the logits, so HBM writes and the exp2 work bound
// the kernel; the key tiles come from L2 (a head's workgroups share an XCD).
#include "rmm_internal.h"
#include "rmm_tile.h"

namespace rmm {

constexpr int kHD = 128;                 // head dimension D
constexpr int kQB = 128;                 // queries per block
constexpr int kKT = 128;                 // keys per tile
constexpr int kPitch = 136;              // LDS row pitch in bf16 (272 bytes: rows 4 banks apart)
constexpr int kTile = 128 * kPitch;      // bf16 per LDS tile
constexpr int kAttnThreads = 512;

// ------------------------------------------------------------------ feature scores
// acc += x*x over rows t0 .. t1-1 of a column with row stride kHD, ascending
// (16 loads in flight; fma of an exact square rounds once, like x*x + acc).
__device__ __forceinline__ void sumsq_col(const uint16_t *p, int64_t t0, int64_t t1, double &acc)
{
    int64_t t = t0;
    for (; t + 16 <= t1; t += 16) {
        double x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) x[u] = (double)bf16_to_f32(p[(t + u) * kHD]);
#pragma unroll
        for (int u = 0; u < 16; ++u) acc = __builtin_fma(x[u], x[u], acc);
    }
    for (; t < t1; ++t) {
        const double x = (double)bf16_to_f32(p[t * kHD]);
        acc = __builtin_fma(x, x, acc);
    }
}

// the same over two columns at once (query and key feature j)
__device__ __forceinline__ void sumsq_cols2(const uint16_t *p, const uint16_t *q, int64_t t0, int64_t t1,
                                            double &a, double &b)
{
    int64_t t = t0;
    for (; t + 16 <= t1; t += 16) {
        double x[16], y[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            x[u] = (double)bf16_to_f32(p[(t + u) * kHD]);
            y[u] = (double)bf16_to_f32(q[(t + u) * kHD]);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            a = __builtin_fma(x[u], x[u], a);
            b = __builtin_fma(y[u], y[u], b);
        }
    }
    for (; t < t1; ++t) {
        const double x = (double)bf16_to_f32(p[t * kHD]), y = (double)bf16_to_f32(q[t * kHD]);
        a = __builtin_fma(x, x, a);
        b = __builtin_fma(y, y, b);
    }
}

// One lane per (head, feature j) walks the rows in order: the key column's
// running sum of squares is the prefix norm of every block in turn, so one
// pass gives all blocks.  scores[h][g][j], binary32 of the fp64 product.
template <int CAUSAL, int USE_K>
__global__ void __launch_bounds__(64)
k_qk_score(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, int64_t L, float *__restrict__ scores)
{
    const int64_t h = blockIdx.x >> 1;
    const int j = (int)((blockIdx.x & 1) << 6) + (int)threadIdx.x;
    const uint16_t *qp = Q + h * L * kHD + j;
    const uint16_t *kp = K + h * L * kHD + j;
    const int64_t G = (L + kQB - 1) / kQB;
    float *out = scores + h * G * kHD + j;
    double kfull = 1.0;
    if (USE_K && !CAUSAL) {
        double a = 0.0;
        sumsq_col(kp, 0, L, a);
        kfull = __builtin_sqrt(a);
    }
    double ka = 0.0;
    for (int64_t g = 0; g < G; ++g) {
        const int64_t t0 = g * kQB, t1 = (t0 + kQB < L) ? t0 + kQB : L;
        double qa = 0.0;
        if (USE_K && CAUSAL) sumsq_cols2(qp, kp, t0, t1, qa, ka);
        else sumsq_col(qp, t0, t1, qa);
        const double kn = USE_K ? (CAUSAL ? __builtin_sqrt(ka) : kfull) : 1.0;
        out[g * kHD] = (float)(__builtin_sqrt(qa) * kn);
    }
}

hipError_t launch_qk_score(const uint16_t *Q, const uint16_t *K, int64_t H, int64_t L, int causal, int use_k,
                           float *scores, hipStream_t s)
{
    dim3 grid((unsigned)(2 * H)), block(64);
    if (causal && use_k) hipLaunchKernelGGL((k_qk_score<1, 1>), grid, block, 0, s, Q, K, L, scores);
    else if (use_k) hipLaunchKernelGGL((k_qk_score<0, 1>), grid, block, 0, s, Q, K, L, scores);
    else hipLaunchKernelGGL((k_qk_score<0, 0>), grid, block, 0, s, Q, K, L, scores);
    return hipGetLastError();
}

// ------------------------------------------------------------------ probabilities
// Window w of a row is its features 8w .. 8w+7 (one 16-byte chunk).  A
// staging thread always handles the same window; `mask` marks its kept
// features and `base` is the slot of the first of them (the number of kept
// features below 8w).
struct Window {
    uint32_t mask;
    int base;
};

template <int IDX>
__device__ __forceinline__ void put_chunk(uint16_t *row, int w, const Window &win, u32x4 v)
{
    if (!IDX) {
        *(u32x4 *)(row + 8 * w) = v;
        return;
    }
    int s = win.base;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if ((win.mask >> e) & 1u) {
            const uint32_t word = v[e >> 1];
            row[s] = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
            ++s;
        }
    }
}

__device__ __forceinline__ u32x4 load_chunk(const uint16_t *base, int64_t row, int64_t rows_valid, int w)
{
    if (row < rows_valid) return *(const u32x4 *)(base + row * kHD + 8 * w);
    return u32x4{0u, 0u, 0u, 0u};
}

template <int IDX, int KS>
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

    // ---- this thread's feature window and its kept features
    const int w = tid & 15;
    Window win{0xffu, 8 * w};
    if (IDX) {
        const int32_t *I = idx + (h * G + g) * ldidx;
        uint32_t m = 0;
        int b = 0;
        for (int j = 0; j < kk; ++j) {
            const int f = I[j];
            if ((f >> 3) == w) m |= 1u << (f & 7);
            b += f < 8 * w;
        }
        win.mask = m;
        win.base = b;
        // pad slots kk .. KP-1 of every row of both key buffers and the query
        // tile stay zero (staging writes only slots below kk)
        for (int r = tid; r < 3 * 128; r += kAttnThreads) {
            uint16_t *row = (r < 256) ? &kbuf[r >> 7][(r & 127) * kPitch] : &pbuf[0][(r & 127) * kPitch];
            for (int s = kk; s < 16 * KS; ++s) row[s] = 0;
        }
    }

    // ---- prologue: query tile into pbuf[0], key tile 0 into kbuf[0]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + kAttnThreads * i, r = c >> 4;
        put_chunk<IDX>(&pbuf[0][r * kPitch], w, win, load_chunk(Qh, q0 + r, L, w));
        put_chunk<IDX>(&kbuf[0][r * kPitch], w, win, load_chunk(Kh, r, L, w));
    }
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
            floatx16 acc[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
            if (u < T) {
                // pass 1, S^T = K Q^T: acc[i][j] rows = keys wk*64 + i*32 + .., cols = queries wq*64 + j*32 + ..
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    bf16x8 kf[2];
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        kf[i] = *(const bf16x8 *)&kb[(wk * 64 + i * 32 + (lane & 31)) * kPitch + 8 * (2 * ks + (lane >> 5))];
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[j][ks], acc[i][j], 0, 0, 0);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (edge) {
                        // key kl = kb + c with c = i*32 + acc_row(0, v) a constant;
                        // cut when c > thr
                        const int ql = wq * 64 + j * 32 + (lane & 31);
                        const int kb = wk * 64 + (lane >> 5) * 4;
                        int thr = klim - kb - 1;
                        if (causal) thr = min(thr, dq + ql - kb);
#pragma unroll
                        for (int i = 0; i < 2; ++i)
#pragma unroll
                            for (int v = 0; v < 16; ++v)
                                if (i * 32 + acc_row(0, v) > thr) acc[i][j][v] = -INFINITY;
                    }
                    float tmax = -INFINITY;
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, acc[i][j][v]);
                    const float mn = fmaxf(m_run[j], tmax * c2);
                    float sum = 0.0f;
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int v = 0; v < 16; ++v) sum += exp2f(acc[i][j][v] * c2 - mn);
                    l_run[j] = l_run[j] * exp2f(m_run[j] - mn) + sum;
                    m_run[j] = mn;
                }
            } else {
                // pass 2, S = Q K^T: acc[i][j] rows = queries wq*64 + i*32 + .., cols = keys wk*64 + j*32 + ..
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    bf16x8 kf[2];
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        kf[j] = *(const bf16x8 *)&kb[(wk * 64 + j * 32 + (lane & 31)) * kPitch + 8 * (2 * ks + (lane >> 5))];
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[i][ks], kf[j], acc[i][j], 0, 0, 0);
                }
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
                            uint32_t hb[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float p = exp2f(acc[i][j][4 * v4 + e] * c2 - mv[e]);
                                if (edge && (gone || i * 32 + acc_row(0, 4 * v4 + e) < thr)) p = 0.0f;
                                hb[e] = f32_to_bf16(p);
                            }
                            const int ql = wq * 64 + qw;
                            *(uint2 *)&pb[kl * kPitch + ql] = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
                        }
                }
            }
            __syncthreads();
        }
    } else {
        // ---------------------------------------------------------------- helper waves
        const int ht = tid - 256;
        u32x4 kreg[8];
        if (U > 1) {
            const int64_t k0 = (int64_t)tile_of(1) * kKT;
#pragma unroll
            for (int i = 0; i < 8; ++i) kreg[i] = load_chunk(Kh, k0 + ((ht + 256 * i) >> 4), L, w);
        }
        __syncthreads();                               // prologue staging done
        for (int u = 0; u <= U; ++u) {
            if (u == T) __syncthreads();               // the compute waves' statistics exchange
            if (u + 1 < U) {
                // key tile u+1 into its buffer (free since the last barrier), loads for tile u+2
                uint16_t *kb = kbuf[(u + 1) & 1];
#pragma unroll
                for (int i = 0; i < 8; ++i) put_chunk<IDX>(&kb[((ht + 256 * i) >> 4) * kPitch], w, win, kreg[i]);
                if (u + 2 < U) {
                    const int64_t kn0 = (int64_t)tile_of(u + 2) * kKT;
#pragma unroll
                    for (int i = 0; i < 8; ++i) kreg[i] = load_chunk(Kh, kn0 + ((ht + 256 * i) >> 4), L, w);
                }
            }
            if (u - 1 >= T) {
                // the P tile of step u-1: key sums (waves 4, 5), stores (waves 6, 7)
                const uint16_t *pb = pbuf[(u - 1) & 1];
                const int64_t kp0 = (int64_t)(u - 1 - T) * kKT;
                if (ht < 128) {
                    const int64_t k = kp0 + ht;
                    if (pvs && k < Kvalid) {
                        double mass = 0.0;
                        for (int c = 0; c < nq / 8; ++c) {
                            const u32x4 v = *(const u32x4 *)&pb[ht * kPitch + 8 * c];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                mass += (double)bf16_lo(v[e]);
                                mass += (double)bf16_hi(v[e]);
                            }
                        }
                        pvs[(h * G + g) * L + k] = (float)(mass * vnorm[h * L + k]);
                    }
                } else {
#pragma unroll 4
                    for (int i = 0; i < 16; ++i) {
                        const int c = (ht - 128) + 128 * i, r = c >> 4, qc = c & 15;
                        const int64_t k = kp0 + r;
                        if (k < Kvalid && 8 * qc < nq)
                            *(u32x4 *)(Pt + (h * L + k) * L + q0 + 8 * qc) = *(const u32x4 *)&pb[r * kPitch + 8 * qc];
                    }
                }
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
    dim3 grid((unsigned)(H * G)), block(kAttnThreads);
#define RMM_ATTN(I, KS_)                                                                                   \
    hipLaunchKernelGGL((k_attn_probs<I, KS_>), grid, block, 0, s, Q, K, H, L, causal, idx, ldidx, (int)kk, Pt, \
                       vnorm, pvs)
    if (!idx) {
        RMM_ATTN(0, 8);
    } else {
        switch ((kk + 15) / 16) {
        case 1: RMM_ATTN(1, 1); break;
        case 2: RMM_ATTN(1, 2); break;
        case 3: RMM_ATTN(1, 3); break;
        case 4: RMM_ATTN(1, 4); break;
        case 5: RMM_ATTN(1, 5); break;
        case 6: RMM_ATTN(1, 6); break;
        case 7: RMM_ATTN(1, 7); break;
        default: RMM_ATTN(1, 8); break;
        }
    }
#undef RMM_ATTN
    return hipGetLastError();
}

}  // namespace rmm
