// Backward pass of the chunked gated delta rule (dq, dk, dv, dalpha, dbeta,
// dS_0 from dO and dS_T), all arithmetic in fp32: the products on the fp32
// matrix cores, the element-wise work (and KDA's channel-dependent decays) on
// the vector ALUs.
//
// The mixers ("Super Apriel: One Checkpoint, Many Speeds", §2.A: GDN and KDA,
// recurrent mixers with scalar and channel-wise gates) are trained in the
// pages' stages §2.B, so their recurrence is differentiated here.  Per chunk
// of n <= 64 tokens entering with state S (rows t, s; key channel c; value
// column j), with G the cumulative log-gate inside the chunk (per channel for
// KDA, floored per token at -40 as in the forward) and
//   E(t,s,c) = exp(G_tc - G_sc)  (s <= t),   e0 = exp(G_t),
//   ek = exp(G_end - G_t),                    eE = exp(G_end),
// the forward is
//   Ahat_ts = sum_c k_tc k_sc E (s < t),  A = diag(beta) Ahat,
//   P_ts    = sum_c q_tc k_sc E (s <= t), Tinv = (I + A)^{-1}
//   Xr = V - (k e0) S,  U = Tinv diag(beta) Xr
//   O  = scale ((q e0) S + P U),  S_end = eE S + (k ek)^T U.
// Reverse, given dO and dS_end (chunk by chunk from the last):
//   dU = scale P^T dO + (k ek) dS_end,   dX = Tinv^T dU,   dV = beta dX
//   dS = eE dS_end + scale (q e0)^T dO - (k e0)^T diag(beta) dX
//   dA = -dX U^T (s < t),  dP = scale dO U^T (s <= t)
//   dQ0 = scale dO S^T,  dK0 = -diag(beta) dX S^T,  dKt = U dS_end^T
//   dbeta_t = sum_j Xr_tj dX_tj + sum_s dA_ts Ahat_ts
// and, with M = diag(beta) dA, N = dP and the four sums
//   a1 = sum_{s<t} M_ts k_sc E(t,s,c),   a2 = sum_{s<=t} N_ts k_sc E(t,s,c),
//   a3 = sum_{r>t} M_rt k_rc E(r,t,c),   a4 = sum_{r>=t} N_rt q_rc E(r,t,c),
//   dq = dQ0 e0 + a2,   dk = dK0 e0 + dKt ek + a1 + a3 + a4,
//   dG = q (dQ0 e0 + a2) + k (dK0 e0 - dKt ek + a1 - a3 - a4),
//   dG_end = eE sum_j dS_end S + sum_t dKt k ek   (added to the last token),
// dlog alpha_s = sum_{t >= s} dG_t inside the chunk, dalpha = dlog alpha / alpha.
// Where the floor is active (alpha ~ 0) dlog alpha_m is ~alpha_m times the
// true dalpha_m and comes out of a sum whose other terms cancel, so it is not
// divided there: bwd_floor sums the terms that carry alpha_m directly, with
// alpha_m taken out of their exponents (see that kernel).
//
// Kernels (one head per (b, h); 16-column value slices where the work
// separates by value column):
//   bwd_prep   (b, h, chunk)  Ahat, P, Tinv and the factored rows
//                             k e0, k ek, q e0, eE of every chunk -> image
//   bwd_fwd    (b, h, slice)  forward chain: S at every chunk start
//                             (checkpoints) and Xr
//   bwd_dout   (b, h, chunk)  the reverse chain's state-free terms
//                             scale P^T dO and scale (q e0)^T dO
//   bwd_chain  (b, h, slice)  reverse chain: dS_end of every chunk, U, dX,
//                             dV and the Xr.dX part of dbeta
//   bwd_local  (b, h, chunk)  the contractions over all value columns and
//                             everything that maps back to q, k, beta, alpha
//   bwd_floor  (b, h, chunk)  dalpha where the log-gate floor is active (only
//                             chunks bwd_local flags do any work)
#include <algorithm>

#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kC = 64;
constexpr int kSl = 16;  // value columns per slice
constexpr float kFloor = -40.0f;
constexpr int kTP = kC + 1;  // pitch of 64 x 64 tiles in LDS
constexpr int kNT = 1024;    // threads per workgroup: the LDS use allows one
                             // workgroup per CU, so four waves per SIMD come
                             // from one workgroup (latency hiding)

template <typename T> __device__ __forceinline__ float ld(const T* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

__device__ __forceinline__ float log_gate(float a) { return fmaxf(__logf(a), kFloor); }

// fp32 matrix-core tile product, v_mfma_f32_16x16x4f32: D[16x16] += A[16x4] B[4x16].
// Lane l (li = l % 16, lk = l / 16) supplies A[li][lk] and B[lk][li] and holds
// D[4 lk + r][li] in component r.  A 16-row tile of a product over K is K/4
// such steps; two accumulators alternate so that consecutive steps do not
// wait on each other.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
template <typename FA, typename FB>
__device__ __forceinline__ f32x4 tile_product(int k0, int k1, FA fa, FB fb) {
    const int lk = (threadIdx.x & 63) >> 4;
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
    int k = k0;
#pragma nounroll
    for (; k + 8 <= k1; k += 8) {
        c0 = mma4(fa(k + lk), fb(k + lk), c0);
        c1 = mma4(fa(k + 4 + lk), fb(k + 4 + lk), c1);
    }
    if (k < k1) c0 = mma4(fa(k + lk), fb(k + lk), c0);
    return c0 + c1;
}

// Cross-lane sums and scans (every lane of the wave takes part).
__device__ __forceinline__ float row16_sum(float v) {  // over the 16 lanes of a row
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) v += __shfl_xor(v, m);
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
    return v;
}
// Inclusive prefix (lanes <= l) and suffix (lanes >= l) sums over the wave.
__device__ __forceinline__ float wave_prefix_sum(float v) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(v, d);
        if (l >= d) v += o;
    }
    return v;
}
__device__ __forceinline__ float wave_suffix_sum(float v) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_down(v, d);
        if (l + d < 64) v += o;
    }
    return v;
}

// Per-chunk image (floats): Ahat, P, Tinv [64][64] each, then K0 = k e0,
// Kt = k ek, Q0 = q e0 [64][dk] each, then eE [dk].
enum { iA = 0, iP = kC * kC, iT = 2 * kC * kC, iK0 = 3 * kC * kC };
__host__ __device__ constexpr size_t img_floats(int dk) { return 3 * kC * kC + 3 * kC * dk + dk; }

// Workspace layout (floats), shared by the host sizing and the kernels.
struct Ws {
    size_t img, ck, dck, xr, u, dx, dbp, pd, hq, fl, total;
    __host__ __device__ Ws(int B, int T, int H, int dk, int dv) {
        const size_t bh = static_cast<size_t>(B) * H;
        const size_t nch = (static_cast<size_t>(T) + kC - 1) / kC;
        const size_t tok = static_cast<size_t>(B) * T * H;
        img = 0;                                  // [bh][chunk][img_floats(dk)]
        ck = img + bh * nch * img_floats(dk);     // [bh][chunk][dk][dv]: S at chunk start
        dck = ck + bh * nch * dk * dv;            // [bh][chunk][dk][dv]: dS at chunk end
        xr = dck + bh * nch * dk * dv;            // [B,T,H,dv]
        u = xr + tok * dv;
        dx = u + tok * dv;
        dbp = dx + tok * dv;                      // [dv/16][B,T,H]
        pd = dbp + tok * (dv / kSl);              // [B,T,H,dv]: scale P^T dO
        hq = pd + tok * dv;                       // [bh][chunk][dk][dv]: scale (q e0)^T dO
        fl = hq + bh * nch * dk * dv;             // [bh][chunk] int: a floored gate in the chunk
        total = fl + bh * nch;
    }
};

struct Args {
    int B, T, H, DV, nch;
    // Chunks c0 .. c0 + nr - 1 run in this launch.  The workspace holds them
    // only: per-chunk items at wc(bh, ch), token rows at wt(b, t, h) (Tw =
    // T for the whole sequence at once, nr * 64 for a range of chunks).
    int c0, nr, Tw;
    const float* s_in;     // state at chunk c0 (NULL: zeros)
    float* s_end;          // checkpoint chain: the state after the range (or NULL)
    const float* ds_end;   // state gradient after the range (NULL: zeros)
    float* ds_start;       // reverse chain: the gradient at chunk c0 (or NULL)
    int nsl_chain;  // value slices of the reverse chain (parts of sum_j Xr dX per token)
    float scale;
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    const float* s0;
    const void* dO;
    const float* dsT;
    void* dq;
    void* dk;
    void* dv;
    float* dalpha;
    float* dbeta;
    float* ds0;
    float* ws;
    __host__ __device__ size_t wc(int bh, int ch) const { return static_cast<size_t>(bh) * nr + (ch - c0); }
    __host__ __device__ size_t wt(int b, int t, int h) const {
        return (static_cast<size_t>(b) * Tw + (t - c0 * kC)) * H + h;
    }
};

// Workgroup -> (head, value slice) of the two chains.  Consecutive workgroups
// go to the eight XCDs in turn, so the slices of one head are placed eight
// workgroups apart: they share an XCD and its L2, where they all read the
// head's chunk images.  The grid is padded to a multiple of eight heads.
__device__ __forceinline__ void slice_of(const Args& a, int nsl, int& bh, int& sl) {
    const int x = blockIdx.x, xcd = x & 7, k = x >> 3;
    sl = k % nsl;
    bh = (k / nsl) * 8 + xcd;
}

// ---------------------------------------------------------------- bwd_prep
// Chunk-local quantities of one chunk: its gates (all threads stage the
// log-gates, one thread per channel sums them in LDS), Ahat and P, the
// factored rows K0, Kt, Q0 and eE, and Tinv by forward substitution.
template <int DK, bool KDA, typename InT>
__global__ __launch_bounds__(kNT) void bwd_prep(Args a) {
    constexpr int KP = DK + 1;
    constexpr int GW = KDA ? DK : 1;
    constexpr int GP = GW + 1;
    extern __shared__ float sm[];
    float* Ks = sm;                 // [64][KP]
    float* Qs = Ks + kC * KP;       // [64][KP]
    float* Gs = Qs + kC * KP;       // [64][GP]
    float* As = Gs + kC * GP;       // [64][kTP]  beta-scaled A
    float* Tl = As + kC * kTP;      // [64][kTP]  Tinv
    float* Bs = Tl + kC * kTP;      // [64]
    const int tid = threadIdx.x;
    const int bh = blockIdx.x / a.nr, ch = a.c0 + static_cast<int>(blockIdx.x - bh * a.nr);
    const int b = bh / a.H, h = bh - b * a.H;
    const int t0 = ch * kC, n = min(kC, a.T - t0);
    const InT* q = static_cast<const InT*>(a.q);
    const InT* k = static_cast<const InT*>(a.k);
    auto tok = [&](int t) { return (static_cast<size_t>(b) * a.T + t0 + t) * a.H + h; };
    for (int i = tid; i < kC * DK; i += kNT) {
        const int t = i / DK, c = i - t * DK;
        Ks[t * KP + c] = t < n ? ld(k + tok(t) * DK + c) : 0.f;
        Qs[t * KP + c] = t < n ? ld(q + tok(t) * DK + c) : 0.f;
    }
    for (int i = tid; i < kC * GW; i += kNT) {
        const int t = i / GW, c = i - t * GW;
        Gs[t * GP + c] = t < n ? log_gate(KDA ? a.alpha[tok(t) * DK + c] : a.alpha[tok(t)]) : 0.f;
    }
    if (tid < kC) Bs[tid] = tid < n ? a.beta[tok(tid)] : 0.f;
    __syncthreads();
    // cumulative log-gate (padded tokens add nothing): a wave per channel,
    // lane = token
    for (int c = tid >> 6; c < GW; c += kNT / 64) {
        const int t = tid & 63;
        Gs[t * GP + c] = wave_prefix_sum(Gs[t * GP + c]);
    }
    __syncthreads();
    float* img = a.ws + Ws(a.B, a.Tw, a.H, DK, a.DV).img + a.wc(bh, ch) * img_floats(DK);
    if constexpr (!KDA) {
        // scalar gate: Ahat = (K K^T) o E and P = (Q K^T) o E with one decay
        // E_ts = exp(G_t - G_s) per pair, so both are matrix products on the
        // matrix cores (wave w: the 16 x 16 tile (w / 4, w % 4)).
        const int wave = tid >> 6, li = tid & 15, l4 = (tid & 63) >> 4;
        const int T = 16 * (wave >> 2), S = 16 * (wave & 3);
        if (S <= T) {
            const f32x4 ka = tile_product(0, DK, [&](int k) { return Ks[(T + li) * KP + k]; },
                                          [&](int k) { return Ks[(S + li) * KP + k]; });
            const f32x4 qa = tile_product(0, DK, [&](int k) { return Qs[(T + li) * KP + k]; },
                                          [&](int k) { return Ks[(S + li) * KP + k]; });
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = T + 4 * l4 + r, s = S + li;
                const float e = __expf(fminf(Gs[t * GP] - Gs[s * GP], 0.f));
                const float sa = s < t ? ka[r] * e : 0.f, sp = s <= t ? qa[r] * e : 0.f;
                img[iA + t * kC + s] = sa;
                img[iP + t * kC + s] = sp;
                As[t * kTP + s] = Bs[t] * sa;
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = T + 4 * l4 + r, s = S + li;
                img[iA + t * kC + s] = 0.f;
                img[iP + t * kC + s] = 0.f;
                As[t * kTP + s] = 0.f;
            }
        }
    } else {
        // channel gate: tiles below the diagonal blocks factor the decay at
        // the column block's last token (exp(G_t - G_g) exp(G_g - G_s), both
        // <= 1) and run on the matrix cores; the four diagonal tiles use
        // exact exponentials on the vector ALUs.
        const int wave = tid >> 6, li = tid & 15, l4 = (tid & 63) >> 4;
        const int T = 16 * (wave >> 2), S = 16 * (wave & 3);
        if (S < T) {
            f32x4 ka = {0.f, 0.f, 0.f, 0.f}, qa = {0.f, 0.f, 0.f, 0.f};
            for (int kk = 0; kk < DK; kk += 4) {
                const int c = kk + l4;
                const float gg = Gs[(S + 15) * GP + c];
                const float bk = Ks[(S + li) * KP + c] * __expf(gg - Gs[(S + li) * GP + c]);
                const float et = __expf(Gs[(T + li) * GP + c] - gg);
                ka = mma4(Ks[(T + li) * KP + c] * et, bk, ka);
                qa = mma4(Qs[(T + li) * KP + c] * et, bk, qa);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = T + 4 * l4 + r, s2 = S + li;
                img[iA + t * kC + s2] = ka[r];
                img[iP + t * kC + s2] = qa[r];
                As[t * kTP + s2] = Bs[t] * ka[r];
            }
        } else if (S > T) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = T + 4 * l4 + r, s2 = S + li;
                img[iA + t * kC + s2] = 0.f;
                img[iP + t * kC + s2] = 0.f;
                As[t * kTP + s2] = 0.f;
            }
        }
        for (int i = tid; i < 4 * 16 * 16; i += kNT) {  // the diagonal tiles
            const int blk = i >> 8, t = 16 * blk + ((i >> 4) & 15), s2 = 16 * blk + (i & 15);
            float sa = 0.f, sp = 0.f;
            if (s2 <= t) {
                for (int c = 0; c < DK; ++c) {
                    const float e = __expf(Gs[t * GP + c] - Gs[s2 * GP + c]);
                    const float kse = Ks[s2 * KP + c] * e;
                    sa += Ks[t * KP + c] * kse;
                    sp += Qs[t * KP + c] * kse;
                }
            }
            if (s2 == t) sa = 0.f;
            img[iA + t * kC + s2] = sa;
            img[iP + t * kC + s2] = sp;
            As[t * kTP + s2] = Bs[t] * sa;
        }
    }
    for (int i = tid; i < kC * DK; i += kNT) {
        const int t = i / DK, c = i - t * DK;
        const float g = Gs[t * GP + (KDA ? c : 0)], ge = Gs[(kC - 1) * GP + (KDA ? c : 0)];
        const float e0 = __expf(g);
        img[iK0 + i] = Ks[t * KP + c] * e0;
        img[iK0 + kC * DK + i] = Ks[t * KP + c] * __expf(ge - g);
        img[iK0 + 2 * kC * DK + i] = Qs[t * KP + c] * e0;
        if (t == 0) img[iK0 + 3 * kC * DK + c] = __expf(ge);
    }
    for (int i = tid; i < kC * kC; i += kNT) Tl[(i >> 6) * kTP + (i & 63)] = (i >> 6) == (i & 63) ? 1.f : 0.f;
    __syncthreads();
    // Tinv = (I + A)^{-1}, unit lower triangular, by 16 x 16 blocks: the four
    // diagonal blocks D_b = (I + A_bb)^{-1} row by row (one wave, lane =
    // block and column; Tinv starts as I, so every lane runs the same range),
    // then the blocks below them by their distance d from the diagonal,
    //   T_ij = -D_i sum_{k=j}^{i-1} A_ik T_kj,
    // as fp32 matrix-core products (wave j takes block (j + d, j)).
    if (tid < kC) {
        const int o = 16 * (tid >> 4), s = tid & 15;
        for (int t = 1; t < 16; ++t) {
            float v = 0.f;
            for (int r = 0; r < t; ++r) v -= As[(o + t) * kTP + o + r] * Tl[(o + r) * kTP + o + s];
            if (s < t) Tl[(o + t) * kTP + o + s] = v;
        }
    }
    __syncthreads();
    {
        constexpr int YP = 17;
        float* Ys = Qs;  // q is written out already: 3 tiles of [16][YP] scratch
        const int wave = tid >> 6, li = tid & 15, l4 = (tid & 63) >> 4;
        for (int d = 1; d < 4; ++d) {
            const int J = 16 * wave, I = J + 16 * d;
            if (wave < 4 - d) {
                const f32x4 y = tile_product(J, I, [&](int k) { return As[(I + li) * kTP + k]; },
                                             [&](int k) { return Tl[k * kTP + J + li]; });
#pragma unroll
                for (int r = 0; r < 4; ++r) Ys[wave * 16 * YP + (4 * l4 + r) * YP + li] = y[r];
            }
            __syncthreads();
            if (wave < 4 - d) {
                const f32x4 t = tile_product(0, 16, [&](int k) { return Tl[(I + li) * kTP + I + k]; },
                                             [&](int k) { return Ys[wave * 16 * YP + k * YP + li]; });
#pragma unroll
                for (int r = 0; r < 4; ++r) Tl[(I + 4 * l4 + r) * kTP + J + li] = -t[r];
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < kC * kC; i += kNT) img[iT + i] = Tl[(i >> 6) * kTP + (i & 63)];
}

// ---------------------------------------------------------------- bwd_fwd
// FS value columns per workgroup: the widest of 64, 32 and 16 that still
// puts a workgroup on every CU (the kernel's LDS has room for them, and a
// wider slice reads each chunk image for more columns).
template <int DK, bool KDA, typename InT, int FS>
__global__ __launch_bounds__(kNT) void bwd_fwd(Args a) {
    constexpr int KP = DK + 1;
    constexpr int NCT = FS / 16;     // 16-column tiles of the slice
    extern __shared__ float sm[];
    float* K0 = sm;                  // [64][KP]
    float* Kt = K0 + kC * KP;        // [64][KP]
    float* Ti = Kt + kC * KP;        // [64][kTP]
    float* Ss = Ti + kC * kTP;       // [DK][FS]
    float* Xs = Ss + DK * FS;        // [64][FS]  Xr
    float* Us = Xs + kC * FS;        // [64][FS]
    float* eE = Us + kC * FS;        // [DK]
    float* Bs = eE + DK;             // [64]
    const int tid = threadIdx.x;
    const int nsl = a.DV / FS;
    int bh, sl;
    slice_of(a, nsl, bh, sl);
    if (bh >= a.B * a.H) return;  // padding of the grid (whole block, before any barrier)
    const int b = bh / a.H, h = bh - b * a.H;
    const int j0 = sl * FS;
    const Ws W(a.B, a.Tw, a.H, DK, a.DV);
    const InT* v = static_cast<const InT*>(a.v);
    for (int i = tid; i < DK * FS; i += kNT) {
        const int c = i / FS, j = i - c * FS;
        Ss[i] = a.s_in ? a.s_in[(static_cast<size_t>(bh) * DK + c) * a.DV + j0 + j] : 0.f;
    }
    // Matrix-core tiles: wave w takes row tile w / NCT and column tile w % NCT
    // of each product (rows t for Xr and U, rows c for S); a lane's column
    // is 16 (w % NCT) + lane % 16.
    const int wave = tid >> 6, li = tid & 15, l4 = (tid & 63) >> 4;
    const int R = 16 * (wave / NCT), col = 16 * (wave % NCT) + li;
    // The next chunk's image (K0, Kt, Tinv, eE) and beta are loaded into
    // registers while the current chunk is computed.
    constexpr int NKF = (kC * DK + kNT - 1) / kNT;
    constexpr int NTF = kC * kC / kNT;
    float fk0[NKF], fkt[NKF], fti[NTF], fee = 0.f, fb = 0.f;
    auto fetch = [&](int ch) {
        const float* im = a.ws + W.img + a.wc(bh, ch) * img_floats(DK);
#pragma unroll
        for (int m = 0; m < NKF; ++m) {
            const int i = tid + m * kNT;
            fk0[m] = i < kC * DK ? im[iK0 + i] : 0.f;
            fkt[m] = i < kC * DK ? im[iK0 + kC * DK + i] : 0.f;
        }
#pragma unroll
        for (int m = 0; m < NTF; ++m) fti[m] = im[iT + tid + m * kNT];
        if (tid < DK) fee = im[iK0 + 3 * kC * DK + tid];
        const int nn = min(kC, a.T - ch * kC);
        if (tid < kC) fb = tid < nn ? a.beta[(static_cast<size_t>(b) * a.T + ch * kC + tid) * a.H + h] : 0.f;
    };
    const int ce = a.c0 + a.nr;
    fetch(a.c0);
    for (int ch = a.c0; ch < ce; ++ch) {
        const int t0 = ch * kC, n = min(kC, a.T - t0);
        __syncthreads();  // the previous chunk is done with every buffer
        float* ck = a.ws + W.ck + a.wc(bh, ch) * DK * a.DV;
        for (int i = tid; i < DK * FS; i += kNT) {
            const int c = i / FS, j = i - c * FS;
            ck[static_cast<size_t>(c) * a.DV + j0 + j] = Ss[i];
        }
#pragma unroll
        for (int m = 0; m < NKF; ++m) {
            const int i = tid + m * kNT;
            if (i < kC * DK) {
                K0[(i / DK) * KP + i % DK] = fk0[m];
                Kt[(i / DK) * KP + i % DK] = fkt[m];
            }
        }
#pragma unroll
        for (int m = 0; m < NTF; ++m) {
            const int i = tid + m * kNT;
            Ti[(i >> 6) * kTP + (i & 63)] = fti[m];
        }
        if (tid < DK) eE[tid] = fee;
        if (tid < kC) Bs[tid] = fb;
        if (ch + 1 < ce) fetch(ch + 1);
        __syncthreads();
        // Xr = V - K0 S
        if (R < kC) {
            const f32x4 acc = tile_product(0, DK, [&](int k) { return K0[(R + li) * KP + k]; },
                                           [&](int k) { return Ss[k * FS + col]; });
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = R + 4 * l4 + r;
                const size_t row = (static_cast<size_t>(b) * a.T + t0 + t) * a.H + h;
                const bool ok = t < n;
                const float x = ok ? ld(v + row * a.DV + j0 + col) - acc[r] : 0.f;
                Xs[t * FS + col] = x;
                if (ok) a.ws[W.xr + a.wt(b, t0 + t, h) * a.DV + j0 + col] = x;
            }
        }
        __syncthreads();
        // U = Tinv diag(beta) Xr  (Tinv is zero above its diagonal)
        if (R < kC) {
            const f32x4 acc = tile_product(0, R + 16, [&](int k) { return Ti[(R + li) * kTP + k]; },
                                           [&](int k) { return Bs[k] * Xs[k * FS + col]; });
#pragma unroll
            for (int r = 0; r < 4; ++r) Us[(R + 4 * l4 + r) * FS + col] = acc[r];
        }
        __syncthreads();
        // S <- eE S + Kt^T U  (DK/16 row tiles; at 64 columns a wave takes two)
        for (int R3 = R; R3 < DK; R3 += 16 * (16 / NCT)) {
            const f32x4 acc = tile_product(0, kC, [&](int k) { return Kt[k * KP + R3 + li]; },
                                           [&](int k) { return Us[k * FS + col]; });
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = R3 + 4 * l4 + r;
                Ss[c * FS + col] = eE[c] * Ss[c * FS + col] + acc[r];
            }
        }
    }
    if (a.s_end) {  // the state after the range, where the next range starts
        __syncthreads();
        for (int i = tid; i < DK * FS; i += kNT) {
            const int c = i / FS, j = i - c * FS;
            a.s_end[(static_cast<size_t>(bh) * DK + c) * a.DV + j0 + j] = Ss[i];
        }
    }
}

// ---------------------------------------------------------------- bwd_dout
// The reverse chain's terms that do not depend on its state, per (b, h,
// chunk) and all value columns: Pd = scale P^T dO [64 x dv] and
// Hq = scale (q e0)^T dO [dk x dv], on the matrix cores.
template <int DK, bool KDA, typename InT>
__global__ __launch_bounds__(kNT) void bwd_dout(Args a) {
    constexpr int KP = DK + 1;
    constexpr int HW = 64;           // dO columns staged at a time (two workgroups fit a CU)
    constexpr int OP = HW + 1;
    extern __shared__ float sm[];
    float* Q0 = sm;                  // [64][KP]
    float* Ps = Q0 + kC * KP;        // [64][kTP]
    float* Os = Ps + kC * kTP;       // [64][OP]
    const int tid = threadIdx.x;
    const int bh = blockIdx.x / a.nr, ch = a.c0 + static_cast<int>(blockIdx.x - bh * a.nr);
    const int b = bh / a.H, h = bh - b * a.H;
    const int t0 = ch * kC, n = min(kC, a.T - t0);
    const Ws W(a.B, a.Tw, a.H, DK, a.DV);
    const InT* dO = static_cast<const InT*>(a.dO);
    const float* im = a.ws + W.img + a.wc(bh, ch) * img_floats(DK);
    float* hq = a.ws + W.hq + a.wc(bh, ch) * DK * a.DV;
    for (int i = tid; i < kC * DK; i += kNT) Q0[(i / DK) * KP + i % DK] = im[iK0 + 2 * kC * DK + i];
    for (int i = tid; i < kC * kC; i += kNT) Ps[(i >> 6) * kTP + (i & 63)] = im[iP + i];
    const int wave = tid >> 6, li = tid & 15, l4 = (tid & 63) >> 4;
    for (int j0 = 0; j0 < a.DV; j0 += HW) {
        const int w = min(HW, a.DV - j0);
        __syncthreads();  // (first pass: Q0, P staged; later: the previous half consumed)
        for (int i = tid; i < kC * w; i += kNT) {
            const int t = i / w, j = i - t * w;
            Os[t * OP + j] = t < n ? ld(dO + ((static_cast<size_t>(b) * a.T + t0 + t) * a.H + h) * a.DV + j0 + j) : 0.f;
        }
        __syncthreads();
        const int nct = w / 16;
        // tiles: 4 row tiles of Pd and DK/16 of Hq, times nct column tiles
        for (int tile = wave; tile < (4 + DK / 16) * nct; tile += kNT / 64) {
            const int rt = tile / nct, C = 16 * (tile - rt * nct);
            if (rt < 4) {
                const int R = 16 * rt;
                const f32x4 acc = tile_product(R, kC, [&](int k) { return Ps[k * kTP + R + li]; },
                                               [&](int k) { return Os[k * OP + C + li]; });
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = R + 4 * l4 + r;
                    if (t < n)
                        a.ws[W.pd + a.wt(b, t0 + t, h) * a.DV + j0 + C + li] = a.scale * acc[r];
                }
            } else {
                const int R = 16 * (rt - 4);
                const f32x4 acc = tile_product(0, kC, [&](int k) { return Q0[k * KP + R + li]; },
                                               [&](int k) { return Os[k * OP + C + li]; });
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    hq[static_cast<size_t>(R + 4 * l4 + r) * a.DV + j0 + C + li] = a.scale * acc[r];
            }
        }
    }
}

// ---------------------------------------------------------------- bwd_chain
// FS = 16 value columns per workgroup.
template <int DK, bool KDA, typename InT, int FS>
__global__ __launch_bounds__(kNT) void bwd_chain(Args a) {
    constexpr int KP = DK + 1;
    constexpr int NCT = FS / 16;
    extern __shared__ float sm[];
    float* K0 = sm;                  // [64][KP]
    float* Kt = K0 + kC * KP;        // [64][KP]
    float* Ti = Kt + kC * KP;        // [64][kTP]
    float* dS = Ti + kC * kTP;       // [DK][FS]
    float* Hq = dS + DK * FS;        // [DK][FS]  scale (q e0)^T dO
    float* Xs = Hq + DK * FS;        // [64][FS]  Xr
    float* Pd = Xs + kC * FS;        // [64][FS]  scale P^T dO
    float* Us = Pd + kC * FS;        // [64][FS]  U
    float* dU = Us + kC * FS;        // [64][FS]  dU, then dX
    float* eE = dU + kC * FS;        // [DK]
    float* Bs = eE + DK;             // [64]
    const int tid = threadIdx.x;
    const int nsl = a.DV / FS;
    int bh, sl;
    slice_of(a, nsl, bh, sl);
    if (bh >= a.B * a.H) return;  // padding of the grid (whole block, before any barrier)
    const int b = bh / a.H, h = bh - b * a.H;
    const int j0 = sl * FS;
    const Ws W(a.B, a.Tw, a.H, DK, a.DV);
    InT* dv = static_cast<InT*>(a.dv);
    for (int i = tid; i < DK * FS; i += kNT) {
        const int c = i / FS, j = i - c * FS;
        dS[i] = a.ds_end ? a.ds_end[(static_cast<size_t>(bh) * DK + c) * a.DV + j0 + j] : 0.f;
    }
    // Matrix-core tiles: wave w takes row tile w / NCT, column tile w % NCT
    // (a lane's column: 16 (w % NCT) + lane % 16).
    const int wave = tid >> 6, li = tid & 15, l4 = (tid & 63) >> 4;
    const int R = 16 * (wave / NCT), col = 16 * (wave % NCT) + li;
    // The next (earlier) chunk's image rows K0, Kt and Tinv are loaded into
    // registers while the current chunk is computed (at 16-column slices the
    // registers have room for them; at 32 they do not).
    static_assert(FS == kSl, "the reverse chain runs 16-column slices");
    constexpr int NKF = (kC * DK + kNT - 1) / kNT;
    constexpr int NTF = kC * kC / kNT;
    float fk0[NKF], fkt[NKF], fti[NTF];
    auto fetch = [&](int ch) {
        const float* im = a.ws + W.img + a.wc(bh, ch) * img_floats(DK);
#pragma unroll
        for (int m = 0; m < NKF; ++m) {
            const int i = tid + m * kNT;
            fk0[m] = i < kC * DK ? im[iK0 + i] : 0.f;
            fkt[m] = i < kC * DK ? im[iK0 + kC * DK + i] : 0.f;
        }
#pragma unroll
        for (int m = 0; m < NTF; ++m) fti[m] = im[iT + tid + m * kNT];
    };
    fetch(a.c0 + a.nr - 1);
    for (int ch = a.c0 + a.nr - 1; ch >= a.c0; --ch) {
        const int t0 = ch * kC, n = min(kC, a.T - t0);
        __syncthreads();
        float* dck = a.ws + W.dck + a.wc(bh, ch) * DK * a.DV;
        const float* hq = a.ws + W.hq + a.wc(bh, ch) * DK * a.DV;
        for (int i = tid; i < DK * FS; i += kNT) {
            const int c = i / FS, j = i - c * FS;
            dck[static_cast<size_t>(c) * a.DV + j0 + j] = dS[i];
            Hq[i] = hq[static_cast<size_t>(c) * a.DV + j0 + j];
        }
        const float* im = a.ws + W.img + a.wc(bh, ch) * img_floats(DK);
#pragma unroll
        for (int m = 0; m < NKF; ++m) {
            const int i = tid + m * kNT;
            if (i < kC * DK) {
                K0[(i / DK) * KP + i % DK] = fk0[m];
                Kt[(i / DK) * KP + i % DK] = fkt[m];
            }
        }
#pragma unroll
        for (int m = 0; m < NTF; ++m) {
            const int i = tid + m * kNT;
            Ti[(i >> 6) * kTP + (i & 63)] = fti[m];
        }
        if (tid < DK) eE[tid] = im[iK0 + 3 * kC * DK + tid];
        if (tid < kC) Bs[tid] = tid < n ? a.beta[(static_cast<size_t>(b) * a.T + t0 + tid) * a.H + h] : 0.f;
        for (int i = tid; i < kC * FS; i += kNT) {
            const int t = i / FS, j = i - t * FS;
            const size_t r = a.wt(b, t0 + t, h);
            Xs[i] = t < n ? a.ws[W.xr + r * a.DV + j0 + j] : 0.f;
            Pd[i] = t < n ? a.ws[W.pd + r * a.DV + j0 + j] : 0.f;
        }
        if (ch > a.c0) fetch(ch - 1);
        __syncthreads();
        // U = Tinv diag(beta) Xr (Tinv zero above its diagonal) on the first
        // 4 NCT waves; dU = Pd + Kt dS_end on the next 4 NCT.
        if (wave < 4 * NCT) {
            const f32x4 acc = tile_product(0, R + 16, [&](int k) { return Ti[(R + li) * kTP + k]; },
                                           [&](int k) { return Bs[k] * Xs[k * FS + col]; });
#pragma unroll
            for (int r = 0; r < 4; ++r) Us[(R + 4 * l4 + r) * FS + col] = acc[r];
        } else if (wave < 8 * NCT) {
            const int R2 = R - 64;
            const f32x4 ak = tile_product(0, DK, [&](int k) { return Kt[(R2 + li) * KP + k]; },
                                          [&](int k) { return dS[k * FS + col]; });
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = R2 + 4 * l4 + r;
                dU[t * FS + col] = Pd[t * FS + col] + ak[r];
            }
        }
        __syncthreads();
        // dX = Tinv^T dU, kept in registers until every tile has read dU
        f32x4 xacc = {0.f, 0.f, 0.f, 0.f};
        if (wave < 4 * NCT)
            xacc = tile_product(R, kC, [&](int k) { return Ti[k * kTP + R + li]; },
                                [&](int k) { return dU[k * FS + col]; });
        __syncthreads();
        if (wave < 4 * NCT) {
#pragma unroll
            for (int r = 0; r < 4; ++r) dU[(R + 4 * l4 + r) * FS + col] = xacc[r];
        }
        __syncthreads();
        float* dX = dU;
        for (int i = tid; i < kC * FS; i += kNT) {
            const int t = i / FS, j = i - t * FS;
            if (t < n) {
                const size_t r = (static_cast<size_t>(b) * a.T + t0 + t) * a.H + h;
                const size_t rw = a.wt(b, t0 + t, h);
                Elem<InT>::store(dv + r * a.DV + j0 + j, Bs[t] * dX[i]);
                a.ws[W.u + rw * a.DV + j0 + j] = Us[i];
                a.ws[W.dx + rw * a.DV + j0 + j] = dX[i];
            }
        }
        if (tid < kC) {  // this slice's part of sum_j Xr dX
            float acc = 0.f;
            for (int j = 0; j < FS; ++j) acc += Xs[tid * FS + j] * dX[tid * FS + j];
            if (tid < n) a.ws[W.dbp + static_cast<size_t>(sl) * a.B * a.Tw * a.H + a.wt(b, t0 + tid, h)] = acc;
        }
        // dS <- eE dS + Hq - K0^T diag(beta) dX
        if (R < DK) {
            const f32x4 ak = tile_product(0, kC, [&](int k) { return K0[k * KP + R + li]; },
                                          [&](int k) { return Bs[k] * dX[k * FS + col]; });
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = R + 4 * l4 + r;
                dS[c * FS + col] = eE[c] * dS[c * FS + col] + Hq[c * FS + col] - ak[r];
            }
        }
    }
    __syncthreads();
    if (a.ds_start) {
        for (int i = tid; i < DK * FS; i += kNT) {
            const int c = i / FS, j = i - c * FS;
            a.ds_start[(static_cast<size_t>(bh) * DK + c) * a.DV + j0 + j] = dS[i];
        }
    }
}

// ---------------------------------------------------------------- bwd_local
// Matrix-core mapping: wave w owns row tile T = 16 (w % 4) of every
// [64 x DK] gradient and column tiles 16 (g + 4 i) (g = w / 4) of them, and
// the (T, 16 g) tile of the [64 x 64] ones; a lane holds rows T + 4 (l / 16)
// + r (r = 0..3), column (tile start) + l % 16 of each.
template <int DK, bool KDA, typename InT>
__global__ __launch_bounds__(kNT) void bwd_local(Args a) {
    constexpr int KP = DK + 1;
    constexpr int GW = KDA ? DK : 1;
    constexpr int GP = GW + 1;
    constexpr int NCTILE = DK / 16;          // 16-column tiles of the [64 x DK] gradients
    constexpr int NCT = (NCTILE + 3) / 4;    // of them per wave
    constexpr int CB = 16;                   // value columns per staged block
    constexpr int SP = CB + 1;
    extern __shared__ float sm[];
    float* Ks = sm;                    // [64][KP]  raw k; later dG
    float* Qs = Ks + kC * KP;          // [64][KP]  raw q
    float* Gs = Qs + kC * KP;          // [64][GP]
    float* Ah = Gs + kC * GP;          // [64][kTP] Ahat
    float* X = Ah + kC * kTP;          // union: column blocks / M, N
    float* Sb = X;                     // [DK][SP]  S
    float* Db = Sb + DK * SP;          // [DK][SP]  dS_end
    float* Ub = Db + DK * SP;          // [64][SP]  U
    float* Xb = Ub + kC * SP;          // [64][SP]  dX
    float* Ob = Xb + kC * SP;          // [64][SP]  dO
    float* Mm = X;                     // [64][kTP] M = beta dA  (GDN: then M o E)
    float* Nm = Mm + kC * kTP;         // [64][kTP] N = dP       (GDN: then N o E)
    constexpr int UNION = (2 * DK * SP + 3 * kC * SP) > 2 * kC * kTP ? (2 * DK * SP + 3 * kC * SP) : 2 * kC * kTP;
    float* Bs = X + UNION;             // [64] beta
    float* dB = Bs + kC;               // [64] dbeta
    float* eE = dB + kC;               // [DK]
    float* dGe = eE + DK;              // [DK] dG_end
    float* dGt = dGe + DK;             // [64] GDN: dG per token
    // partial sums, added in a fixed order (the results do not depend on
    // which wave finishes first)
    float* dBp = dGt + kC;             // [4][64] dbeta by column group
    float* dGtp = dBp + 4 * kC;        // [4][64] GDN: dG by column group
    float* gep = dGtp + 4 * kC;        // [2][16] GDN: dG_end by wave (through eE; through Kt)

    const int tid = threadIdx.x;
    const int bh = blockIdx.x / a.nr, ch = a.c0 + static_cast<int>(blockIdx.x - bh * a.nr);
    const int b = bh / a.H, h = bh - b * a.H;
    const int t0c = ch * kC, n = min(kC, a.T - t0c);
    const Ws W(a.B, a.Tw, a.H, DK, a.DV);
    const InT* q = static_cast<const InT*>(a.q);
    const InT* k = static_cast<const InT*>(a.k);
    const InT* dO = static_cast<const InT*>(a.dO);
    auto tok = [&](int t) { return (static_cast<size_t>(b) * a.T + t0c + t) * a.H + h; };
    auto wtok = [&](int t) { return a.wt(b, t0c + t, h); };  // workspace row

    for (int i = tid; i < kC * DK; i += kNT) {
        const int t = i / DK, c = i - t * DK;
        Ks[t * KP + c] = t < n ? ld(k + tok(t) * DK + c) : 0.f;
        Qs[t * KP + c] = t < n ? ld(q + tok(t) * DK + c) : 0.f;
    }
    int floored = 0;  // a gate of this chunk at the log floor (bwd_floor's flag)
    for (int i = tid; i < kC * GW; i += kNT) {
        const int t = i / GW, c = i - t * GW;
        const float lg = t < n ? __logf(KDA ? a.alpha[tok(t) * DK + c] : a.alpha[tok(t)]) : 0.f;
        floored |= !(lg > kFloor);
        Gs[t * GP + c] = fmaxf(lg, kFloor);
    }
    if (tid < kC) {
        Bs[tid] = tid < n ? a.beta[tok(tid)] : 0.f;
        dB[tid] = 0.f;
        dGt[tid] = 0.f;
    }
    if (tid < DK) dGe[tid] = 0.f;
    const float* im = a.ws + W.img + a.wc(bh, ch) * img_floats(DK);
    for (int i = tid; i < kC * kC; i += kNT) Ah[(i >> 6) * kTP + (i & 63)] = im[iA + i];
    floored = __syncthreads_or(floored);
    if (tid == 0) reinterpret_cast<int*>(a.ws + W.fl)[a.wc(bh, ch)] = floored;
    for (int c = tid >> 6; c < GW; c += kNT / 64) {  // cumulative log-gate in place
        const int t = tid & 63;
        const float g = wave_prefix_sum(Gs[t * GP + c]);
        Gs[t * GP + c] = g;
        if (t == kC - 1) eE[c] = __expf(g);  // G_end
    }

    const int wave = tid >> 6, li = tid & 15, l4 = (tid & 63) >> 4;
    const int T = 16 * (wave & 3), g = wave >> 2;
    auto has_ct = [&](int i) { return g + 4 * i < NCTILE; };
    auto ct = [&](int i) { return 16 * (g + 4 * i); };
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 aQ[NCT], aK[NCT], aT[NCT], aA = z4, aP = z4;
#pragma unroll
    for (int i = 0; i < NCT; ++i) aQ[i] = aK[i] = aT[i] = z4;
    float ge = 0.f;  // tid < DK: sum_j dS_end S of channel tid
    const float* Sg = a.ws + W.ck + a.wc(bh, ch) * DK * a.DV;
    const float* Dg = a.ws + W.dck + a.wc(bh, ch) * DK * a.DV;
    // Contractions over the value columns, block by block:
    //   dQ0' = dO S^T, dK0' = dX S^T, dKt = U dS_end^T, dA' = dX U^T, dP' = dO U^T
    // The next block's values are loaded into registers (each thread a fixed
    // set of elements per array) while the current block is multiplied.
    constexpr int NS = (DK * CB + kNT - 1) / kNT;   // S / dS_end elements per thread
    static_assert(kC * CB == kNT, "one U, dX, dO element per thread");
    float ps[NS], pd[NS], pu, px, po;
    const int ut = tid / CB, uj = tid - (tid / CB) * CB;
    auto fetch = [&](int jb) {
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const int i = tid + m * kNT;
            const int c = i / CB, j = i - c * CB;
            const bool ok = i < DK * CB;
            ps[m] = ok ? Sg[static_cast<size_t>(c) * a.DV + jb + j] : 0.f;
            pd[m] = ok ? Dg[static_cast<size_t>(c) * a.DV + jb + j] : 0.f;
        }
        const bool ok = ut < n;
        const size_t r = wtok(ut) * a.DV + jb + uj;  // workspace row
        pu = ok ? a.ws[W.u + r] : 0.f;
        px = ok ? a.ws[W.dx + r] : 0.f;
        po = ok ? ld(dO + tok(ut) * a.DV + jb + uj) : 0.f;
    };
    fetch(0);
    for (int jb = 0; jb < a.DV; jb += CB) {
        __syncthreads();  // previous block consumed (first pass: staging above done)
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const int i = tid + m * kNT;
            if (i < DK * CB) {
                const int c = i / CB, j = i - c * CB;
                Sb[c * SP + j] = ps[m];
                Db[c * SP + j] = pd[m];
            }
        }
        Ub[ut * SP + uj] = pu;
        Xb[ut * SP + uj] = px;
        Ob[ut * SP + uj] = po;
        if (jb + CB < a.DV) fetch(jb + CB);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < CB; kk += 4) {
            const int j = kk + l4;
            const float o = Ob[(T + li) * SP + j], x = Xb[(T + li) * SP + j], u = Ub[(T + li) * SP + j];
            const float us = Ub[(16 * g + li) * SP + j];
            aA = mma4(x, us, aA);
            aP = mma4(o, us, aP);
#pragma unroll
            for (int i = 0; i < NCT; ++i) {
                if (!has_ct(i)) continue;
                const int c = ct(i) + li;
                const float sv = Sb[c * SP + j], dv = Db[c * SP + j];
                aQ[i] = mma4(o, sv, aQ[i]);
                aK[i] = mma4(x, sv, aK[i]);
                aT[i] = mma4(u, dv, aT[i]);
            }
        }
        if (tid < DK) {
            for (int j = 0; j < CB; ++j) ge += Db[tid * SP + j] * Sb[tid * SP + j];
        }
    }
    __syncthreads();  // the column blocks are consumed: M, N take their place
    // dA = -dX U^T (s < t), M = beta dA;  dP = scale dO U^T (s <= t);
    // dbeta_t += sum_s dA_ts Ahat_ts
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = T + 4 * l4 + r, s2 = 16 * g + li;
        const float dA = s2 < t ? -aA[r] : 0.f;
        Mm[t * kTP + s2] = Bs[t] * dA;
        Nm[t * kTP + s2] = s2 <= t ? a.scale * aP[r] : 0.f;
        const float db = row16_sum(dA * Ah[t * kTP + s2]);  // over the row's 16 s
        if (li == 0) dBp[g * kC + t] = db;
    }
    if constexpr (KDA) {
        if (tid < DK) dGe[tid] = eE[tid] * ge;
    } else if (tid < ((DK + 63) & ~63)) {  // whole waves; ge = 0 beyond DK
        const float sg = wave_sum(ge);
        if ((tid & 63) == 0) gep[tid >> 6] = sg;
    }
    __syncthreads();
    // The four gate-weighted sums of the lane's outputs:
    //   a1 = sum_{s<t} M_ts k_sc E(t,s,c),   a2 = sum_{s<=t} N_ts k_sc E(t,s,c),
    //   a3 = sum_{r>t} M_rt k_rc E(r,t,c),   a4 = sum_{r>=t} N_rt q_rc E(r,t,c).
    f32x4 a1[NCT], a2[NCT], a3[NCT], a4[NCT];
#pragma unroll
    for (int i = 0; i < NCT; ++i) a1[i] = a2[i] = a3[i] = a4[i] = z4;
    if constexpr (!KDA) {
        // scalar gate: E(t,s) is one matrix, folded into M and N, after which
        // the sums are four matrix products (M E) K, (N E) K, (M E)^T K,
        // (N E)^T Q.  G decreases along the chunk, so the exponent is <= 0
        // wherever M or N can be nonzero; clamping it leaves 0 * 1 elsewhere.
        for (int i = tid; i < kC * kC; i += kNT) {
            const int t = i >> 6, s2 = i & 63;
            const float e = __expf(fminf(Gs[t * GP] - Gs[s2 * GP], 0.f));
            Mm[t * kTP + s2] *= e;
            Nm[t * kTP + s2] *= e;
        }
        __syncthreads();
#pragma unroll 2
        for (int kk = 0; kk < kC; kk += 4) {
            const int s2 = kk + l4;
            const float m1 = Mm[(T + li) * kTP + s2], n1 = Nm[(T + li) * kTP + s2];
            const float m3 = Mm[s2 * kTP + T + li], n3 = Nm[s2 * kTP + T + li];
#pragma unroll
            for (int i = 0; i < NCT; ++i) {
                if (!has_ct(i)) continue;
                const float kv = Ks[s2 * KP + ct(i) + li], qv = Qs[s2 * KP + ct(i) + li];
                a1[i] = mma4(m1, kv, a1[i]);
                a2[i] = mma4(n1, kv, a2[i]);
                a3[i] = mma4(m3, kv, a3[i]);
                a4[i] = mma4(n3, qv, a4[i]);
            }
        }
    } else {
        // channel gate: E(t,s,c) depends on c.  Across 16-token blocks it
        // factors through the cumulative gate at a block boundary into two
        // factors that are each <= 1 (G decreases along the chunk):
        //   s < T <= t:        E = exp(G_t - G_{T-1}) exp(G_{T-1} - G_s),
        //   t <= T+15 < r:     E = exp(G_r - G_{T+15}) exp(G_{T+15} - G_t),
        // so the parts of a1, a2 (s before the row block) and a3, a4 (r after
        // it) are matrix products with the second factor in the B operand and
        // the first applied to the output; inside the row block the same holds
        // between its 4-token groups, and only pairs within one group take
        // exact exponentials on the vector ALUs.
#pragma unroll
        for (int i = 0; i < NCT; ++i) {
            if (!has_ct(i)) continue;
            const int c = ct(i) + li;
            if (T > 0) {
                const float gr = Gs[(T - 1) * GP + c];
                f32x4 c1 = z4, c2 = z4;
                for (int kk = 0; kk < T; kk += 4) {
                    const int s2 = kk + l4;
                    const float bk = Ks[s2 * KP + c] * __expf(gr - Gs[s2 * GP + c]);
                    c1 = mma4(Mm[(T + li) * kTP + s2], bk, c1);
                    c2 = mma4(Nm[(T + li) * kTP + s2], bk, c2);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float f = __expf(Gs[(T + 4 * l4 + r) * GP + c] - gr);
                    a1[i][r] = c1[r] * f;
                    a2[i][r] = c2[r] * f;
                }
            }
            if (T + 16 < kC) {
                const float gr = Gs[(T + 15) * GP + c];
                f32x4 c3 = z4, c4 = z4;
                for (int kk = T + 16; kk < kC; kk += 4) {
                    const int r2 = kk + l4;
                    const float e = __expf(Gs[r2 * GP + c] - gr);
                    c3 = mma4(Mm[r2 * kTP + T + li], Ks[r2 * KP + c] * e, c3);
                    c4 = mma4(Nm[r2 * kTP + T + li], Qs[r2 * KP + c] * e, c4);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float f = __expf(gr - Gs[(T + 4 * l4 + r) * GP + c]);
                    a3[i][r] = c3[r] * f;
                    a4[i][r] = c4[r] * f;
                }
            }
            // The row block itself, in 4-token groups (the lane's four rows
            // t = T + 4 l4 + r are group l4).  Pairs in different groups factor
            // through a group boundary as above, a K = 4 matrix product per
            // group: s in group j < group of t through b = T + 4j + 3, r in
            // group j > group of t through b = T + 4j - 1; rows outside the
            // valid groups get zero A operands.
#pragma nounroll
            for (int j = 0; j < 3; ++j) {
                const int s2 = T + 4 * j + l4, bb = T + 4 * j + 3;
                const float gb = Gs[bb * GP + c];
                const float bk = Ks[s2 * KP + c] * __expf(gb - Gs[s2 * GP + c]);
                const bool on = li > 4 * j + 3;
                const f32x4 d1 = mma4(on ? Mm[(T + li) * kTP + s2] : 0.f, bk, z4);
                const f32x4 d2 = mma4(on ? Nm[(T + li) * kTP + s2] : 0.f, bk, z4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float f = __expf(fminf(Gs[(T + 4 * l4 + r) * GP + c] - gb, 0.f));
                    a1[i][r] += d1[r] * f;
                    a2[i][r] += d2[r] * f;
                }
            }
#pragma nounroll
            for (int j = 1; j < 4; ++j) {
                const int r2 = T + 4 * j + l4, bb = T + 4 * j - 1;
                const float gb = Gs[bb * GP + c];
                const float e = __expf(Gs[r2 * GP + c] - gb);
                const bool on = li < 4 * j;
                const f32x4 d3 = mma4(on ? Mm[r2 * kTP + T + li] : 0.f, Ks[r2 * KP + c] * e, z4);
                const f32x4 d4 = mma4(on ? Nm[r2 * kTP + T + li] : 0.f, Qs[r2 * KP + c] * e, z4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float f = __expf(fminf(gb - Gs[(T + 4 * l4 + r) * GP + c], 0.f));
                    a3[i][r] += d3[r] * f;
                    a4[i][r] += d4[r] * f;
                }
            }
            // pairs inside the lane's own group, exact: E between tokens u < w
            // of the group is exp(G_w - G_u) for both the lower sums (row w)
            // and the upper ones (row u)
            {
                const int u0 = T + 4 * l4;
                float gg[4], kg[4], qg[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    gg[r] = Gs[(u0 + r) * GP + c];
                    kg[r] = Ks[(u0 + r) * KP + c];
                    qg[r] = Qs[(u0 + r) * KP + c];
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float nd = Nm[(u0 + r) * kTP + u0 + r];
                    a2[i][r] += nd * kg[r];
                    a4[i][r] += nd * qg[r];
                }
#pragma unroll
                for (int w = 1; w < 4; ++w) {
#pragma unroll
                    for (int u = 0; u < w; ++u) {
                        const float e = __expf(fminf(gg[w] - gg[u], 0.f));
                        const float mwu = Mm[(u0 + w) * kTP + u0 + u], nwu = Nm[(u0 + w) * kTP + u0 + u];
                        a1[i][w] += mwu * kg[u] * e;  // row w, s = u
                        a2[i][w] += nwu * kg[u] * e;
                        a3[i][u] += mwu * kg[w] * e;  // row u, r = w
                        a4[i][u] += nwu * qg[w] * e;
                    }
                }
            }
        }
    }
    // gradients of the lane's outputs
    float dq[NCT][4], dk[NCT][4], dg[NCT][4];
    float gk[NCT][4];    // KDA: dKt k ek, G_end's gradient through Kt (summed per channel below)
    float ge_all = 0.f;  // GDN: the lane's part of sum_t dKt k ek (a scalar G_end)
#pragma unroll
    for (int i = 0; i < NCT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dq[i][r] = dk[i][r] = dg[i][r] = gk[i][r] = 0.f;
            if (!has_ct(i)) continue;
            const int t = T + 4 * l4 + r, c = ct(i) + li;
            const float gt = Gs[t * GP + (KDA ? c : 0)];
            const float e0 = __expf(gt);
            const float ek = __expf(Gs[(kC - 1) * GP + (KDA ? c : 0)] - gt);  // exp(G_end - G_t) <= 1
            const float kv = Ks[t * KP + c], qv = Qs[t * KP + c];
            const float dQ0 = a.scale * aQ[i][r], dK0 = -Bs[t] * aK[i][r], dKt = aT[i][r];
            dq[i][r] = dQ0 * e0 + a2[i][r];
            dk[i][r] = dK0 * e0 + dKt * ek + a1[i][r] + a3[i][r] + a4[i][r];
            dg[i][r] = qv * (dQ0 * e0 + a2[i][r]) + kv * (dK0 * e0 - dKt * ek + a1[i][r] - a3[i][r] - a4[i][r]);
            // G_end = G_{n-1}: its gradient through Kt (and, above, eE)
            if constexpr (KDA) gk[i][r] = dKt * kv * ek;
            else ge_all += dKt * kv * ek;
        }
    }
    if constexpr (!KDA) {
        const float sg = wave_sum(ge_all);
        if ((tid & 63) == 0) gep[16 + (tid >> 6)] = sg;
    }
    __syncthreads();  // k, q no longer read: dG goes where k was (KDA: dKt k ek where q was)
    float* dG = Ks;
    float* gK = Qs;
#pragma unroll
    for (int i = 0; i < NCT; ++i) {
        if (!has_ct(i)) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = T + 4 * l4 + r;
            if constexpr (KDA) {
                dG[t * KP + ct(i) + li] = dg[i][r];
                gK[t * KP + ct(i) + li] = gk[i][r];
            }
        }
    }
    if constexpr (!KDA) {  // dG_t = sum over channels: the lane's tiles, then the row's 16 lanes
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float sg = 0.f;
#pragma unroll
            for (int i = 0; i < NCT; ++i) sg += dg[i][r];
            sg = row16_sum(sg);
            if (li == 0) dGtp[g * kC + T + 4 * l4 + r] = sg;
        }
    }
    InT* dqo = static_cast<InT*>(a.dq);
    InT* dko = static_cast<InT*>(a.dk);
#pragma unroll
    for (int i = 0; i < NCT; ++i) {
        if (!has_ct(i)) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = T + 4 * l4 + r;
            if (t < n) {
                Elem<InT>::store(dqo + tok(t) * DK + ct(i) + li, dq[i][r]);
                Elem<InT>::store(dko + tok(t) * DK + ct(i) + li, dk[i][r]);
            }
        }
    }
    __syncthreads();
    if constexpr (!KDA) {  // the partial sums, in a fixed order
        if (tid < kC) dGt[tid] = ((dGtp[tid] + dGtp[kC + tid]) + dGtp[2 * kC + tid]) + dGtp[3 * kC + tid];
        if (tid == 0) {
            float a1 = 0.f, a2 = 0.f;
            for (int w = 0; w < (DK + 63) / 64; ++w) a1 += gep[w];
            for (int w = 0; w < kNT / 64; ++w) a2 += gep[16 + w];
            dGe[0] = eE[0] * a1 + a2;
        }
        __syncthreads();
    }
    // dlog alpha_s = sum_{t >= s} dG_t inside the chunk (G_end's gradient on
    // the last token); dalpha = dlog alpha / alpha unless the floor is active
    // (there bwd_floor writes it).
    float* dL = KDA ? dG : dGt;  // dlog alpha, in place
    constexpr int LP = KDA ? KP : 1;
    for (int c = tid >> 6; c < GW; c += kNT / 64) {  // a wave per channel, lane = token
        const int t = tid & 63;
        const float gke = KDA ? wave_sum(gK[t * KP + c]) : 0.f;  // G_end's gradient through Kt
        const float x = wave_suffix_sum(t < n ? dL[t * LP + c] : 0.f);
        if (t < n) dL[t * LP + c] = x + dGe[c] + gke;
    }
    __syncthreads();
    for (int i = tid; i < n * GW; i += kNT) {
        const int t = i / GW, c = i - t * GW;
        const size_t r = KDA ? tok(t) * DK + c : tok(t);
        const float al = a.alpha[r];
        a.dalpha[r] = __logf(al) > kFloor ? dL[t * LP + c] / al : 0.f;
    }
    if (tid < n) {
        float db = ((dBp[tid] + dBp[kC + tid]) + dBp[2 * kC + tid]) + dBp[3 * kC + tid];
        for (int sl = 0; sl < a.nsl_chain; ++sl) db += a.ws[W.dbp + static_cast<size_t>(sl) * a.B * a.Tw * a.H + wtok(tid)];
        a.dbeta[tok(tid)] = db;
    }
}

// ---------------------------------------------------------------- bwd_floor
// dalpha where the log floor is active (alpha_m ~ 0).  Every term of
// dlog alpha_m that depends on alpha_m carries it as a factor: the pairs
// s < m <= t (through E(t,s,c)), the state terms of the tokens t >= m
// (through e0) and t < m (through ek), and eE.  bwd_local's per-token sums
// also hold terms free of alpha_m, which cancel in dlog alpha_m but leave
// rounding that a division by alpha_m would magnify.  Here the terms that
// carry alpha_m are summed directly, each with alpha_m taken out of its
// exponent (every exponent stays <= 0), per channel c (g = floored log-gate):
//   dalpha_mc = sum_{t>=m} exp(G_tc - G_mc) sum_{s<m} (M_ts k_tc + N_ts q_tc) k_sc exp(G_{m-1},c - G_sc)
//             + exp(-g_mc) [ sum_{t>=m} (dK0_tc k_tc + dQ0_tc q_tc) e0_tc
//                            + sum_{t<m} dKt_tc k_tc ek_tc + (sum_j dS_end[c,j] S[c,j]) eE_c ]
// (GDN sums it over the channels).  The bracket's terms all carry exp(g_mc),
// so exp(-g_mc) restores them (where e0 or ek underflowed the restored term
// is below e^-47).  One workgroup per (b, h, chunk); chunks without a floored
// gate return at once.  All sums run in a fixed order (deterministic).
constexpr int kFT = 1024;  // threads of bwd_floor (few accumulators per thread)
constexpr int kJB = 16;   // value columns per staged block
template <int DK>
constexpr int floor_cb() { return DK < 64 ? DK : 64; }  // channels per pass
template <int DK>
constexpr int floor_stage() {
    constexpr int SP = kJB + 1, CP = floor_cb<DK>() + 1;
    return (3 * kC * SP + 2 * floor_cb<DK>() * SP) > kC * CP ? (3 * kC * SP + 2 * floor_cb<DK>() * SP) : kC * CP;
}
template <int DK>
constexpr int floor_lds() {
    constexpr int CB = floor_cb<DK>(), CP = CB + 1;
    return 4 * (2 * kC * kTP + floor_stage<DK>() + 5 * kC * CP + 3 * CB + 3 * kC);
}
template <int DK, bool KDA, typename InT>
__global__ __launch_bounds__(kFT) void bwd_floor(Args a) {
    constexpr int CB = floor_cb<DK>(), CP = CB + 1, SP = kJB + 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x / a.nr, ch = a.c0 + static_cast<int>(blockIdx.x - bh * a.nr);
    const Ws W(a.B, a.Tw, a.H, DK, a.DV);
    if (reinterpret_cast<const int*>(a.ws + W.fl)[a.wc(bh, ch)] == 0) return;
    extern __shared__ float sm[];
    float* Mm = sm;                          // [64][kTP] beta dA (s < t)
    float* Nm = Mm + kC * kTP;               // [64][kTP] dP (s <= t)
    float* Ust = Nm + kC * kTP;              // staging: U, dX, dO [64][SP]; S, dS_end [CB][SP]
    float* Xst = Ust + kC * SP;
    float* Ost = Xst + kC * SP;
    float* Sst = Ost + kC * SP;
    float* Dst = Sst + CB * SP;
    float* F2 = Ust;                         // [64][CP] after the staging: the ek terms, then k exp(...)
    float* Kb = Ust + floor_stage<DK>();     // [64][CP] k of the pass's channels
    float* Qb = Kb + kC * CP;                // [64][CP] q
    float* Gb = Qb + kC * CP;                // [64][CP] cumulative log-gate
    float* gb = Gb + kC * CP;                // [64][CP] log-gate (floored)
    float* F1 = gb + kC * CP;                // [64][CP] the e0 terms, then the bracket
    float* dE = F1 + kC * CP;                // [CB] sum_j dS_end S
    float* eE = dE + CB;                     // [CB] exp(G_end)
    float* vv = eE + CB;                     // [CB] GDN: one token's terms per channel
    float* Bs = vv + CB;                     // [64] beta
    float* dA = Bs + kC;                     // [64] GDN: dalpha per token
    int* mrow = reinterpret_cast<int*>(dA + kC);  // [64] a floored gate in row m (this pass)

    const int b = bh / a.H, h = bh - b * a.H;
    const int t0c = ch * kC, n = min(kC, a.T - t0c);
    const InT* q = static_cast<const InT*>(a.q);
    const InT* k = static_cast<const InT*>(a.k);
    const InT* dO = static_cast<const InT*>(a.dO);
    auto tok = [&](int t) { return (static_cast<size_t>(b) * a.T + t0c + t) * a.H + h; };
    const float* Sg = a.ws + W.ck + a.wc(bh, ch) * DK * a.DV;
    const float* Dg = a.ws + W.dck + a.wc(bh, ch) * DK * a.DV;
    if (tid < kC) {
        Bs[tid] = tid < n ? a.beta[tok(tid)] : 0.f;
        dA[tid] = 0.f;
    }
    auto stage_tok = [&](int jb) {  // U, dX, dO of the chunk's rows, columns jb .. jb + 15
        for (int i = tid; i < kC * kJB; i += kFT) {
            const int t = i / kJB, j = i - t * kJB;
            float u = 0.f, x = 0.f, o = 0.f;
            if (t < n) {
                const size_t r = a.wt(b, t0c + t, h) * a.DV + jb + j;  // workspace row
                u = a.ws[W.u + r];
                x = a.ws[W.dx + r];
                o = ld(dO + tok(t) * a.DV + jb + j);
            }
            Ust[t * SP + j] = u;
            Xst[t * SP + j] = x;
            Ost[t * SP + j] = o;
        }
    };
    // M = beta dA = -beta dX U^T (s < t), N = dP = scale dO U^T (s <= t)
    constexpr int PPT = kC * kC / kFT;
    float am[PPT], an[PPT];
#pragma unroll
    for (int x = 0; x < PPT; ++x) am[x] = an[x] = 0.f;
    for (int jb = 0; jb < a.DV; jb += kJB) {
        __syncthreads();
        stage_tok(jb);
        __syncthreads();
#pragma unroll
        for (int x = 0; x < PPT; ++x) {
            const int p = tid + x * kFT, t = p >> 6, s2 = p & 63;
#pragma unroll 4
            for (int j = 0; j < kJB; ++j) {
                const float us = Ust[s2 * SP + j];
                am[x] += Xst[t * SP + j] * us;
                an[x] += Ost[t * SP + j] * us;
            }
        }
    }
#pragma unroll
    for (int x = 0; x < PPT; ++x) {
        const int p = tid + x * kFT, t = p >> 6, s2 = p & 63;
        Mm[t * kTP + s2] = s2 < t ? -Bs[t] * am[x] : 0.f;
        Nm[t * kTP + s2] = s2 <= t ? a.scale * an[x] : 0.f;
    }
    constexpr int EPT = (kC * CB + kFT - 1) / kFT;
    for (int cb = 0; cb < DK; cb += CB) {
        __syncthreads();  // the previous pass is done with every array
        if (tid < kC) mrow[tid] = 0;
        for (int i = tid; i < kC * CB; i += kFT) {
            const int t = i / CB, c = i - t * CB;
            float kv = 0.f, qv = 0.f, lg = 0.f;
            if (t < n) {
                const size_t r = tok(t);
                kv = ld(k + r * DK + cb + c);
                qv = ld(q + r * DK + cb + c);
                lg = fmaxf(__logf(KDA ? a.alpha[r * DK + cb + c] : a.alpha[r]), kFloor);
            }
            Kb[t * CP + c] = kv;
            Qb[t * CP + c] = qv;
            gb[t * CP + c] = lg;
        }
        __syncthreads();
        for (int i = tid; i < kC * CB; i += kFT) {
            const int t = i / CB, c = i - t * CB;
            if (t < n && gb[t * CP + c] == kFloor) mrow[t] = 1;
        }
        for (int c = wave; c < CB; c += kFT / 64) {  // cumulative log-gate: a wave per channel, lane = token
            const float g = wave_prefix_sum(gb[lane * CP + c]);
            Gb[lane * CP + c] = g;
            if (lane == kC - 1) eE[c] = __expf(g);
        }
        // dQ0 = scale dO S^T, dK0 = -beta dX S^T, dKt = U dS_end^T of the pass's channels
        float aq[EPT], ak[EPT], at[EPT];
#pragma unroll
        for (int x = 0; x < EPT; ++x) aq[x] = ak[x] = at[x] = 0.f;
        float de = 0.f;
        for (int jb = 0; jb < a.DV; jb += kJB) {
            __syncthreads();
            stage_tok(jb);
            for (int i = tid; i < CB * kJB; i += kFT) {
                const int c = i / kJB, j = i - c * kJB;
                Sst[c * SP + j] = Sg[static_cast<size_t>(cb + c) * a.DV + jb + j];
                Dst[c * SP + j] = Dg[static_cast<size_t>(cb + c) * a.DV + jb + j];
            }
            __syncthreads();
#pragma unroll
            for (int x = 0; x < EPT; ++x) {
                const int p = tid + x * kFT;
                if (p >= kC * CB) break;
                const int t = p / CB, c = p - t * CB;
#pragma unroll 4
                for (int j = 0; j < kJB; ++j) {
                    const float sv = Sst[c * SP + j], dv = Dst[c * SP + j];
                    aq[x] += Ost[t * SP + j] * sv;
                    ak[x] += Xst[t * SP + j] * sv;
                    at[x] += Ust[t * SP + j] * dv;
                }
            }
            if (tid < CB) {
#pragma unroll 4
                for (int j = 0; j < kJB; ++j) de += Dst[tid * SP + j] * Sst[tid * SP + j];
            }
        }
        __syncthreads();  // the staging is consumed: F2 takes its place
#pragma unroll
        for (int x = 0; x < EPT; ++x) {
            const int p = tid + x * kFT;
            if (p >= kC * CB) break;
            const int t = p / CB, c = p - t * CB;
            const float kv = Kb[t * CP + c], qv = Qb[t * CP + c], G = Gb[t * CP + c];
            const float dQ0 = a.scale * aq[x], dK0 = -Bs[t] * ak[x], dKt = at[x];
            F1[t * CP + c] = (dK0 * kv + dQ0 * qv) * __expf(G);
            F2[t * CP + c] = dKt * kv * __expf(Gb[(kC - 1) * CP + c] - G);
        }
        if (tid < CB) dE[tid] = de;
        __syncthreads();
        // bracket[m] = sum_{t >= m} F1 + sum_{t < m} F2 + dE eE (the ek sum
        // runs over the lanes before m only: no term of row m enters it)
        for (int c = wave; c < CB; c += kFT / 64) {
            const float f1 = F1[lane * CP + c];
            const float f2 = __shfl_up(F2[lane * CP + c], 1);
            const float v = wave_suffix_sum(f1) + wave_prefix_sum(lane > 0 ? f2 : 0.f) + dE[c] * eE[c];
            F1[lane * CP + c] = v;
        }
        __syncthreads();
        for (int m = 0; m < n; ++m) {
            if (!mrow[m]) continue;  // uniform: LDS value, read after a barrier
            // F2 <- k_sc exp(G_{m-1},c - G_sc) for s < m (each factor <= 1)
            for (int i = tid; i < kC * CB; i += kFT) {
                const int s2 = i / CB, c = i - s2 * CB;
                const float gm1 = m > 0 ? Gb[(m - 1) * CP + c] : 0.f;
                F2[s2 * CP + c] = s2 < m ? Kb[s2 * CP + c] * __expf(gm1 - Gb[s2 * CP + c]) : 0.f;
            }
            __syncthreads();
            // channels c = wave + NW x per wave, lane = t >= m
            constexpr int NW = kFT / 64;
            constexpr int CPW = (CB + NW - 1) / NW;
            float accm[CPW], accn[CPW];
#pragma unroll
            for (int x = 0; x < CPW; ++x) accm[x] = accn[x] = 0.f;
            const int t = lane;
            if (t >= m && t < n) {
#pragma unroll 2
                for (int s2 = 0; s2 < m; ++s2) {
                    const float mts = Mm[t * kTP + s2], nts = Nm[t * kTP + s2];
#pragma unroll
                    for (int x = 0; x < CPW; ++x) {
                        const int c = wave + NW * x;
                        if (c < CB) {
                            const float as = F2[s2 * CP + c];
                            accm[x] += mts * as;
                            accn[x] += nts * as;
                        }
                    }
                }
            }
#pragma unroll
            for (int x = 0; x < CPW; ++x) {
                const int c = wave + NW * x;
                if (c >= CB) continue;
                float y = 0.f;
                if (t >= m && t < n)
                    y = __expf(Gb[t * CP + c] - Gb[m * CP + c]) * (Kb[t * CP + c] * accm[x] + Qb[t * CP + c] * accn[x]);
                y = wave_sum(y);
                if (lane == 0) {
                    const float gm = gb[m * CP + c];
                    const float v = y + __expf(-gm) * F1[m * CP + c];
                    if constexpr (KDA) {
                        if (gm == kFloor) a.dalpha[tok(m) * DK + cb + c] = v;
                    } else {
                        vv[c] = v;
                    }
                }
            }
            __syncthreads();
            if constexpr (!KDA) {
                if (tid == 0) {
                    float sum = dA[m];
                    for (int c = 0; c < CB; ++c) sum += vv[c];
                    dA[m] = sum;
                }
            }
            __syncthreads();
        }
    }
    if constexpr (!KDA) {
        __syncthreads();
        if (tid < n && mrow[tid]) a.dalpha[tok(tid)] = dA[tid];
    }
}

template <int DK, bool KDA>
constexpr int prep_lds() { return 4 * (2 * kC * (DK + 1) + kC * ((KDA ? DK : 1) + 1) + 2 * kC * kTP + kC); }
template <int DK, int FS>
constexpr int fwd_lds() { return 4 * (2 * kC * (DK + 1) + kC * kTP + DK * FS + 2 * kC * FS + DK + kC); }
template <int DK, int FS>
constexpr int chain_lds() { return 4 * (2 * kC * (DK + 1) + kC * kTP + 2 * DK * FS + 4 * kC * FS + DK + kC); }
template <int DK>
constexpr int dout_lds() { return 4 * (kC * (DK + 1) + kC * kTP + kC * 65); }
template <int DK, bool KDA>
constexpr int local_lds() {
    constexpr int SP = 17;
    constexpr int un = (2 * DK * SP + 3 * kC * SP) > 2 * kC * kTP ? (2 * DK * SP + 3 * kC * SP) : 2 * kC * kTP;
    return 4 * (2 * kC * (DK + 1) + kC * ((KDA ? DK : 1) + 1) + kC * kTP + un + 3 * kC + 2 * DK + 8 * kC + 32);
}

template <int DK, bool KDA, typename InT>
hipError_t run(Args a, hipStream_t s, int rc) {
    static_assert(local_lds<DK, KDA>() <= 160 * 1024 && chain_lds<DK, kSl>() <= 160 * 1024 &&
                  prep_lds<DK, KDA>() <= 160 * 1024 && fwd_lds<DK, 64>() <= 160 * 1024 &&
                  dout_lds<DK>() <= 160 * 1024 && floor_lds<DK>() <= 160 * 1024, "LDS budget");
    auto set = [](const void* f, int bytes) {
        return bytes > 64 * 1024 ? hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes)
                                 : hipSuccess;
    };
    hipError_t e;
    const unsigned long long h8 = (static_cast<unsigned long long>(a.B) * a.H + 7) / 8 * 8;
    if (!grid_fits(static_cast<unsigned long long>(a.B) * a.H * a.nch, kNT) || !grid_fits(h8 * (a.DV / kSl), kNT))
        return hipErrorInvalidConfiguration;
    const unsigned heads8 = static_cast<unsigned>(h8);  // slice grids: whole groups of 8 heads
    // The checkpoint chain takes the widest slices (64, 32 or 16 columns)
    // that still put a workgroup on every CU; the reverse chain always takes
    // 16 (at 16 it has the registers to load the next chunk's image during
    // the current one, which costs less than the extra rounds of workgroups).
    const long long BH = static_cast<long long>(a.B) * a.H;
    const int FSF = a.DV >= 64 && BH * (a.DV / 64) >= 256 ? 64 : a.DV >= 32 && BH * (a.DV / 32) >= 256 ? 32 : 16;
    a.nsl_chain = a.DV / kSl;
    const unsigned fwd_slices = heads8 * static_cast<unsigned>(a.DV / FSF);
    const unsigned chain_slices = heads8 * static_cast<unsigned>(a.DV / kSl);
    const void* fwd = FSF == 64 ? reinterpret_cast<const void*>(bwd_fwd<DK, KDA, InT, 64>)
                    : FSF == 32 ? reinterpret_cast<const void*>(bwd_fwd<DK, KDA, InT, 32>)
                                : reinterpret_cast<const void*>(bwd_fwd<DK, KDA, InT, 16>);
    if ((e = set(reinterpret_cast<const void*>(bwd_prep<DK, KDA, InT>), prep_lds<DK, KDA>())) != hipSuccess) return e;
    if ((e = set(reinterpret_cast<const void*>(bwd_dout<DK, KDA, InT>), dout_lds<DK>())) != hipSuccess) return e;
    if ((e = set(fwd, FSF == 64 ? fwd_lds<DK, 64>() : FSF == 32 ? fwd_lds<DK, 32>() : fwd_lds<DK, 16>())) != hipSuccess)
        return e;
    if ((e = set(reinterpret_cast<const void*>(bwd_chain<DK, KDA, InT, kSl>), chain_lds<DK, kSl>())) != hipSuccess) return e;
    if ((e = set(reinterpret_cast<const void*>(bwd_local<DK, KDA, InT>), local_lds<DK, KDA>())) != hipSuccess) return e;
    if ((e = set(reinterpret_cast<const void*>(bwd_floor<DK, KDA, InT>), floor_lds<DK>())) != hipSuccess) return e;
    // the chunk-local forward work of a range (prep, and the checkpoint chain)
    auto forward = [&](const Args& r) {
        const unsigned per_chunk = static_cast<unsigned>(static_cast<unsigned long long>(r.B) * r.H * r.nr);
        hipLaunchKernelGGL((bwd_prep<DK, KDA, InT>), dim3(per_chunk), dim3(kNT), (prep_lds<DK, KDA>()), s, r);
        if (FSF == 64)
            hipLaunchKernelGGL((bwd_fwd<DK, KDA, InT, 64>), dim3(fwd_slices), dim3(kNT), (fwd_lds<DK, 64>()), s, r);
        else if (FSF == 32)
            hipLaunchKernelGGL((bwd_fwd<DK, KDA, InT, 32>), dim3(fwd_slices), dim3(kNT), (fwd_lds<DK, 32>()), s, r);
        else
            hipLaunchKernelGGL((bwd_fwd<DK, KDA, InT, 16>), dim3(fwd_slices), dim3(kNT), (fwd_lds<DK, 16>()), s, r);
        return hipGetLastError();
    };
    // the gradient work of a range whose forward work is in the workspace
    auto reverse = [&](const Args& r) {
        const unsigned per_chunk = static_cast<unsigned>(static_cast<unsigned long long>(r.B) * r.H * r.nr);
        hipLaunchKernelGGL((bwd_dout<DK, KDA, InT>), dim3(per_chunk), dim3(kNT), (dout_lds<DK>()), s, r);
        hipLaunchKernelGGL((bwd_chain<DK, KDA, InT, kSl>), dim3(chain_slices), dim3(kNT), (chain_lds<DK, kSl>()), s, r);
        hipLaunchKernelGGL((bwd_local<DK, KDA, InT>), dim3(per_chunk), dim3(kNT), (local_lds<DK, KDA>()), s, r);
        hipLaunchKernelGGL((bwd_floor<DK, KDA, InT>), dim3(per_chunk), dim3(kFT), (floor_lds<DK>()), s, r);
        return hipGetLastError();
    };
    if (rc >= a.nch) {  // the whole sequence at once
        a.c0 = 0; a.nr = a.nch; a.Tw = a.T;
        a.s_in = a.s0; a.s_end = nullptr; a.ds_end = a.dsT; a.ds_start = a.ds0;
        if ((e = forward(a)) != hipSuccess) return e;
        return reverse(a);
    }
    // Ranges of rc chunks: the workspace holds one range.  A forward pass
    // keeps only the state at each range start; the reverse pass then runs
    // the ranges from the last, each from its start state (the last range's
    // forward work is still in the workspace), carrying the state gradient
    // from range to range.
    const int R = (a.nch + rc - 1) / rc;
    const size_t state = static_cast<size_t>(BH) * DK * a.DV;
    float* starts = a.ws + Ws(a.B, rc * kC, a.H, DK, a.DV).total;  // R - 1 states: ranges 1 .. R-1
    float* dcarry = starts + (R - 1) * state;                      // the state gradient between ranges
    auto range = [&](int r) {
        Args x = a;
        x.c0 = r * rc; x.nr = std::min(rc, a.nch - x.c0); x.Tw = rc * kC;
        x.s_in = r == 0 ? a.s0 : starts + (r - 1) * state;
        x.s_end = r + 1 < R ? starts + r * state : nullptr;
        x.ds_end = r + 1 == R ? a.dsT : dcarry;
        x.ds_start = r == 0 ? a.ds0 : dcarry;
        return x;
    };
    for (int r = 0; r < R; ++r)
        if ((e = forward(range(r))) != hipSuccess) return e;
    for (int r = R - 1; r >= 0; --r) {
        const Args x = range(r);
        if (r + 1 < R && (e = forward(x)) != hipSuccess) return e;
        if ((e = reverse(x)) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK>
hipError_t run_dk(int kda, int dtype, const Args& a, hipStream_t s, int rc) {
    if (dtype == GDR_DTYPE_BF16)
        return kda ? run<DK, true, bf16_t>(a, s, rc) : run<DK, false, bf16_t>(a, s, rc);
    return kda ? run<DK, true, float>(a, s, rc) : run<DK, false, float>(a, s, rc);
}

}  // namespace

size_t backward_workspace_floats(int B, int T, int H, int dk, int dv) {
    return Ws(B, T, H, dk, dv).total;
}

size_t backward_workspace_floats_ranged(int B, int T, int H, int dk, int dv, int rc) {
    const int nch = (T + kC - 1) / kC;
    if (rc >= nch) return Ws(B, T, H, dk, dv).total;
    const size_t state = static_cast<size_t>(B) * H * dk * dv;
    const int R = (nch + rc - 1) / rc;
    return Ws(B, rc * kC, H, dk, dv).total + static_cast<size_t>(R) * state;  // R - 1 starts + the carry
}

hipError_t launch_backward(int kda, int dtype, int B, int T, int H, int dk, int dv, float scale,
                           const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* state_in, const void* d_o,
                           const float* d_state_out, void* dq, void* dkk, void* dvv, float* dalpha,
                           float* dbeta, float* d_state_in, float* ws, size_t ws_floats, hipStream_t s) {
    // the widest chunk range the workspace holds (the whole sequence if it can)
    const int nch = (T + kC - 1) / kC;
    int rc = nch;
    if (ws_floats < Ws(B, T, H, dk, dv).total) {
        rc = 0;
        for (int c = nch - 1; c >= 1 && rc == 0; --c)
            if (backward_workspace_floats_ranged(B, T, H, dk, dv, c) <= ws_floats) rc = c;
        if (rc == 0) return hipErrorInvalidValue;
    }
    Args a;
    a.B = B; a.T = T; a.H = H; a.DV = dv; a.nch = (T + kC - 1) / kC;
    a.scale = scale;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.s0 = state_in;
    a.dO = d_o; a.dsT = d_state_out;
    a.dq = dq; a.dk = dkk; a.dv = dvv; a.dalpha = dalpha; a.dbeta = dbeta; a.ds0 = d_state_in;
    a.ws = ws;
    switch (dk) {
        case 16: return run_dk<16>(kda, dtype, a, s, rc);
        case 32: return run_dk<32>(kda, dtype, a, s, rc);
        case 64: return run_dk<64>(kda, dtype, a, s, rc);
        default: return run_dk<128>(kda, dtype, a, s, rc);
    }
}

}  // namespace gdr
