// Chunked prefill with bf16 inputs: every contraction on bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16 / 16x16x16_bf16, fp32 accumulation), the state
// in fp32 registers for the whole sequence.
//
// Method ("Super Apriel: One Checkpoint, Many Speeds", §2.A: GDN and KDA are
// recurrent mixers with a fixed-size state and a scalar resp. channel-wise
// gate).  For a chunk of n <= 64 tokens entering with state S, G_t is the
// cumulative log2-gate from the chunk start (per key channel for KDA) and the
// recurrence S_t = (I - beta_t k_t k_t^T) D_t S_{t-1} + beta_t k_t v_t^T
// unrolls exactly to
//     A_tj = beta_t sum_c k_tc k_jc 2^(G_tc - G_jc)     j <  t   (else 0)
//     P_tj =        sum_c q_tc k_jc 2^(G_tc - G_jc)     j <= t   (else 0)
//     X    = diag(beta) (V - Khat S),  Khat_t = k_t 2^G_t
//     U    = (I + A)^{-1} X
//     O    = scale (Qhat S + P U),     Qhat_t = q_t 2^G_t
//     S   <- diag(2^G_end) S + Ktil^T U,  Ktil_t = k_t 2^(G_end - G_t)
// (the WY form W = (I + A)^{-1} diag(beta) Khat is folded into X).
//
// U = (I + A)^{-1} X is a blocked forward substitution over the four 16-token
// blocks, U_r = D_r^{-1} (X_r - sum_{k<r} A_rk U_k), with the inverses D_r^{-1}
// of the unit lower triangular 16x16 diagonal blocks of I + A computed in fp32
// by forward substitution (one lane per column).
//
// Gates inside the contractions.  GDN: one scalar per token, so the MFMAs run
// on raw q and k and the factors 2^(G_t - G_j) <= 1, 2^G_t, 2^(G_end - G_t)
// scale their outputs.  KDA: the decay differs per channel and is folded into
// the operands around a per-channel reference R = G_end / 2, so every factor
// stays within 2^(|G_end| / 2); S is scaled by 2^R where it is rounded to bf16.
// log2(alpha) is floored at -115.4 (alpha ~ e^-80), so alpha == 0 is legal;
// KDA needs the total log-decay of a channel within one chunk above about -170.
//
// Mapping.  One workgroup per (b, h, slice of 16*NSW value columns); the value
// columns of S are independent, so the slices of a head run on different CUs
// (their block ids are congruent mod 8: one XCD, shared L2).  Waves 0..3 are
// "prep" waves, waves 4.. are "serial" waves owning 16 value columns each:
//   iteration i, phase 1: prep gates chunk i+1 into LDS buffer (i+1)&1 and
//                         prefetches chunk i+2; serial computes Khat S, X and
//                         U for chunk i from buffer i&1;
//   phase 2:              prep forms A, P and the D_r^{-1} of chunk i+1;
//                         serial forms O and updates S for chunk i.
// Two workgroup barriers per chunk.  The serial chain keeps S, X and U in
// MFMA registers: an fp32 accumulator tile holds rows 4g..4g+3 of column l%16
// in lane l (g = l/16), so two row tiles together are the B operand of a
// K=32 step whose k order is {4g..4g+3, 16+4g..16+4g+3}; the LDS operand of
// that step is read in the same k order, which keeps every product exact
// without any register shuffle.
#include "gdr_internal.h"

namespace gdr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;                 // chunk
constexpr int kPrepWaves = 4;
constexpr float kLog2Floor = -115.4f;  // log2(alpha) floor, alpha ~ e^-80

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// but leaves global loads in flight (a full __syncthreads also drains vmcnt,
// which would stall the prefetch of the next chunk).  Waves exchange data
// only through LDS in this kernel.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                      __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4 cvt4(const f32x4& x) {
    bf16x4 r;
    r[0] = static_cast<__bf16>(x[0]);
    r[1] = static_cast<__bf16>(x[1]);
    r[2] = static_cast<__bf16>(x[2]);
    r[3] = static_cast<__bf16>(x[3]);
    return r;
}
__device__ __forceinline__ bf16x8 cat8(const bf16x4& a, const bf16x4& b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 lds4(const bf16_t* p) {
    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ bf16x8 lds8(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
// k order {0..3, 16..19} relative to p: matches two stacked accumulator tiles.
__device__ __forceinline__ bf16x8 lds_perm(const bf16_t* p) { return cat8(lds4(p), lds4(p + 16)); }
__device__ __forceinline__ void st4(bf16_t* p, const f32x4& x) {
    *reinterpret_cast<uint2*>(p) = __builtin_bit_cast(uint2, cvt4(x));
}
__device__ __forceinline__ uint32_t bf_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DK, int NSW, bool KDA>
struct Layout {
    static constexpr int DKP = DK < 32 ? 32 : DK;  // contraction pad (dk = 16)
    static constexpr int PK = DKP + 8;             // pitch of [token][channel] tiles (bf16)
    static constexpr int PT = kC + 4;              // pitch of [channel][token] tiles (bf16)
    static constexpr int PD = 16 + 8;              // pitch of packed 16x16 tiles (bf16)
    static constexpr int TILE = 16 * PD * 2;       // bytes of one packed tile
    static constexpr int NPAIR = DK / 2;           // channel pairs
    static constexpr int TPP = 256 / NPAIR;        // lanes per pair (one wave segment)
    static constexpr int PPW = 64 / TPP;           // pairs per prep wave
    static constexpr int TPT = kC / TPP;           // tokens per lane
    // one chunk buffer (byte offsets)
    static constexpr int oKh = 0;                         // Khat [64][PK]
    static constexpr int oQh = oKh + kC * PK * 2;         // Qhat [64][PK]
    static constexpr int oKt = oQh + kC * PK * 2;         // Ktil^T [DK][PT]
    static constexpr int oP = oKt + DK * PT * 2;          // P, 10 lower tiles
    static constexpr int oA = oP + 10 * TILE;             // -A, 6 off-diagonal tiles
    static constexpr int oD = oA + 6 * TILE;              // D_r^{-1}, 4 tiles
    static constexpr int oBeta = oD + 4 * TILE;           // beta_t [64]
    static constexpr int oEg = oBeta + kC * 4;            // GDN 2^G_t [64]
    static constexpr int oEk = oEg + kC * 4;              // GDN 2^(G_end - G_t) [64]
    static constexpr int oGend = oEk + kC * 4;            // 2^G_end per channel (GDN: [0])
    static constexpr int oSref = oGend + DK * 4;          // KDA 2^R per channel
    static constexpr int BUF = ((oSref + DK * 4) + 15) / 16 * 16;
    // prep-private
    static constexpr int oKc = 2 * BUF;                   // KDA Kcheck [64][PK]
    static constexpr int oG = oKc + (KDA ? kC * PK * 2 : 0);  // GDN G_t [64]
    static constexpr int PS = 20;                         // pitch of the fp32 scratch tiles
    static constexpr int oScr = oG + kC * 4;              // fp32 diagonal tiles [4][16][PS]
    static constexpr int bytes = oScr + kPrepWaves * 16 * PS * 4;
    static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
    static_assert(TPT >= 2 && TPT % 2 == 0 && TPP <= 64, "token split");
};

__device__ __forceinline__ int ptile(int rt, int ct) { return rt * (rt + 1) / 2 + ct; }  // ct <= rt
__device__ __forceinline__ int atile(int rt, int ct) { return rt * (rt - 1) / 2 + ct; }  // ct < rt

template <int DK, int NSW, bool KDA>
__global__ __launch_bounds__(64 * (kPrepWaves + NSW)) void prefill_bf16_kernel(
    int B, int T, int H, int DV, int NS, float scale, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, const float* __restrict__ state_in,
    float* __restrict__ state_out, bf16_t* __restrict__ o) {
    using L = Layout<DK, NSW, KDA>;
    constexpr int DVS = 16 * NSW;
    constexpr int NRT = DK / 16;          // 16-row tiles of S
    constexpr int NKS = L::DKP / 32;      // K=32 steps over dk
    constexpr int TPT = L::TPT;

    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    const int BH = B * H;
    const int grp = blockIdx.x / (8 * NS);
    const int rem = blockIdx.x - grp * 8 * NS;
    const int bh = grp * 8 + (rem & 7);
    const int slice = rem >> 3;
    if (bh >= BH) return;  // whole block exits before any barrier
    const int b = bh / H, h = bh - b * H;
    const int nch = (T + kC - 1) / kC;
    const bool prep = wave < kPrepWaves;

    auto bfp = [&](int c, int off) { return reinterpret_cast<bf16_t*>(smem + (c & 1) * L::BUF + off); };
    auto f32p = [&](int c, int off) { return reinterpret_cast<float*>(smem + (c & 1) * L::BUF + off); };
    bf16_t* Kc = reinterpret_cast<bf16_t*>(smem + L::oKc);  // used by KDA only
    float* sG = reinterpret_cast<float*>(smem + L::oG);

    if constexpr (L::DKP != DK) {  // zero the contraction padding once (both buffers, Kc)
        constexpr int W = L::DKP - DK;
        for (int idx = tid; idx < 2 * kC * W; idx += blockDim.x) {
            const int c = idx / (kC * W), r = idx % (kC * W);
            const int t = r / W, col = DK + r % W;
            bfp(c, L::oKh)[t * L::PK + col] = 0;
            bfp(c, L::oQh)[t * L::PK + col] = 0;
            if (KDA && c == 0) Kc[t * L::PK + col] = 0;
        }
    }

    // ================= prep-wave work =================
    const int pl = lane / L::TPP, tg = lane % L::TPP;
    const int ch = 2 * (wave * L::PPW + pl);
    const int tlo = tg * TPT;
    struct PrepIn {
        float a0[TPT], a1[TPT], bt[TPT];
        uint32_t kw[TPT], qw[TPT];
    };
    auto prep_load = [&](int c, PrepIn& R) {
        const int t0 = c * kC, nn = min(kC, T - t0);
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
            const int tc = min(tlo + u, nn - 1);
            const size_t gi = (static_cast<size_t>(b) * T + t0 + tc) * H + h;
            if constexpr (KDA) {
                const float2 a2 = *reinterpret_cast<const float2*>(alpha + gi * DK + ch);
                R.a0[u] = a2.x;
                R.a1[u] = a2.y;
            } else {
                R.a0[u] = R.a1[u] = alpha[gi];
            }
            R.bt[u] = beta[gi];
            R.kw[u] = *reinterpret_cast<const uint32_t*>(k + gi * DK + ch);
            R.qw[u] = *reinterpret_cast<const uint32_t*>(q + gi * DK + ch);
        }
    };

    // Gates and gated operands of chunk c into buffer c & 1.  Lane = (channel
    // pair, run of TPT tokens); the TPP lanes of a pair are one wave segment,
    // so the cumulative sum over the chunk is an in-wave scan.
    auto prep_gate = [&](int c, const PrepIn& R) {
        const int n = min(kC, T - c * kC);
        float g0[TPT], g1[TPT];
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
            const bool valid = tlo + u < n;
            const float l0 = valid ? fmaxf(__log2f(R.a0[u]), kLog2Floor) : 0.f;
            const float l1 = KDA ? (valid ? fmaxf(__log2f(R.a1[u]), kLog2Floor) : 0.f) : l0;
            acc0 += l0;
            acc1 += l1;
            g0[u] = acc0;
            g1[u] = acc1;
        }
        float inc0 = acc0, inc1 = acc1;
#pragma unroll
        for (int d = 1; d < L::TPP; d <<= 1) {
            const float y0 = __shfl_up(inc0, d, L::TPP), y1 = __shfl_up(inc1, d, L::TPP);
            if (tg >= d) { inc0 += y0; inc1 += y1; }
        }
        const float off0 = inc0 - acc0, off1 = inc1 - acc1;
        const float end0 = __shfl(inc0, L::TPP - 1, L::TPP), end1 = __shfl(inc1, L::TPP - 1, L::TPP);
        bf16_t* Kh = bfp(c, L::oKh);
        bf16_t* Qh = bfp(c, L::oQh);
        bf16_t* Kt = bfp(c, L::oKt);
        const bool lead = (wave == 0 && pl == 0);  // one pair writes the per-token vectors
        if (lead) {
            float* sb = f32p(c, L::oBeta);
#pragma unroll
            for (int u = 0; u < TPT; ++u) sb[tlo + u] = tlo + u < n ? R.bt[u] : 0.f;
        }
        uint32_t kt0[TPT / 2], kt1[TPT / 2];
        if constexpr (KDA) {
            const float ref0 = 0.5f * end0, ref1 = 0.5f * end1;
            const float ce0 = exp2f(end0 - ref0), ce1 = exp2f(end1 - ref1);
            if (tg == 0) {
                f32p(c, L::oGend)[ch] = exp2f(end0);
                f32p(c, L::oGend)[ch + 1] = exp2f(end1);
                f32p(c, L::oSref)[ch] = exp2f(ref0);
                f32p(c, L::oSref)[ch + 1] = exp2f(ref1);
            }
#pragma unroll
            for (int u = 0; u < TPT; ++u) {
                const int t = tlo + u;
                const bool valid = t < n;
                const uint32_t kw = valid ? R.kw[u] : 0u, qw = valid ? R.qw[u] : 0u;
                const float k0 = bf_lo(kw), k1 = bf_hi(kw), q0 = bf_lo(qw), q1 = bf_hi(qw);
                const float up0 = exp2f(off0 + g0[u] - ref0), up1 = exp2f(off1 + g1[u] - ref1);
                const float dn0 = __builtin_amdgcn_rcpf(up0), dn1 = __builtin_amdgcn_rcpf(up1);
                bf16x2 x;
                x[0] = static_cast<__bf16>(k0 * up0);
                x[1] = static_cast<__bf16>(k1 * up1);
                *reinterpret_cast<bf16x2*>(Kh + t * L::PK + ch) = x;
                x[0] = static_cast<__bf16>(q0 * up0);
                x[1] = static_cast<__bf16>(q1 * up1);
                *reinterpret_cast<bf16x2*>(Qh + t * L::PK + ch) = x;
                x[0] = static_cast<__bf16>(k0 * dn0);
                x[1] = static_cast<__bf16>(k1 * dn1);
                *reinterpret_cast<bf16x2*>(Kc + t * L::PK + ch) = x;
                const uint32_t b0 = bf_bits(k0 * dn0 * ce0), b1 = bf_bits(k1 * dn1 * ce1);
                if (u & 1) { kt0[u >> 1] |= b0 << 16; kt1[u >> 1] |= b1 << 16; }
                else { kt0[u >> 1] = b0; kt1[u >> 1] = b1; }
            }
        } else {
            if (lead) {
                float* eg = f32p(c, L::oEg);
                float* ek = f32p(c, L::oEk);
#pragma unroll
                for (int u = 0; u < TPT; ++u) {
                    const float G = off0 + g0[u];
                    sG[tlo + u] = G;
                    eg[tlo + u] = exp2f(G);
                    ek[tlo + u] = exp2f(end0 - G);
                }
                if (tg == 0) f32p(c, L::oGend)[0] = exp2f(end0);
            }
#pragma unroll
            for (int u = 0; u < TPT; ++u) {
                const int t = tlo + u;
                const bool valid = t < n;
                const uint32_t kw = valid ? R.kw[u] : 0u, qw = valid ? R.qw[u] : 0u;
                *reinterpret_cast<uint32_t*>(Kh + t * L::PK + ch) = kw;
                *reinterpret_cast<uint32_t*>(Qh + t * L::PK + ch) = qw;
                if (u & 1) { kt0[u >> 1] |= kw << 16; kt1[u >> 1] |= kw & 0xffff0000u; }
                else { kt0[u >> 1] = kw & 0xffffu; kt1[u >> 1] = kw >> 16; }
            }
        }
#pragma unroll
        for (int u = 0; u < TPT / 2; ++u) {
            *reinterpret_cast<uint32_t*>(Kt + ch * L::PT + tlo + 2 * u) = kt0[u];
            *reinterpret_cast<uint32_t*>(Kt + (ch + 1) * L::PT + tlo + 2 * u) = kt1[u];
        }
    };

    // A, P and the diagonal-block inverses of chunk c (buffer c & 1).  The
    // tile products run transposed, C^T = Kr M^T, so a lane ends up with 4
    // consecutive j of one row t and stores 8 bytes.
    auto prep_ap = [&](int c) {
        const bf16_t* Kh = bfp(c, L::oKh);
        const bf16_t* Qh = bfp(c, L::oQh);
        const bf16_t* Kr = KDA ? Kc : Kh;  // right factor (j side)
        const float* sb = f32p(c, L::oBeta);
        bf16_t* Pt = bfp(c, L::oP);
        bf16_t* At = bfp(c, L::oA);
        bf16_t* Dt = bfp(c, L::oD);
        float* scr = reinterpret_cast<float*>(smem + L::oScr) + wave * 16 * L::PS;
        // tile 0: this wave's diagonal A tile; then 4 of the 16 others
        // (6 off-diagonal A tiles, then 10 P tiles), round-robin over waves
#pragma unroll
        for (int m = 0; m < 5; ++m) {
            bool isP;
            int rt, ct;
            if (m == 0) {
                isP = false;
                rt = ct = wave;
            } else {
                const int x = wave + 4 * (m - 1);  // 0..15
                if (x < 6) {
                    isP = false;
                    rt = x < 1 ? 1 : (x < 3 ? 2 : 3);
                    ct = x - rt * (rt - 1) / 2;
                } else {
                    isP = true;
                    const int y = x - 6;
                    rt = y < 1 ? 0 : (y < 3 ? 1 : (y < 6 ? 2 : 3));
                    ct = y - rt * (rt + 1) / 2;
                }
            }
            f32x4 acc = zero4();
            const bf16_t* M = isP ? Qh : Kh;
#pragma unroll
            for (int s = 0; s < NKS; ++s)
                acc = mfma32(lds8(Kr + (16 * ct + lr) * L::PK + 32 * s + 8 * lg),
                             lds8(M + (16 * rt + lr) * L::PK + 32 * s + 8 * lg), acc);
            const int t = 16 * rt + lr;
            const float bt = sb[t];
            f32x4 val;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 16 * ct + 4 * lg + i;
                float x = acc[i];
                if constexpr (!KDA) x *= exp2f(fminf(sG[t] - sG[j], 0.f));
                val[i] = isP ? (j <= t ? x : 0.f) : (j < t ? bt * x : 0.f);
            }
            if (m == 0) {
                *reinterpret_cast<float4*>(scr + lr * L::PS + 4 * lg) =
                    make_float4(val[0], val[1], val[2], val[3]);
            } else if (isP) {
                st4(Pt + ptile(rt, ct) * 16 * L::PD + lr * L::PD + 4 * lg, val);
            } else {
                st4(At + atile(rt, ct) * 16 * L::PD + lr * L::PD + 4 * lg, -val);
            }
        }
        // D_w^{-1} = (I + A_ww)^{-1}: lane c solves column c by forward substitution.
        if (lane < 16) {
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = (i == lane) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) acc -= scr[i * L::PS + j] * x[j];
                x[i] = acc;
            }
            bf16_t* Dw = Dt + wave * 16 * L::PD;
#pragma unroll
            for (int i = 0; i < 16; ++i) Dw[i * L::PD + lane] = static_cast<bf16_t>(bf_bits(x[i]));
        }
    };

    // ================= serial-wave work =================
    const int sw = wave - kPrepWaves;
    const int col0 = slice * DVS + 16 * sw;  // first value column of this wave
    f32x4 S[NRT];
    f32x4 Uf[4];
    bf16x4 Ub[4];
    bf16x8 bS[NKS];
    const size_t sbase = static_cast<size_t>(bh) * DK * DV;
    auto serial_vload = [&](int c, bf16_t (&V)[4][4]) {
        const int t0 = c * kC, nn = min(kC, T - t0);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tc = min(16 * rt + 4 * lg + i, nn - 1);
                V[rt][i] = v[((static_cast<size_t>(b) * T + t0 + tc) * H + h) * DV + col0 + lr];
            }
    };
    // B operands of S for the K=32 steps over dk (KDA: scaled by 2^R per row).
    auto build_bS = [&](int c) {
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            f32x4 lo = S[2 * s];
            f32x4 hi = (2 * s + 1 < NRT) ? S[2 * s + 1] : zero4();
            if constexpr (KDA) {
                const float* sr = f32p(c, L::oSref);
                const float4 f0 = *reinterpret_cast<const float4*>(sr + 32 * s + 4 * lg);
                lo[0] *= f0.x; lo[1] *= f0.y; lo[2] *= f0.z; lo[3] *= f0.w;
                if (2 * s + 1 < NRT) {
                    const float4 f1 = *reinterpret_cast<const float4*>(sr + 32 * s + 16 + 4 * lg);
                    hi[0] *= f1.x; hi[1] *= f1.y; hi[2] *= f1.z; hi[3] *= f1.w;
                }
            }
            bS[s] = cat8(cvt4(lo), cvt4(hi));
        }
    };
    // phase 1: Khat S -> X -> U (blocked forward substitution)
    auto serial_a = [&](int c, const bf16_t (&V)[4][4]) {
        build_bS(c);
        const bf16_t* Kh = bfp(c, L::oKh);
        const float* sb = f32p(c, L::oBeta);
        const float* eg = f32p(c, L::oEg);
        const bf16_t* At = bfp(c, L::oA);
        const bf16_t* Dt = bfp(c, L::oD);
        f32x4 X[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < NKS; ++s)
                acc = mfma32(lds_perm(Kh + (16 * rt + lr) * L::PK + 32 * s + 4 * lg), bS[s], acc);
            const float4 b4 = *reinterpret_cast<const float4*>(sb + 16 * rt + 4 * lg);
            float4 e4 = make_float4(1.f, 1.f, 1.f, 1.f);
            if constexpr (!KDA) e4 = *reinterpret_cast<const float4*>(eg + 16 * rt + 4 * lg);
            const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, ee[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) X[rt][i] = bb[i] * (bf16_to_f32(V[rt][i]) - ee[i] * acc[i]);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 w = X[rt];
#pragma unroll
            for (int kb = 0; kb < rt; ++kb)
                w = mfma16(lds4(At + atile(rt, kb) * 16 * L::PD + lr * L::PD + 4 * lg), Ub[kb], w);
            Uf[rt] = mfma16(lds4(Dt + rt * 16 * L::PD + lr * L::PD + 4 * lg), cvt4(w), zero4());
            Ub[rt] = cvt4(Uf[rt]);
        }
    };
    // phase 2: O = scale (Qhat S + P U) (computed transposed), and
    // S <- diag(2^G_end) S + Ktil^T U
    auto serial_b = [&](int c) {
        const int t0 = c * kC, n = min(kC, T - t0);
        const bf16_t* Qh = bfp(c, L::oQh);
        const bf16_t* Pt = bfp(c, L::oP);
        const bf16_t* Kt = bfp(c, L::oKt);
        const float* eg = f32p(c, L::oEg);
        const float* ek = f32p(c, L::oEk);
        const float* ge = f32p(c, L::oGend);
        const bf16x4 z4 = cvt4(zero4());
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            // O^T tile: rows = this wave's 16 value columns, columns = tokens 16 rt..
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < NKS; ++s)
                acc = mfma32(bS[s], lds_perm(Qh + (16 * rt + lr) * L::PK + 32 * s + 4 * lg), acc);
            if constexpr (!KDA) acc *= eg[16 * rt + lr];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (2 * s <= rt) {
                    const bf16x4 plo = lds4(Pt + ptile(rt, 2 * s) * 16 * L::PD + lr * L::PD + 4 * lg);
                    const bf16x4 phi = (2 * s + 1 <= rt)
                        ? lds4(Pt + ptile(rt, 2 * s + 1) * 16 * L::PD + lr * L::PD + 4 * lg) : z4;
                    acc = mfma32(cat8(Ub[2 * s], Ub[2 * s + 1]), cat8(plo, phi), acc);
                }
            }
            const int t = 16 * rt + lr;
            if (t < n)
                st4(o + ((static_cast<size_t>(b) * T + t0 + t) * H + h) * DV + col0 + 4 * lg, acc * scale);
        }
        bf16x8 bU[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if constexpr (KDA) {
                bU[s] = cat8(Ub[2 * s], Ub[2 * s + 1]);
            } else {
                const float4 k0 = *reinterpret_cast<const float4*>(ek + 32 * s + 4 * lg);
                const float4 k1 = *reinterpret_cast<const float4*>(ek + 32 * s + 16 + 4 * lg);
                f32x4 lo = Uf[2 * s], hi = Uf[2 * s + 1];
                lo[0] *= k0.x; lo[1] *= k0.y; lo[2] *= k0.z; lo[3] *= k0.w;
                hi[0] *= k1.x; hi[1] *= k1.y; hi[2] *= k1.z; hi[3] *= k1.w;
                bU[s] = cat8(cvt4(lo), cvt4(hi));
            }
        }
#pragma unroll
        for (int r = 0; r < NRT; ++r) {
            if constexpr (KDA) {
                const float4 g4 = *reinterpret_cast<const float4*>(ge + 16 * r + 4 * lg);
                S[r][0] *= g4.x; S[r][1] *= g4.y; S[r][2] *= g4.z; S[r][3] *= g4.w;
            } else {
                S[r] *= ge[0];
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
                S[r] = mfma32(lds_perm(Kt + (16 * r + lr) * L::PT + 32 * s + 4 * lg), bU[s], S[r]);
        }
    };

    // ================= pipeline =================
    // Each role runs its own loop: nch + 1 iterations with exactly two
    // workgroup barriers each, so the barriers pair up across roles while the
    // compiler keeps only one role's loop-carried registers live.
    if (prep) {
        PrepIn pin;
        if (nch > 0) prep_load(0, pin);
        for (int i = -1; i < nch; ++i) {
            if (i + 1 < nch) {
                prep_gate(i + 1, pin);
                if (i + 2 < nch) prep_load(i + 2, pin);  // in flight until the next iteration
            }
            lds_barrier();
            if (i + 1 < nch) prep_ap(i + 1);
            lds_barrier();
        }
    } else {
#pragma unroll
        for (int r = 0; r < NRT; ++r) {
            S[r] = zero4();
            if (state_in) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[r][i] = state_in[sbase + static_cast<size_t>(16 * r + 4 * lg + i) * DV + col0 + lr];
            }
        }
        bf16_t vin[4][4];
        if (nch > 0) serial_vload(0, vin);
        for (int i = -1; i < nch; ++i) {
            if (i >= 0) {
                serial_a(i, vin);
                if (i + 1 < nch) serial_vload(i + 1, vin);  // in flight until the next iteration
            }
            lds_barrier();
            if (i >= 0) serial_b(i);
            lds_barrier();
        }
#pragma unroll
        for (int r = 0; r < NRT; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                state_out[sbase + static_cast<size_t>(16 * r + 4 * lg + i) * DV + col0 + lr] = S[r][i];
    }
}

template <int DK, int NSW, bool KDA>
hipError_t launch(int B, int T, int H, int DV, float scale, const bf16_t* q, const bf16_t* k,
                  const bf16_t* v, const float* alpha, const float* beta, const float* s_in,
                  float* s_out, bf16_t* o, hipStream_t s) {
    using L = Layout<DK, NSW, KDA>;
    auto kern = prefill_bf16_kernel<DK, NSW, KDA>;
    if (L::bytes > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::bytes);
        if (e != hipSuccess) return e;
    }
    const int NS = DV / (16 * NSW);
    const int groups = (B * H + 7) / 8;
    const unsigned blocks = static_cast<unsigned>(groups) * 8u * static_cast<unsigned>(NS);
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * (kPrepWaves + NSW)), L::bytes, s, B, T, H, DV,
                       NS, scale, q, k, v, alpha, beta, s_in, s_out, o);
    return hipGetLastError();
}

template <int DK, bool KDA>
hipError_t dispatch_dvs(int dvs, int B, int T, int H, int DV, float scale, const bf16_t* q,
                        const bf16_t* k, const bf16_t* v, const float* alpha, const float* beta,
                        const float* s_in, float* s_out, bf16_t* o, hipStream_t s) {
    switch (dvs) {
        case 16: return launch<DK, 1, KDA>(B, T, H, DV, scale, q, k, v, alpha, beta, s_in, s_out, o, s);
        case 32: return launch<DK, 2, KDA>(B, T, H, DV, scale, q, k, v, alpha, beta, s_in, s_out, o, s);
        default: return launch<DK, 4, KDA>(B, T, H, DV, scale, q, k, v, alpha, beta, s_in, s_out, o, s);
    }
}

template <int DK>
hipError_t dispatch_gate(int kda, int dvs, int B, int T, int H, int DV, float scale,
                         const bf16_t* q, const bf16_t* k, const bf16_t* v, const float* alpha,
                         const float* beta, const float* s_in, float* s_out, bf16_t* o,
                         hipStream_t s) {
    return kda ? dispatch_dvs<DK, true>(dvs, B, T, H, DV, scale, q, k, v, alpha, beta, s_in, s_out, o, s)
               : dispatch_dvs<DK, false>(dvs, B, T, H, DV, scale, q, k, v, alpha, beta, s_in, s_out, o, s);
}

}  // namespace

// Value-column slice width per workgroup: at most 64 columns (four serial
// waves), and heads are split further until the grid covers the 256 CUs
// (exact: columns of S never interact), down to 16 columns.
int prefill_bf16_slice_width(int B, int H, int dv) {
    int ns = dv > 64 ? dv / 64 : 1;
    while (static_cast<long long>(B) * H * ns < 256 && dv / ns > 16) ns *= 2;
    return dv / ns;
}

hipError_t launch_prefill_bf16(int kda, int B, int T, int H, int dk, int dv, float scale,
                               const bf16_t* q, const bf16_t* k, const bf16_t* v,
                               const float* alpha, const float* beta, const float* state_in,
                               float* state_out, bf16_t* o, hipStream_t s) {
    const int dvs = prefill_bf16_slice_width(B, H, dv);
    switch (dk) {
        case 16: return dispatch_gate<16>(kda, dvs, B, T, H, dv, scale, q, k, v, alpha, beta, state_in, state_out, o, s);
        case 32: return dispatch_gate<32>(kda, dvs, B, T, H, dv, scale, q, k, v, alpha, beta, state_in, state_out, o, s);
        case 64: return dispatch_gate<64>(kda, dvs, B, T, H, dv, scale, q, k, v, alpha, beta, state_in, state_out, o, s);
        default: return dispatch_gate<128>(kda, dvs, B, T, H, dv, scale, q, k, v, alpha, beta, state_in, state_out, o, s);
    }
}

}  // namespace gdr
