// Chunked prefill with bf16 inputs: every contraction on bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation), the state in fp32.
//
// Method ("Super Apriel: One Checkpoint, Many Speeds", §2.A: GDN and KDA are
// recurrent mixers with a fixed-size state, scalar resp. channel-wise gate).
// For a chunk of n <= 64 tokens entering with state S, G_t is the cumulative
// log-gate from the chunk start (per key channel for KDA), beta_t the write
// strength, and the recurrence S_t = (I - beta_t k_t k_t^T) D_t S_{t-1} +
// beta_t k_t v_t^T unrolls to
//     A_tj = beta_t sum_c k_tc k_jc exp(G_tc - G_jc)     j <  t   (else 0)
//     P_tj =        sum_c q_tc k_jc exp(G_tc - G_jc)     j <= t   (else 0)
//     T    = (I + A)^{-1}                                (UT transform)
//     X    = diag(beta) (V - Khat S),  Khat_t = k_t exp(G_t)
//     U    = T X
//     O    = scale (Qhat S + P U),     Qhat_t = q_t exp(G_t)
//     S   <- diag(exp(G_end)) S + Ktil^T U,  Ktil_t = k_t exp(G_end - G_t)
// (the WY form with W = T diag(beta) Khat is never materialised: U = T X
// folds W S into Khat S).
//
// Gates inside the contractions.  GDN: the decay is one scalar per token, so
// the MFMAs run on raw q, k and exp(G_t - G_j) (always <= 1) scales their
// outputs.  KDA: the decay differs per channel and must be folded into the
// operands; with a per-channel reference R = G_end / 2 the factors
// exp(G_t - R) and exp(R - G_j) both stay within exp(|G_end| / 2), and S is
// scaled by exp(R) when it is rounded to bf16 for the products.  log(alpha)
// is floored at -80 (exp(-80) ~ 2e-35), so alpha == 0 is legal; KDA needs
// the total log-decay of a channel within one chunk above about -170.
//
// UT transform in fp32.  The four 16x16 diagonal blocks of I + A are inverted
// by forward substitution (one lane per column), then the off-diagonal blocks
// follow from two doubling levels,
//     T_10 = -T_11 A_10 T_00,  T_32 = -T_33 A_32 T_22,
//     T_[23][01] = -T_[23][23] A_[23][01] T_[01][01],
// on fp32 matrix cores (v_mfma_f32_16x16x4_f32).  T is rounded to bf16 once.
//
// Mapping.  One workgroup of four wavefronts per (b, h, slice of DVS value
// columns); the value columns of S are independent, so slices of one head
// run on different CUs (sharing q/k/gates through L2: the slices of a head
// are placed on one XCD).  The fp32 state slice lives in MFMA accumulators
// for the whole sequence; only a bf16 copy goes through LDS per chunk.
#include "gdr_internal.h"

namespace gdr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;             // chunk
constexpr float kLogFloor = -80.0f;
constexpr int kThreads = 256;

__device__ __forceinline__ bf16x8 ld_op(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// acc(16x16) += A[0:16, k0:k0+32*steps] * Bt[0:16, k0:...]^T, both K-contiguous.
// Lane l holds row (l & 15) of A / of Bt and k-octet (l >> 4); the output
// element acc[i] is C[4 * (l >> 4) + i][l & 15].
template <int STEPS>
__device__ __forceinline__ void mma_nt(f32x4& acc, const bf16_t* A, int pa, const bf16_t* Bt,
                                       int pb, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
        acc = mfma_bf16(ld_op(A + r * pa + s * 32 + g * 8), ld_op(Bt + r * pb + s * 32 + g * 8), acc);
}
__device__ __forceinline__ void mma_nt_dyn(f32x4& acc, const bf16_t* A, int pa, const bf16_t* Bt,
                                           int pb, int lane, int steps) {
    const int r = lane & 15, g = lane >> 4;
    for (int s = 0; s < steps; ++s)
        acc = mfma_bf16(ld_op(A + r * pa + s * 32 + g * 8), ld_op(Bt + r * pb + s * 32 + g * 8), acc);
}

// fp32 16x16 block product X * Y (row-major in LDS with pitches px, py),
// accumulated into `acc` in the accumulator layout described above.
__device__ __forceinline__ f32x4 mm16_f32(const float* X, int px, const float* Y, int py,
                                          int lane, f32x4 acc) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[r * px + 4 * s + g], Y[(4 * s + g) * py + r],
                                                   acc, 0, 0, 0);
    return acc;
}

template <int DK, int DVS, bool KDA>
struct Layout {
    static constexpr int DKP = DK < 32 ? 32 : DK;  // contraction pad for dk = 16
    static constexpr int PK = DKP + 8;             // pitch of [token][channel] tiles (bf16)
    static constexpr int PT = kC + 8;              // pitch of [*][token] tiles (bf16)
    static constexpr int PF = kC + 4;              // pitch of fp32 64x64 tiles
    static constexpr int PY = 16 + 4;              // pitch of fp32 16x16 scratch
    static constexpr int NPAIR = DK / 2;           // channel pairs
    static constexpr int TPP = kThreads / NPAIR;   // threads per channel pair
    static constexpr int TPT = kC / TPP;           // tokens per thread
    // byte offsets
    static constexpr int oKh = 0;
    static constexpr int oQh = oKh + kC * PK * 2;
    static constexpr int oKc = oQh + kC * PK * 2;
    static constexpr int oKtT = oKc + (KDA ? kC * PK * 2 : 0);
    static constexpr int oTb = oKtT + DK * PT * 2;
    static constexpr int oPb = oTb + kC * PT * 2;
    static constexpr int oR0 = oPb + kC * PT * 2;
    // region R0: serial-phase tiles, aliased with the fp32 solve scratch
    static constexpr int oSt = oR0;
    static constexpr int oXt = oSt + DVS * PK * 2;
    static constexpr int oUt = oXt + DVS * PT * 2;
    static constexpr int oU2t = oUt + DVS * PT * 2;
    static constexpr int endSerial = oU2t + (KDA ? 0 : DVS * PT * 2);
    static constexpr int oAf = oR0;
    static constexpr int oTf = oAf + kC * PF * 4;
    static constexpr int oYf = oTf + kC * PF * 4;
    static constexpr int endSolve = oYf + 4 * 16 * PY * 4;
    static constexpr int oBeta = endSerial > endSolve ? endSerial : endSolve;  // beta_t
    static constexpr int oGl = oBeta + kC * 4;         // GDN: G_t
    static constexpr int oGend = oGl + kC * 4;         // exp(G_end) per channel
    static constexpr int oGref = oGend + DK * 4;       // KDA: exp(R) per channel
    static constexpr int oPart = oGref + DK * 4;       // cumsum partials [TPP][DK]
    static constexpr int bytes = oPart + TPP * DK * 4;
    static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
    static_assert(TPT >= 2 && TPT % 2 == 0, "token split");
};

template <int DK, int DVS, bool KDA>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(
    int B, int T, int H, int DV, int NS, float scale, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, const float* __restrict__ state_in,
    float* __restrict__ state_out, bf16_t* __restrict__ o) {
    using L = Layout<DK, DVS, KDA>;
    constexpr int NCT = DVS / 16;            // value-column tiles
    constexpr int NRT = DK / 16;             // key-row tiles of S
    constexpr int NST = NRT * NCT;           // S tiles
    constexpr int MST = (NST + 3) / 4;       // S tiles per wave (max)
    constexpr int KSTEPS = L::DKP / 32;      // contraction steps over dk

    extern __shared__ __align__(16) unsigned char smem[];
    bf16_t* Kh = reinterpret_cast<bf16_t*>(smem + L::oKh);
    bf16_t* Qh = reinterpret_cast<bf16_t*>(smem + L::oQh);
    bf16_t* Kc = KDA ? reinterpret_cast<bf16_t*>(smem + L::oKc) : Kh;
    bf16_t* KtT = reinterpret_cast<bf16_t*>(smem + L::oKtT);
    bf16_t* Tb = reinterpret_cast<bf16_t*>(smem + L::oTb);
    bf16_t* Pb = reinterpret_cast<bf16_t*>(smem + L::oPb);
    bf16_t* St = reinterpret_cast<bf16_t*>(smem + L::oSt);
    bf16_t* Xt = reinterpret_cast<bf16_t*>(smem + L::oXt);
    bf16_t* Ut = reinterpret_cast<bf16_t*>(smem + L::oUt);
    bf16_t* U2t = KDA ? Ut : reinterpret_cast<bf16_t*>(smem + L::oU2t);
    float* Af = reinterpret_cast<float*>(smem + L::oAf);
    float* Tf = reinterpret_cast<float*>(smem + L::oTf);
    float* Yf = reinterpret_cast<float*>(smem + L::oYf);
    float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);
    float* sGl = reinterpret_cast<float*>(smem + L::oGl);
    float* sGend = reinterpret_cast<float*>(smem + L::oGend);
    float* sGref = reinterpret_cast<float*>(smem + L::oGref);
    float* sPart = reinterpret_cast<float*>(smem + L::oPart);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // Block -> (head, slice): the NS slices of a head get block ids that are
    // congruent mod 8, i.e. land on one XCD and share its L2.
    const int BH = B * H;
    const int grp = blockIdx.x / (8 * NS);
    const int rem = blockIdx.x - grp * 8 * NS;
    const int bh = grp * 8 + (rem & 7);
    const int slice = rem >> 3;
    if (bh >= BH) return;  // whole block exits before any barrier
    const int b = bh / H, h = bh - b * H;
    const int c0 = slice * DVS;

    // ---- constant zeros: upper tiles of T and P, dk padding -----------------
    for (int idx = tid; idx < kC * kC; idx += kThreads) {
        const int t = idx / kC, j = idx % kC;
        if ((j >> 4) > (t >> 4)) { Tb[t * L::PT + j] = 0; Pb[t * L::PT + j] = 0; }
    }
    if constexpr (L::DKP != DK) {
        for (int idx = tid; idx < kC * (L::DKP - DK); idx += kThreads) {
            const int t = idx / (L::DKP - DK), c = DK + idx % (L::DKP - DK);
            Kh[t * L::PK + c] = 0; Qh[t * L::PK + c] = 0;
            if constexpr (KDA) Kc[t * L::PK + c] = 0;
        }
    }

    // ---- fp32 state slice in accumulators -----------------------------------
    // owned tile index s = wave + 4 m: key-row tile s / NCT, column tile s % NCT.
    f32x4 S[MST];
    const size_t sbase = static_cast<size_t>(bh) * DK * DV;
#pragma unroll
    for (int m = 0; m < MST; ++m) {
        const int s = wave + 4 * m;
        S[m] = zero4();
        if (s < NST && state_in) {
            const int rt = s / NCT, ct = s % NCT;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[m][i] = state_in[sbase + static_cast<size_t>(16 * rt + 4 * lg + i) * DV + c0 +
                                   16 * ct + lr];
        }
    }

    const int pair = tid % L::NPAIR;
    const int tgrp = tid / L::NPAIR;
    const int ch = 2 * pair;
    const int tlo = tgrp * L::TPT;

    for (int t0 = 0; t0 < T; t0 += kC) {
        const int n = min(kC, T - t0);
        __syncthreads();  // previous chunk finished reading every tile

        // ---- gates and gated operands: thread = (channel pair, token run) ---
        float g0[L::TPT], g1[L::TPT];
        {
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int u = 0; u < L::TPT; ++u) {
                const int t = tlo + u;
                float l0 = 0.f, l1 = 0.f;
                if (t < n) {
                    const size_t gi = (static_cast<size_t>(b) * T + t0 + t) * H + h;
                    if constexpr (KDA) {
                        const float2 a2 = *reinterpret_cast<const float2*>(alpha + gi * DK + ch);
                        l0 = fmaxf(__logf(a2.x), kLogFloor);
                        l1 = fmaxf(__logf(a2.y), kLogFloor);
                    } else {
                        l0 = l1 = fmaxf(__logf(alpha[gi]), kLogFloor);
                    }
                }
                acc0 += l0;
                acc1 += l1;
                g0[u] = acc0;
                g1[u] = acc1;
            }
            sPart[tgrp * DK + ch] = acc0;
            sPart[tgrp * DK + ch + 1] = acc1;
        }
        if (pair == 0) {
#pragma unroll
            for (int u = 0; u < L::TPT; ++u) {
                const int t = tlo + u;
                sBeta[t] = t < n ? beta[(static_cast<size_t>(b) * T + t0 + t) * H + h] : 0.f;
            }
        }
        __syncthreads();  // partial sums visible
        {
            float off0 = 0.f, off1 = 0.f, end0 = 0.f, end1 = 0.f;
            for (int gq = 0; gq < L::TPP; ++gq) {
                const float p0 = sPart[gq * DK + ch], p1 = sPart[gq * DK + ch + 1];
                if (gq < tgrp) { off0 += p0; off1 += p1; }
                end0 += p0;
                end1 += p1;
            }
            const float ref0 = KDA ? 0.5f * end0 : 0.f, ref1 = KDA ? 0.5f * end1 : 0.f;
            if (tgrp == 0) {
                sGend[ch] = __expf(end0);
                sGend[ch + 1] = __expf(end1);
                if constexpr (KDA) { sGref[ch] = __expf(ref0); sGref[ch + 1] = __expf(ref1); }
            }
            uint32_t kt0[L::TPT / 2], kt1[L::TPT / 2];
#pragma unroll
            for (int u = 0; u < L::TPT; ++u) {
                const int t = tlo + u;
                const float G0 = off0 + g0[u], G1 = off1 + g1[u];
                float k0 = 0.f, k1 = 0.f, q0 = 0.f, q1 = 0.f;
                if (t < n) {
                    const size_t ri = ((static_cast<size_t>(b) * T + t0 + t) * H + h) * DK + ch;
                    const uint32_t kw = *reinterpret_cast<const uint32_t*>(k + ri);
                    const uint32_t qw = *reinterpret_cast<const uint32_t*>(q + ri);
                    k0 = __uint_as_float(kw << 16);
                    k1 = __uint_as_float(kw & 0xffff0000u);
                    q0 = __uint_as_float(qw << 16);
                    q1 = __uint_as_float(qw & 0xffff0000u);
                }
                if (!KDA && pair == 0) sGl[t] = G0;
                float kt_0, kt_1;
                if constexpr (KDA) {
                    const float up0 = __expf(G0 - ref0), up1 = __expf(G1 - ref1);
                    const float dn0 = __expf(ref0 - G0), dn1 = __expf(ref1 - G1);
                    *reinterpret_cast<uint32_t*>(Kh + t * L::PK + ch) = pack2(k0 * up0, k1 * up1);
                    *reinterpret_cast<uint32_t*>(Qh + t * L::PK + ch) = pack2(q0 * up0, q1 * up1);
                    *reinterpret_cast<uint32_t*>(Kc + t * L::PK + ch) = pack2(k0 * dn0, k1 * dn1);
                    kt_0 = k0 * __expf(end0 - G0);
                    kt_1 = k1 * __expf(end1 - G1);
                } else {
                    *reinterpret_cast<uint32_t*>(Kh + t * L::PK + ch) = pack2(k0, k1);
                    *reinterpret_cast<uint32_t*>(Qh + t * L::PK + ch) = pack2(q0, q1);
                    kt_0 = k0;
                    kt_1 = k1;
                }
                if (u & 1) {
                    kt0[u >> 1] |= static_cast<uint32_t>(f32_to_bf16(kt_0)) << 16;
                    kt1[u >> 1] |= static_cast<uint32_t>(f32_to_bf16(kt_1)) << 16;
                } else {
                    kt0[u >> 1] = f32_to_bf16(kt_0);
                    kt1[u >> 1] = f32_to_bf16(kt_1);
                }
            }
#pragma unroll
            for (int u = 0; u < L::TPT / 2; ++u) {
                *reinterpret_cast<uint32_t*>(KtT + ch * L::PT + tlo + 2 * u) = kt0[u];
                *reinterpret_cast<uint32_t*>(KtT + (ch + 1) * L::PT + tlo + 2 * u) = kt1[u];
            }
        }
        __syncthreads();  // operands ready

        // ---- A and P: 10 lower tiles each, 5 tiles per wave ------------------
        for (int tix = wave; tix < 20; tix += 4) {
            const bool isP = tix >= 10;
            int rem2 = isP ? tix - 10 : tix, rt = 0;
            while (rem2 > rt) { rem2 -= rt + 1; ++rt; }
            const int ct = rem2;
            f32x4 acc = zero4();
            mma_nt<KSTEPS>(acc, (isP ? Qh : Kh) + 16 * rt * L::PK, L::PK, Kc + 16 * ct * L::PK,
                           L::PK, lane);
            const int j = 16 * ct + lr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * rt + 4 * lg + i;
                float x = acc[i];
                if constexpr (!KDA) x *= __expf(sGl[t] - sGl[j]);
                if (isP) {
                    Pb[t * L::PT + j] = f32_to_bf16(j <= t ? x : 0.f);
                } else {
                    Af[t * L::PF + j] = j < t ? sBeta[t] * x : 0.f;
                }
            }
        }
        __syncthreads();  // A in LDS

        // ---- UT transform, level 0: diagonal blocks, one lane per column -----
        if (lane < 16) {
            const int base = 16 * wave;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = (i == lane) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) acc -= Af[(base + i) * L::PF + base + j] * x[j];
                x[i] = acc;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                Tf[(base + i) * L::PF + base + lane] = x[i];
                Tb[(base + i) * L::PT + base + lane] = f32_to_bf16(x[i]);
            }
        }
        __syncthreads();
        // level 1a: Y0 = A_10 T_00 (wave 0), Y1 = A_32 T_22 (wave 1)
        if (wave < 2) {
            const int d = 32 * wave;
            const f32x4 y = mm16_f32(Af + (d + 16) * L::PF + d, L::PF, Tf + d * L::PF + d, L::PF,
                                     lane, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) Yf[(16 * wave + 4 * lg + i) * L::PY + lr] = y[i];
        }
        __syncthreads();
        // level 1b: T_10 = -T_11 Y0, T_32 = -T_33 Y1
        if (wave < 2) {
            const int d = 32 * wave;
            const f32x4 y = mm16_f32(Tf + (d + 16) * L::PF + d + 16, L::PF, Yf + 16 * wave * L::PY,
                                     L::PY, lane, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = d + 16 + 4 * lg + i, j = d + lr;
                Tf[t * L::PF + j] = -y[i];
                Tb[t * L::PT + j] = f32_to_bf16(-y[i]);
            }
        }
        __syncthreads();
        // level 2a: Z_rc = sum_{kb=c..1} A_[2+r][kb] T_[kb][c]   (wave = 2 r + c)
        {
            const int r = wave >> 1, c = wave & 1;
            f32x4 z = zero4();
            for (int kb = c; kb < 2; ++kb)
                z = mm16_f32(Af + (32 + 16 * r) * L::PF + 16 * kb, L::PF,
                             Tf + 16 * kb * L::PF + 16 * c, L::PF, lane, z);
#pragma unroll
            for (int i = 0; i < 4; ++i) Yf[(16 * wave + 4 * lg + i) * L::PY + lr] = z[i];
        }
        __syncthreads();
        // level 2b: T_[2+r][c] = -sum_{kb=0..r} T_[2+r][2+kb] Z_[kb][c]
        {
            const int r = wave >> 1, c = wave & 1;
            f32x4 y = zero4();
            for (int kb = 0; kb <= r; ++kb)
                y = mm16_f32(Tf + (32 + 16 * r) * L::PF + 32 + 16 * kb, L::PF,
                             Yf + 16 * (2 * kb + c) * L::PY, L::PY, lane, y);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Tb[(32 + 16 * r + 4 * lg + i) * L::PT + 16 * c + lr] = f32_to_bf16(-y[i]);
        }
        __syncthreads();  // T complete; solve scratch is dead from here

        // ---- S (fp32 accumulators) -> bf16 S^T in LDS -------------------------
#pragma unroll
        for (int m = 0; m < MST; ++m) {
            const int s = wave + 4 * m;
            if (s < NST) {
                const int rt = s / NCT, ct = s % NCT;
                float x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[i] = S[m][i];
                    if constexpr (KDA) x[i] *= sGref[16 * rt + 4 * lg + i];
                }
                uint2 w;
                w.x = pack2(x[0], x[1]);
                w.y = pack2(x[2], x[3]);
                *reinterpret_cast<uint2*>(St + (16 * ct + lr) * L::PK + 16 * rt + 4 * lg) = w;
            }
        }
        if constexpr (L::DKP != DK) {
            for (int idx = tid; idx < DVS * (L::DKP - DK); idx += kThreads)
                St[(idx / (L::DKP - DK)) * L::PK + DK + idx % (L::DKP - DK)] = 0;
        }
        __syncthreads();

        // ---- Khat S -> X = diag(beta)(V - Khat S); Qhat S kept in registers --
        f32x4 Oacc[NCT];
        {
            const int t_base = 16 * wave + 4 * lg;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 ak = zero4(), aq = zero4();
                mma_nt<KSTEPS>(ak, Kh + 16 * wave * L::PK, L::PK, St + 16 * ct * L::PK, L::PK, lane);
                mma_nt<KSTEPS>(aq, Qh + 16 * wave * L::PK, L::PK, St + 16 * ct * L::PK, L::PK, lane);
                float x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = t_base + i;
                    float kS = ak[i], qS = aq[i];
                    if constexpr (!KDA) {
                        const float e = __expf(sGl[t]);
                        kS *= e;
                        qS *= e;
                    }
                    aq[i] = qS;
                    float vv = 0.f;
                    if (t < n)
                        vv = bf16_to_f32(v[((static_cast<size_t>(b) * T + t0 + t) * H + h) * DV + c0 +
                                           16 * ct + lr]);
                    x[i] = sBeta[t] * (vv - kS);
                }
                Oacc[ct] = aq;
                uint2 w;
                w.x = pack2(x[0], x[1]);
                w.y = pack2(x[2], x[3]);
                *reinterpret_cast<uint2*>(Xt + (16 * ct + lr) * L::PT + t_base) = w;
            }
        }
        __syncthreads();

        // ---- U = T X ------------------------------------------------------------
        const int tsteps = wave < 2 ? 1 : 2;  // T is lower triangular
        {
            const int t_base = 16 * wave + 4 * lg;
            const float gl_end = KDA ? 0.f : sGl[kC - 1];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 u = zero4();
                mma_nt_dyn(u, Tb + 16 * wave * L::PT, L::PT, Xt + 16 * ct * L::PT, L::PT, lane, tsteps);
                uint2 w;
                w.x = pack2(u[0], u[1]);
                w.y = pack2(u[2], u[3]);
                *reinterpret_cast<uint2*>(Ut + (16 * ct + lr) * L::PT + t_base) = w;
                if constexpr (!KDA) {
                    float y[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[i] = u[i] * __expf(gl_end - sGl[t_base + i]);
                    w.x = pack2(y[0], y[1]);
                    w.y = pack2(y[2], y[3]);
                    *reinterpret_cast<uint2*>(U2t + (16 * ct + lr) * L::PT + t_base) = w;
                }
            }
        }
        __syncthreads();

        // ---- O = scale (Qhat S + P U) -------------------------------------------
        {
            const int t_base = 16 * wave + 4 * lg;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                mma_nt_dyn(Oacc[ct], Pb + 16 * wave * L::PT, L::PT, Ut + 16 * ct * L::PT, L::PT, lane,
                           tsteps);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = t_base + i;
                    if (t < n)
                        o[((static_cast<size_t>(b) * T + t0 + t) * H + h) * DV + c0 + 16 * ct + lr] =
                            f32_to_bf16(scale * Oacc[ct][i]);
                }
            }
        }
        // ---- S <- diag(exp(G_end)) S + Ktil^T U ----------------------------------
#pragma unroll
        for (int m = 0; m < MST; ++m) {
            const int s = wave + 4 * m;
            if (s < NST) {
                const int rt = s / NCT, ct = s % NCT;
#pragma unroll
                for (int i = 0; i < 4; ++i) S[m][i] *= sGend[KDA ? 16 * rt + 4 * lg + i : 0];
                mma_nt<2>(S[m], KtT + 16 * rt * L::PT, L::PT, U2t + 16 * ct * L::PT, L::PT, lane);
            }
        }
    }

#pragma unroll
    for (int m = 0; m < MST; ++m) {
        const int s = wave + 4 * m;
        if (s < NST) {
            const int rt = s / NCT, ct = s % NCT;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                state_out[sbase + static_cast<size_t>(16 * rt + 4 * lg + i) * DV + c0 + 16 * ct + lr] =
                    S[m][i];
        }
    }
}

template <int DK, int DVS, bool KDA>
hipError_t launch(int B, int T, int H, int DV, float scale, const bf16_t* q, const bf16_t* k,
                  const bf16_t* v, const float* alpha, const float* beta, const float* s_in,
                  float* s_out, bf16_t* o, hipStream_t s) {
    using L = Layout<DK, DVS, KDA>;
    auto kern = prefill_bf16_kernel<DK, DVS, KDA>;
    if (L::bytes > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::bytes);
        if (e != hipSuccess) return e;
    }
    const int NS = DV / DVS;
    const int groups = (B * H + 7) / 8;
    const unsigned blocks = static_cast<unsigned>(groups) * 8u * static_cast<unsigned>(NS);
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), L::bytes, s, B, T, H, DV, NS, scale, q,
                       k, v, alpha, beta, s_in, s_out, o);
    return hipGetLastError();
}

template <int DK, bool KDA>
hipError_t dispatch_dvs(int dvs, int B, int T, int H, int DV, float scale, const bf16_t* q,
                        const bf16_t* k, const bf16_t* v, const float* alpha, const float* beta,
                        const float* s_in, float* s_out, bf16_t* o, hipStream_t s) {
    switch (dvs) {
        case 16: return launch<DK, 16, KDA>(B, T, H, DV, scale, q, k, v, alpha, beta, s_in, s_out, o, s);
        case 32: return launch<DK, 32, KDA>(B, T, H, DV, scale, q, k, v, alpha, beta, s_in, s_out, o, s);
        default: return launch<DK, 64, KDA>(B, T, H, DV, scale, q, k, v, alpha, beta, s_in, s_out, o, s);
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

// Value-column slice width: at most 64 columns (LDS budget), and heads are
// split further until the grid covers the 256 CUs (the slices are exact:
// columns of S never interact), down to 16 columns.
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
