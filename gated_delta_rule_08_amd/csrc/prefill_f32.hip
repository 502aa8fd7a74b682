// Chunked prefill in fp32 (dtype GDR_DTYPE_F32): every product in fp32 on
// the vector ALUs, staged through LDS.  This is the exact-precision path; the
// bf16 matrix-core path lives in prefill_bf16.hip.
//
// Chunked form of the gated delta rule ("Super Apriel: One Checkpoint, Many
// Speeds", §2.A: GDN / KDA recurrent mixers, scalar / channel-wise gate).
// For a chunk of n <= 64 tokens entering with state S, with G_t the
// cumulative log-gate inside the chunk (per channel for KDA),
//     A_tj = beta_t sum_c k_tc k_jc exp(G_tc - G_jc)   (j < t)
//     P_tj = sum_c q_tc k_jc exp(G_tc - G_jc)          (j <= t)
//     X    = diag(beta) (V - Khat S),  Khat_t = k_t * exp(G_t)
//     U    = (I + A)^{-1} X             (forward substitution)
//     O    = scale (Qhat S + P U),      Qhat_t = q_t * exp(G_t)
//     S   <- diag(exp(G_end)) S + Ktil^T U,  Ktil_t = k_t * exp(G_end - G_t)
// Every exponent is a difference G_a - G_b with a >= b, so no factor exceeds 1.
// log(alpha) is floored at -40 (exp(-40) ~ 4e-18), which makes alpha == 0 legal.
// Input prologue (GDR_PRO_*): beta and the log-gates are formed from logits
// as they are loaded, and the staged q, k rows are scaled by their inverse
// norms before any product.
//
// Mapping: one workgroup (256 threads) per (b, h, slice of up to 32 value
// columns); the state slice stays in LDS for the whole sequence.
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kChunk = 64;
constexpr float kLogFloor = -40.0f;

template <int DK, int DVS, bool KDA>
struct F32Smem {
    static constexpr int kG = KDA ? kChunk * DK : kChunk;
    static constexpr int kQ = 0;
    static constexpr int kK = kQ + kChunk * DK;
    static constexpr int kGo = kK + kChunk * DK;
    static constexpr int kB = kGo + kG;
    static constexpr int kA = kB + kChunk;
    static constexpr int kP = kA + kChunk * kChunk;
    static constexpr int kS = kP + kChunk * kChunk;
    static constexpr int kX = kS + DK * DVS;
    static constexpr int kN = kX + kChunk * DVS;  // prologue: 1/||q_t||, 1/||k_t||
    static constexpr int kTotal = kN + 2 * kChunk;
    static constexpr size_t bytes = sizeof(float) * kTotal;
};

template <int DK, int DVS, bool KDA>
__global__ __launch_bounds__(256) void prefill_f32_kernel(
    int Tmax, int H, int DV, float scale, const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* __restrict__ state_in, float* __restrict__ state_out, float* __restrict__ o,
    Opts vl) {
    using L = F32Smem<DK, DVS, KDA>;
    extern __shared__ float smem[];
    float* Qs = smem + L::kQ;
    float* Ks = smem + L::kK;
    float* Gs = smem + L::kGo;
    float* Bs = smem + L::kB;
    float* As = smem + L::kA;
    float* Ps = smem + L::kP;
    float* Ss = smem + L::kS;
    float* Xs = smem + L::kX;
    float* Ns = smem + L::kN;
    const bool sig = (vl.pro & GDR_PRO_SIGMOID) != 0;
    // natural log of a gate (of sigmoid(logit) with the prologue)
    auto log_gate = [&](float a) { return sig ? 0.6931471805599453f * log2_sigmoid(a) : __logf(a); };

    const int nslice = DV / DVS;
    const int slice = blockIdx.x % nslice;
    const int bh = blockIdx.x / nslice;
    const int h = bh % H;
    const int b = bh / H;
    const int c0 = slice * DVS;
    const int tid = threadIdx.x;
    // This sequence (packed variable-length input: its own length, first
    // token row and state row; skipped, before any barrier, if out of range).
    int T = Tmax;
    size_t tb = static_cast<size_t>(b) * Tmax;  // row of the sequence's first token (before x H)
    int srow = bh;
    bool init = state_in != nullptr;
    if (vl.cu) {
        const int s0 = vl.cu[b], s1 = vl.cu[b + 1];
        if (s0 < 0 || s1 < s0 || s1 - s0 > Tmax || s1 > vl.total) return;
        T = s1 - s0;
        tb = static_cast<size_t>(s0);
        if (T == 0) return;  // an empty sequence leaves its state row untouched
    }
    if (vl.slot) {
        const int r = vl.slot[b];
        if (r < 0 || r >= vl.n_slots) return;
        srow = r * H + h;
    }
    if (vl.has && vl.has[b] == 0) init = false;
    const size_t sbase = static_cast<size_t>(srow) * DK * DV;

    for (int idx = tid; idx < DK * DVS; idx += 256) {
        const int i = idx / DVS, j = idx % DVS;
        Ss[idx] = init ? state_in[sbase + static_cast<size_t>(i) * DV + c0 + j] : 0.0f;
    }

    for (int t0 = 0; t0 < T; t0 += kChunk) {
        const int n = min(kChunk, T - t0);
        __syncthreads();  // previous chunk done with every buffer
        for (int idx = tid; idx < kChunk * DK; idx += 256) {
            const int t = idx / DK, c = idx % DK;
            const size_t g = ((tb + t0 + t) * H + h) * DK + c;
            Qs[idx] = t < n ? q[g] : 0.0f;
            Ks[idx] = t < n ? k[g] : 0.0f;
        }
        for (int idx = tid; idx < kChunk * DVS; idx += 256) {
            const int t = idx / DVS, j = idx % DVS;
            Xs[idx] = t < n ? v[((tb + t0 + t) * H + h) * DV + c0 + j] : 0.0f;
        }
        if (tid < kChunk) {
            const size_t g = (tb + t0 + tid) * H + h;
            Bs[tid] = tid < n ? (sig ? sigmoid_f(beta[g]) : beta[g]) : 0.0f;
            if constexpr (!KDA) Gs[tid] = tid < n ? fmaxf(log_gate(alpha[g]), kLogFloor) : 0.0f;
        }
        __syncthreads();
        if (vl.pro & GDR_PRO_L2NORM_QK) {
            // inverse norms of the 64 q rows and 64 k rows (each thread walks
            // its row from its own start, so the 64 rows hit distinct banks)
            if (tid < 2 * kChunk) {
                const float* row = (tid < kChunk ? Qs : Ks) + (tid % kChunk) * DK;
                float ss = 0.0f;
                for (int c = 0; c < DK; ++c) {
                    const float x = row[(c + tid) % DK];
                    ss += x * x;
                }
                Ns[tid] = inv_norm(ss);
            }
            __syncthreads();
            for (int idx = tid; idx < kChunk * DK; idx += 256) {
                Qs[idx] *= Ns[idx / DK];
                Ks[idx] *= Ns[kChunk + idx / DK];
            }
        }
        // Cumulative log-gate inside the chunk.
        if constexpr (KDA) {
            if (tid < DK) {
                float acc = 0.0f;
                for (int t = 0; t < kChunk; ++t) {
                    float g = 0.0f;
                    if (t < n)
                        g = fmaxf(log_gate(alpha[((tb + t0 + t) * H + h) * DK + tid]),
                                  kLogFloor);
                    acc += g;
                    Gs[t * DK + tid] = acc;
                }
            }
        } else {
            if (tid == 0) {
                float acc = 0.0f;
                for (int t = 0; t < kChunk; ++t) { acc += Gs[t]; Gs[t] = acc; }
            }
        }
        __syncthreads();
        // A (strictly lower, scaled by beta_t) and P (lower, diagonal included).
        for (int idx = tid; idx < kChunk * kChunk; idx += 256) {
            const int t = idx / kChunk, j = idx % kChunk;
            float sa = 0.0f, sp = 0.0f;
            if (j <= t) {
                if constexpr (KDA) {
                    for (int c = 0; c < DK; ++c) {
                        const float d = __expf(Gs[t * DK + c] - Gs[j * DK + c]);
                        const float kj = Ks[j * DK + c] * d;
                        sa += Ks[t * DK + c] * kj;
                        sp += Qs[t * DK + c] * kj;
                    }
                } else {
                    for (int c = 0; c < DK; ++c) {
                        sa += Ks[t * DK + c] * Ks[j * DK + c];
                        sp += Qs[t * DK + c] * Ks[j * DK + c];
                    }
                    const float d = __expf(Gs[t] - Gs[j]);
                    sa *= d;
                    sp *= d;
                }
            }
            As[idx] = j < t ? Bs[t] * sa : 0.0f;
            Ps[idx] = sp;
        }
        // X = diag(beta) (V - Khat S).
        for (int idx = tid; idx < kChunk * DVS; idx += 256) {
            const int t = idx / DVS, j = idx % DVS;
            float acc = 0.0f;
            for (int c = 0; c < DK; ++c) {
                const float g = KDA ? Gs[t * DK + c] : Gs[t];
                acc += Ks[t * DK + c] * __expf(g) * Ss[c * DVS + j];
            }
            Xs[idx] = Bs[t] * (Xs[idx] - acc);
        }
        __syncthreads();
        // U = (I + A)^{-1} X by forward substitution, one thread per column.
        if (tid < DVS) {
            for (int i = 1; i < n; ++i) {
                float acc = Xs[i * DVS + tid];
                for (int j = 0; j < i; ++j) acc -= As[i * kChunk + j] * Xs[j * DVS + tid];
                Xs[i * DVS + tid] = acc;
            }
        }
        __syncthreads();
        // O = scale (Qhat S + P U).
        for (int idx = tid; idx < n * DVS; idx += 256) {
            const int t = idx / DVS, j = idx % DVS;
            float acc = 0.0f;
            for (int c = 0; c < DK; ++c) {
                const float g = KDA ? Gs[t * DK + c] : Gs[t];
                acc += Qs[t * DK + c] * __expf(g) * Ss[c * DVS + j];
            }
            for (int jj = 0; jj <= t; ++jj) acc += Ps[t * kChunk + jj] * Xs[jj * DVS + j];
            o[((tb + t0 + t) * H + h) * DV + c0 + j] = scale * acc;
        }
        __syncthreads();
        // S <- diag(exp(G_end)) S + Ktil^T U.
        for (int idx = tid; idx < DK * DVS; idx += 256) {
            const int c = idx / DVS, j = idx % DVS;
            const float ge = KDA ? Gs[(n - 1) * DK + c] : Gs[n - 1];
            float acc = __expf(ge) * Ss[idx];
            for (int t = 0; t < n; ++t) {
                const float g = KDA ? Gs[t * DK + c] : Gs[t];
                acc += Ks[t * DK + c] * __expf(ge - g) * Xs[t * DVS + j];
            }
            Ss[idx] = acc;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < DK * DVS; idx += 256) {
        const int i = idx / DVS, j = idx % DVS;
        state_out[sbase + static_cast<size_t>(i) * DV + c0 + j] = Ss[idx];
    }
}

template <int DK, int DVS, bool KDA>
hipError_t launch(int B, int T, int H, int DV, float scale, const float* q, const float* k,
                  const float* v, const float* alpha, const float* beta, const float* s_in,
                  float* s_out, float* o, hipStream_t s, const Opts& vl) {
    using L = F32Smem<DK, DVS, KDA>;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    auto kern = prefill_f32_kernel<DK, DVS, KDA>;
    if (!grid_fits(static_cast<unsigned long long>(B) * H * (DV / DVS), 256)) return hipErrorInvalidConfiguration;
    if (L::bytes > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(L::bytes));
        if (e != hipSuccess) return e;
    }
    const unsigned blocks = static_cast<unsigned>(B) * H * (DV / DVS);
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), L::bytes, s, T, H, DV, scale, q, k, v,
                       alpha, beta, s_in, s_out, o, vl);
    return hipGetLastError();
}

template <int DK, bool KDA>
hipError_t dispatch_dv(int B, int T, int H, int dv, float scale, const float* q,
                       const float* k, const float* v, const float* alpha, const float* beta,
                       const float* s_in, float* s_out, float* o, hipStream_t s, const Opts& vl) {
    if (dv == 16)
        return launch<DK, 16, KDA>(B, T, H, dv, scale, q, k, v, alpha, beta, s_in, s_out, o, s, vl);
    return launch<DK, 32, KDA>(B, T, H, dv, scale, q, k, v, alpha, beta, s_in, s_out, o, s, vl);
}

template <int DK>
hipError_t dispatch_gate(int kda, int B, int T, int H, int dv, float scale, const float* q,
                         const float* k, const float* v, const float* alpha, const float* beta,
                         const float* s_in, float* s_out, float* o, hipStream_t s, const Opts& vl) {
    return kda ? dispatch_dv<DK, true>(B, T, H, dv, scale, q, k, v, alpha, beta, s_in, s_out, o, s, vl)
               : dispatch_dv<DK, false>(B, T, H, dv, scale, q, k, v, alpha, beta, s_in, s_out, o, s, vl);
}

}  // namespace

hipError_t launch_prefill_f32(int kda, int B, int T, int H, int dk, int dv, float scale,
                              const float* q, const float* k, const float* v,
                              const float* alpha, const float* beta, const float* state_in,
                              float* state_out, float* o, hipStream_t s, const Opts& vl) {
    switch (dk) {
        case 16: return dispatch_gate<16>(kda, B, T, H, dv, scale, q, k, v, alpha, beta, state_in, state_out, o, s, vl);
        case 32: return dispatch_gate<32>(kda, B, T, H, dv, scale, q, k, v, alpha, beta, state_in, state_out, o, s, vl);
        case 64: return dispatch_gate<64>(kda, B, T, H, dv, scale, q, k, v, alpha, beta, state_in, state_out, o, s, vl);
        default: return dispatch_gate<128>(kda, B, T, H, dv, scale, q, k, v, alpha, beta, state_in, state_out, o, s, vl);
    }
}

}  // namespace gdr
