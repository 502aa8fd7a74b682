// Decode step of the gated delta rule: one token per head, state streamed
// through registers once (read 4*dk*dv bytes, write 4*dk*dv bytes).
//
// Per head (b, h), with a = alpha (scalar for GDN, vector over the key axis
// for KDA), the step S_t = (I - beta k k^T) D S + beta k v^T, o = S_t^T q
// ("Super Apriel: One Checkpoint, Many Speeds", §2.A: GDN and KDA are
// recurrent mixers with scalar and channel-wise gates) is evaluated in one
// pass over the state as
//     S' = D S;   p = S'^T k;   r = S'^T q;   e = v - p
//     S  = S' + beta k e^T;     o = scale * (r + beta (k . q) e)
// (o = S^T q expanded, so no second pass over the new state is needed).
//
// Mapping.  The state of one head is dk rows of dv fp32.  Each wavefront owns
// a slice of up to 32 value columns over all dk rows: a lane holds one float4
// (4 columns) of every (64/LPR)-th row, LPR = columns/4 lanes covering a row
// segment, so one wavefront load instruction fetches 64/LPR full 128-byte
// row segments.  The dk-reductions of p, r and k.q are in-lane sums over the
// lane's rows followed by a butterfly over the lanes that share columns.  No
// LDS, no barriers: waves are independent.  With dv = 128 the four waves of a
// workgroup cover the four column slices of one head, so a workgroup streams
// one contiguous 64 KiB state.
//
// Input prologue (GDR_PRO_*): sigmoid of the gate logits on load; raw q and
// k enter the dk-sums unchanged, their squared norms take one more butterfly,
// and the sums are rescaled by 1/||k||, 1/||q|| afterwards (no extra pass
// over the state).
#include "gdr_internal.h"

namespace gdr {
namespace {

// The state is touched exactly once per step: nontemporal loads and stores
// (the `nt` bit on global_load/store_dwordx4) keep it from displacing other
// data in the caches; measured ~14% higher bandwidth than plain accesses for
// this read-modify-write stream.
__device__ __forceinline__ float4 ld_state(const float* p) {
    return make_float4(__builtin_nontemporal_load(p), __builtin_nontemporal_load(p + 1),
                       __builtin_nontemporal_load(p + 2), __builtin_nontemporal_load(p + 3));
}
__device__ __forceinline__ void st_state(float* p, const float4& x) {
    __builtin_nontemporal_store(x.x, p);
    __builtin_nontemporal_store(x.y, p + 1);
    __builtin_nontemporal_store(x.z, p + 2);
    __builtin_nontemporal_store(x.w, p + 3);
}

template <typename InT> struct Vec4Out;
template <> struct Vec4Out<float> {
    __device__ __forceinline__ static void store(float* p, float a, float b, float c, float d) {
        *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
    }
};
template <> struct Vec4Out<bf16_t> {
    __device__ __forceinline__ static void store(bf16_t* p, float a, float b, float c, float d) {
        uint2 w;
        w.x = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
        w.y = static_cast<uint32_t>(f32_to_bf16(c)) | (static_cast<uint32_t>(f32_to_bf16(d)) << 16);
        *reinterpret_cast<uint2*>(p) = w;
    }
};

template <typename InT>
__device__ __forceinline__ float4 load4(const InT* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 load4<bf16_t>(const bf16_t* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

template <int DK, int DV, typename InT, bool KDA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void decode_step_kernel(
    int n_units, float scale, const InT* __restrict__ q, const InT* __restrict__ k,
    const InT* __restrict__ v, const float* __restrict__ alpha, const float* __restrict__ beta,
    float* __restrict__ state, InT* __restrict__ o, int pro) {
    constexpr int COLS = DV < 32 ? DV : 32;  // value columns per wavefront
    constexpr int NSLICE = DV / COLS;
    constexpr int LPR = COLS / 4;            // lanes per row segment
    constexpr int RPI = 64 / LPR;            // rows per load instruction
    constexpr int NI = DK / RPI;             // rows per lane
    static_assert(NI >= 1 && NI * RPI == DK, "head size does not tile the wavefront");

    constexpr int UPW = 4 / NSLICE;          // heads per workgroup
    constexpr int NL = (UPW * DK + 255) / 256;  // shared elements per thread
    static_assert(UPW >= 1 && UPW * NSLICE == 4, "the four waves cover whole heads");
    // q, k and (KDA) the gate of the workgroup's heads, read by every wave
    // of the head from LDS when a row needs them instead of being held in
    // registers: both gates then fit 128 VGPRs, four waves per SIMD (GDN
    // measured 48.8 -> 47.4 us per launch at B=64, H=32, d=128; KDA, whose
    // three reads per row the compiler would otherwise hoist for all 16 rows
    // (129 VGPRs, three waves), takes them 8 rows at a time: 203 -> 195 us
    // at B=256).
    __shared__ float qs[UPW][DK], ks[UPW][DK], gs[KDA ? UPW : 1][KDA ? DK : 1];

    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int unit = wave / NSLICE;
    const int lu = (threadIdx.x >> 6) / NSLICE;  // the wave's head within the workgroup
    const int u0 = blockIdx.x * UPW;
    const bool live = unit < n_units;            // padding waves only join the barrier
    const int slice = wave - unit * NSLICE;
    const int rg = lane / LPR;
    const int col = slice * COLS + (lane % LPR) * 4;

    // Load order: the small vectors first (shared ones cooperatively), then
    // the state rows in row order (each pinned by a scheduling fence).  Loads
    // complete in order, so each row is scaled and reduced as soon as it
    // arrives; left alone, the compiler issued row 0 last and waited for the
    // whole state.
    float tq[NL], tk[NL], tg[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int i = threadIdx.x + 256 * j, uu = i / DK, c = i - uu * DK;
        const bool ok = i < UPW * DK && u0 + uu < n_units;
        const size_t e = static_cast<size_t>(u0 + uu) * DK + c;
        tq[j] = ok ? Elem<InT>::load(q + e) : 0.f;
        tk[j] = ok ? Elem<InT>::load(k + e) : 0.f;
        if constexpr (KDA) tg[j] = ok ? alpha[e] : 0.f;
    }
    float ag = 0.f, b = 0.f;
    float4 vv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) {
        if constexpr (!KDA) ag = alpha[unit];
        b = beta[unit];
        vv = load4<InT>(v + static_cast<size_t>(unit) * DV + col);
    }
    __builtin_amdgcn_sched_barrier(0);

    float* S = state + static_cast<size_t>(live ? unit : 0) * DK * DV + col;
    float4 s[NI];
    if (live) {
#pragma unroll
        for (int m = 0; m < NI; ++m) {
            s[m] = ld_state(S + static_cast<size_t>(m * RPI + rg) * DV);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    const bool sig = pro & GDR_PRO_SIGMOID;  // gates given as logits
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int i = threadIdx.x + 256 * j;
        if (i < UPW * DK) {
            const int uu = i / DK, c = i - uu * DK;
            qs[uu][c] = tq[j];
            ks[uu][c] = tk[j];
            if constexpr (KDA) gs[uu][c] = sig ? sigmoid_f(tg[j]) : tg[j];
        }
    }
    __syncthreads();
    if (!live) return;  // no barriers below
    if (sig) {
        b = sigmoid_f(b);
        if constexpr (!KDA) ag = sigmoid_f(ag);
    }
    const float* qv = qs[lu];
    const float* kv = ks[lu];

    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
    float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
    float kq = 0.f;
#pragma unroll
    for (int m = 0; m < NI; ++m) {
        if (KDA && (m & 7) == 0) __builtin_amdgcn_sched_barrier(0);  // the next 8 rows' reads
        const int row = m * RPI + rg;
        const float a = KDA ? gs[lu][row] : ag, kr = kv[row], qr = qv[row];
        s[m].x *= a; s[m].y *= a; s[m].z *= a; s[m].w *= a;
        p0 += kr * s[m].x; p1 += kr * s[m].y; p2 += kr * s[m].z; p3 += kr * s[m].w;
        r0 += qr * s[m].x; r1 += qr * s[m].y; r2 += qr * s[m].z; r3 += qr * s[m].w;
        kq += kr * qr;
    }
    // Butterfly over the lanes that hold the same columns (lane bits >= log2(LPR)).
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
        p0 += __shfl_xor(p0, off); p1 += __shfl_xor(p1, off);
        p2 += __shfl_xor(p2, off); p3 += __shfl_xor(p3, off);
        r0 += __shfl_xor(r0, off); r1 += __shfl_xor(r1, off);
        r2 += __shfl_xor(r2, off); r3 += __shfl_xor(r3, off);
        kq += __shfl_xor(kq, off);
    }
    // Raw q, k: the sums above used them as given; with ik = 1/||k|| and
    // iq = 1/||q|| the normalised step has p * ik, r * iq, (k.q) ik iq, and
    // the update adds beta (ik k) e^T.
    float ik = 1.f;
    if (pro & GDR_PRO_L2NORM_QK) {
        float kk = 0.f, qq = 0.f;
#pragma unroll
        for (int m = 0; m < NI; ++m) {
            const float kr = kv[m * RPI + rg], qr = qv[m * RPI + rg];
            kk += kr * kr;
            qq += qr * qr;
        }
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
            kk += __shfl_xor(kk, off);
            qq += __shfl_xor(qq, off);
        }
        ik = inv_norm(kk);
        const float iq = inv_norm(qq);
        p0 *= ik; p1 *= ik; p2 *= ik; p3 *= ik;
        r0 *= iq; r1 *= iq; r2 *= iq; r3 *= iq;
        kq *= ik * iq;
    }
    const float e0 = vv.x - p0, e1 = vv.y - p1, e2 = vv.z - p2, e3 = vv.w - p3;
    const float bn = b * ik;
#pragma unroll
    for (int m = 0; m < NI; ++m) {
        const float bk = bn * kv[m * RPI + rg];
        s[m].x += bk * e0; s[m].y += bk * e1; s[m].z += bk * e2; s[m].w += bk * e3;
        st_state(S + static_cast<size_t>(m * RPI + rg) * DV, s[m]);
    }
    if (rg == 0) {
        const float bkq = b * kq;
        Vec4Out<InT>::store(o + static_cast<size_t>(unit) * DV + col,
                            scale * (r0 + bkq * e0), scale * (r1 + bkq * e1),
                            scale * (r2 + bkq * e2), scale * (r3 + bkq * e3));
    }
}

template <int DK, int DV, typename InT, bool KDA>
hipError_t launch(int n_units, float scale, const void* q, const void* k, const void* v,
                  const float* alpha, const float* beta, float* state, void* o, hipStream_t s,
                  int pro) {
    constexpr int COLS = DV < 32 ? DV : 32;
    const long long waves = static_cast<long long>(n_units) * (DV / COLS);
    if (!grid_fits((waves + 3) / 4, 256)) return hipErrorInvalidConfiguration;
    const unsigned blocks = static_cast<unsigned>((waves + 3) / 4);
    hipLaunchKernelGGL((decode_step_kernel<DK, DV, InT, KDA>), dim3(blocks), dim3(256), 0, s,
                       n_units, scale, static_cast<const InT*>(q), static_cast<const InT*>(k),
                       static_cast<const InT*>(v), alpha, beta, state, static_cast<InT*>(o), pro);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t dispatch_type(int kda, int dtype, int n, float scale, const void* q, const void* k,
                         const void* v, const float* alpha, const float* beta, float* state,
                         void* o, hipStream_t s, int pro) {
    if (dtype == GDR_DTYPE_BF16) {
        return kda ? launch<DK, DV, bf16_t, true>(n, scale, q, k, v, alpha, beta, state, o, s, pro)
                   : launch<DK, DV, bf16_t, false>(n, scale, q, k, v, alpha, beta, state, o, s, pro);
    }
    return kda ? launch<DK, DV, float, true>(n, scale, q, k, v, alpha, beta, state, o, s, pro)
               : launch<DK, DV, float, false>(n, scale, q, k, v, alpha, beta, state, o, s, pro);
}

template <int DK>
hipError_t dispatch_dv(int kda, int dtype, int dv, int n, float scale, const void* q,
                       const void* k, const void* v, const float* alpha, const float* beta,
                       float* state, void* o, hipStream_t s, int pro) {
    switch (dv) {
        case 16: return dispatch_type<DK, 16>(kda, dtype, n, scale, q, k, v, alpha, beta, state, o, s, pro);
        case 32: return dispatch_type<DK, 32>(kda, dtype, n, scale, q, k, v, alpha, beta, state, o, s, pro);
        case 64: return dispatch_type<DK, 64>(kda, dtype, n, scale, q, k, v, alpha, beta, state, o, s, pro);
        default: return dispatch_type<DK, 128>(kda, dtype, n, scale, q, k, v, alpha, beta, state, o, s, pro);
    }
}


// T decode steps per head in one launch (the verify step of speculative
// decoding): the state stays in registers across the T tokens, so it is read
// and written once; token t's inputs are loaded while token t-1 is applied.
// Token tensors are [B, T, H, .]; with SAVE the state after each token goes to
// states[b, t, h] (the caller rolls back to an accepted prefix from there).
// The per-token arithmetic is the decode step's, in the same order.
template <int DK, int DV, typename InT, bool KDA, bool SAVE>
__global__ __launch_bounds__(256) void decode_multi_kernel(
    int n_units, int T, int H, float scale, const InT* __restrict__ q, const InT* __restrict__ k,
    const InT* __restrict__ v, const float* __restrict__ alpha, const float* __restrict__ beta,
    float* __restrict__ state, InT* __restrict__ o, float* __restrict__ states, int pro) {
    constexpr int COLS = DV < 32 ? DV : 32;
    constexpr int NSLICE = DV / COLS;
    constexpr int LPR = COLS / 4;
    constexpr int RPI = 64 / LPR;
    constexpr int NI = DK / RPI;
    static_assert(NI >= 1 && NI * RPI == DK, "head size does not tile the wavefront");

    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int unit = wave / NSLICE;
    if (unit >= n_units) return;  // no barriers below: whole waves retire
    const int slice = wave - unit * NSLICE;
    const int rg = lane / LPR;
    const int col = slice * COLS + (lane % LPR) * 4;
    const int b = unit / H, h = unit - (unit / H) * H;

    struct In {
        float qv[NI], kv[NI], av[KDA ? NI : 1], b;
        float4 vv;
    };
    auto load_in = [&](int t, In& x) {
        const size_t tok = (static_cast<size_t>(b) * T + t) * H + h;  // row of token (b, t, h)
        const InT* qu = q + tok * DK;
        const InT* ku = k + tok * DK;
#pragma unroll
        for (int m = 0; m < NI; ++m) {
            x.qv[m] = Elem<InT>::load(qu + m * RPI + rg);
            x.kv[m] = Elem<InT>::load(ku + m * RPI + rg);
        }
        if constexpr (KDA) {
#pragma unroll
            for (int m = 0; m < NI; ++m) x.av[m] = alpha[tok * DK + m * RPI + rg];
        } else {
            x.av[0] = alpha[tok];
        }
        x.b = beta[tok];
        x.vv = load4<InT>(v + tok * DV + col);
    };
    const bool sig = (pro & GDR_PRO_SIGMOID) != 0, nrm = (pro & GDR_PRO_L2NORM_QK) != 0;
    // Load order as in the decode step: the first token's inputs, then the
    // state rows in row order, so the first token's rows are reduced as they
    // arrive.
    In cur, nxt;
    load_in(0, cur);
    __builtin_amdgcn_sched_barrier(0);
    float* S = state + static_cast<size_t>(unit) * DK * DV + col;
    float4 s[NI];
#pragma unroll
    for (int m = 0; m < NI; ++m) {
        s[m] = ld_state(S + static_cast<size_t>(m * RPI + rg) * DV);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int t = 0; t < T; ++t) {
        load_in(t + 1 < T ? t + 1 : t, nxt);  // the next token's inputs (the last one reloads)
        if (sig) {  // gates given as logits
            cur.b = sigmoid_f(cur.b);
#pragma unroll
            for (int m = 0; m < (KDA ? NI : 1); ++m) cur.av[m] = sigmoid_f(cur.av[m]);
        }
        float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
        float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
        float kq = 0.f;
#pragma unroll
        for (int m = 0; m < NI; ++m) {
            const float a = KDA ? cur.av[m] : cur.av[0];
            s[m].x *= a; s[m].y *= a; s[m].z *= a; s[m].w *= a;
            p0 += cur.kv[m] * s[m].x; p1 += cur.kv[m] * s[m].y; p2 += cur.kv[m] * s[m].z; p3 += cur.kv[m] * s[m].w;
            r0 += cur.qv[m] * s[m].x; r1 += cur.qv[m] * s[m].y; r2 += cur.qv[m] * s[m].z; r3 += cur.qv[m] * s[m].w;
            kq += cur.kv[m] * cur.qv[m];
        }
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
            p0 += __shfl_xor(p0, off); p1 += __shfl_xor(p1, off);
            p2 += __shfl_xor(p2, off); p3 += __shfl_xor(p3, off);
            r0 += __shfl_xor(r0, off); r1 += __shfl_xor(r1, off);
            r2 += __shfl_xor(r2, off); r3 += __shfl_xor(r3, off);
            kq += __shfl_xor(kq, off);
        }
        float ik = 1.f;  // raw q, k: rescale the sums as the decode step does
        if (nrm) {
            float kk = 0.f, qq = 0.f;
#pragma unroll
            for (int m = 0; m < NI; ++m) {
                kk += cur.kv[m] * cur.kv[m];
                qq += cur.qv[m] * cur.qv[m];
            }
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) {
                kk += __shfl_xor(kk, off);
                qq += __shfl_xor(qq, off);
            }
            ik = inv_norm(kk);
            const float iq = inv_norm(qq);
            p0 *= ik; p1 *= ik; p2 *= ik; p3 *= ik;
            r0 *= iq; r1 *= iq; r2 *= iq; r3 *= iq;
            kq *= ik * iq;
        }
        const float e0 = cur.vv.x - p0, e1 = cur.vv.y - p1, e2 = cur.vv.z - p2, e3 = cur.vv.w - p3;
        const size_t tok = (static_cast<size_t>(b) * T + t) * H + h;
        const float bn = cur.b * ik;
#pragma unroll
        for (int m = 0; m < NI; ++m) {
            const float bk = bn * cur.kv[m];
            s[m].x += bk * e0; s[m].y += bk * e1; s[m].z += bk * e2; s[m].w += bk * e3;
            if constexpr (SAVE)
                st_state(states + tok * DK * DV + col + static_cast<size_t>(m * RPI + rg) * DV, s[m]);
        }
        if (rg == 0) {
            const float bkq = cur.b * kq;
            Vec4Out<InT>::store(o + tok * DV + col, scale * (r0 + bkq * e0), scale * (r1 + bkq * e1),
                                scale * (r2 + bkq * e2), scale * (r3 + bkq * e3));
        }
        cur = nxt;
    }
#pragma unroll
    for (int m = 0; m < NI; ++m) st_state(S + static_cast<size_t>(m * RPI + rg) * DV, s[m]);
}

template <int DK, int DV, typename InT, bool KDA>
hipError_t launch_multi(int n_units, int T, int H, float scale, const void* q, const void* k,
                        const void* v, const float* alpha, const float* beta, float* state,
                        void* o, float* states, hipStream_t s, int pro) {
    constexpr int COLS = DV < 32 ? DV : 32;
    const long long waves = static_cast<long long>(n_units) * (DV / COLS);
    if (!grid_fits((waves + 3) / 4, 256)) return hipErrorInvalidConfiguration;
    const unsigned blocks = static_cast<unsigned>((waves + 3) / 4);
    if (states) {
        hipLaunchKernelGGL((decode_multi_kernel<DK, DV, InT, KDA, true>), dim3(blocks), dim3(256), 0, s,
                           n_units, T, H, scale, static_cast<const InT*>(q), static_cast<const InT*>(k),
                           static_cast<const InT*>(v), alpha, beta, state, static_cast<InT*>(o), states, pro);
    } else {
        hipLaunchKernelGGL((decode_multi_kernel<DK, DV, InT, KDA, false>), dim3(blocks), dim3(256), 0, s,
                           n_units, T, H, scale, static_cast<const InT*>(q), static_cast<const InT*>(k),
                           static_cast<const InT*>(v), alpha, beta, state, static_cast<InT*>(o), states, pro);
    }
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t multi_type(int kda, int dtype, int n, int T, int H, float scale, const void* q,
                      const void* k, const void* v, const float* alpha, const float* beta,
                      float* state, void* o, float* states, hipStream_t s, int pro) {
    if (dtype == GDR_DTYPE_BF16) {
        return kda ? launch_multi<DK, DV, bf16_t, true>(n, T, H, scale, q, k, v, alpha, beta, state, o, states, s, pro)
                   : launch_multi<DK, DV, bf16_t, false>(n, T, H, scale, q, k, v, alpha, beta, state, o, states, s, pro);
    }
    return kda ? launch_multi<DK, DV, float, true>(n, T, H, scale, q, k, v, alpha, beta, state, o, states, s, pro)
               : launch_multi<DK, DV, float, false>(n, T, H, scale, q, k, v, alpha, beta, state, o, states, s, pro);
}

template <int DK>
hipError_t multi_dv(int kda, int dtype, int dv, int n, int T, int H, float scale, const void* q,
                    const void* k, const void* v, const float* alpha, const float* beta,
                    float* state, void* o, float* states, hipStream_t s, int pro) {
    switch (dv) {
        case 16: return multi_type<DK, 16>(kda, dtype, n, T, H, scale, q, k, v, alpha, beta, state, o, states, s, pro);
        case 32: return multi_type<DK, 32>(kda, dtype, n, T, H, scale, q, k, v, alpha, beta, state, o, states, s, pro);
        case 64: return multi_type<DK, 64>(kda, dtype, n, T, H, scale, q, k, v, alpha, beta, state, o, states, s, pro);
        default: return multi_type<DK, 128>(kda, dtype, n, T, H, scale, q, k, v, alpha, beta, state, o, states, s, pro);
    }
}

}  // namespace

hipError_t launch_decode(int kda, int dtype, int B, int H, int dk, int dv, float scale,
                         const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, float* state, void* o, hipStream_t s, int pro) {
    const int n = B * H;
    switch (dk) {
        case 16: return dispatch_dv<16>(kda, dtype, dv, n, scale, q, k, v, alpha, beta, state, o, s, pro);
        case 32: return dispatch_dv<32>(kda, dtype, dv, n, scale, q, k, v, alpha, beta, state, o, s, pro);
        case 64: return dispatch_dv<64>(kda, dtype, dv, n, scale, q, k, v, alpha, beta, state, o, s, pro);
        default: return dispatch_dv<128>(kda, dtype, dv, n, scale, q, k, v, alpha, beta, state, o, s, pro);
    }
}

hipError_t launch_decode_multi(int kda, int dtype, int B, int T, int H, int dk, int dv,
                               float scale, const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta, float* state, void* o,
                               float* states, hipStream_t s, int pro) {
    const int n = B * H;
    switch (dk) {
        case 16: return multi_dv<16>(kda, dtype, dv, n, T, H, scale, q, k, v, alpha, beta, state, o, states, s, pro);
        case 32: return multi_dv<32>(kda, dtype, dv, n, T, H, scale, q, k, v, alpha, beta, state, o, states, s, pro);
        case 64: return multi_dv<64>(kda, dtype, dv, n, T, H, scale, q, k, v, alpha, beta, state, o, states, s, pro);
        default: return multi_dv<128>(kda, dtype, dv, n, T, H, scale, q, k, v, alpha, beta, state, o, states, s, pro);
    }
}

}  // namespace gdr
