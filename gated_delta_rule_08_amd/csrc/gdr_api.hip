// C ABI of libgdr: argument validation and dispatch.  Every check runs before
// the first HIP call, so invalid calls never touch the device.
#include <limits.h>
#include <stdint.h>

#include "gdr_internal.h"

namespace gdr {
namespace {

__global__ __launch_bounds__(256) void state_copy_kernel(const float4* __restrict__ in,
                                                         float4* __restrict__ out, size_t n4) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
         i += static_cast<size_t>(gridDim.x) * 256)
        out[i] = in ? in[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

hipError_t launch_state_copy(const float* state_in, float* state_out, size_t n, hipStream_t s) {
    if (state_in == state_out || n == 0) return hipSuccess;
    const size_t n4 = n / 4;  // n = B*H*dk*dv is a multiple of 256
    const size_t want = (n4 + 255) / 256;
    const unsigned blocks = static_cast<unsigned>(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(state_copy_kernel, dim3(blocks), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(state_in),
                       reinterpret_cast<float4*>(state_out), n4);
    return hipGetLastError();
}

}  // namespace gdr

namespace {

inline bool head_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
constexpr int kMaxMultiTokens = 64;  // gdr_decode_multi: a verify window, not a prompt
inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Largest element count of any tensor must fit comfortably in size_t and
// every grid dimension in an int.
inline bool sizes_ok(long long B, long long T, long long H, long long dk, long long dv) {
    const long long lim = 1LL << 40;
    if (B * H > INT_MAX / 8) return false;
    if (B * H * dk * dv > lim) return false;
    if (B * T > lim / (H > 0 ? H : 1)) return false;
    if (B * T * H > lim / 128) return false;
    return true;
}

// The backward runs 1024-thread workgroups, one per (b, h, chunk) and one per
// (b, h, 16 value columns) over whole groups of 8 heads: each dispatch's
// work-item count has to fit 32 bits.
inline bool backward_grid_ok(long long B, long long T, long long H, long long dv) {
    return B * H * ((T + 63) / 64) < (1LL << 22) && (B * H + 7) / 8 * 8 * (dv / 16) < (1LL << 22);
}
// A launcher's hipErrorInvalidConfiguration means a grid too large for one
// dispatch (checked before any HIP call): reported as a shape error.
inline int status_of(hipError_t e) {
    return e == hipSuccess ? GDR_OK : e == hipErrorInvalidConfiguration ? GDR_ERR_BAD_SHAPE : GDR_ERR_HIP;
}

constexpr int kProFlags = GDR_PRO_L2NORM_QK | GDR_PRO_SIGMOID;
constexpr int kSchedFlags = GDR_SCHED_FUSED | GDR_SCHED_SPLIT;
// decode calls: prologue bits only
inline bool flags_ok(int flags) { return (flags & ~kProFlags) == 0; }
// prefill calls: prologue bits and at most one schedule bit
inline bool prefill_flags_ok(int flags) {
    return (flags & ~(kProFlags | kSchedFlags)) == 0 && (flags & kSchedFlags) != kSchedFlags;
}
// The schedule bits against the dtype and gate, and the prologue against the
// schedule that runs: only bf16 has two schedules, KDA runs split only, and
// the bf16 schedules normalise q, k where the kernel forming the chunk-local
// products stages them itself (GDN fused, KDA split).
int schedule_status(int flags, int gate, int dtype) {
    const int sched = flags & kSchedFlags;
    if (dtype != GDR_DTYPE_BF16) return sched ? GDR_ERR_UNSUPPORTED : GDR_OK;
    const int kda = gate == GDR_GATE_KDA;
    if (kda && (sched & GDR_SCHED_FUSED)) return GDR_ERR_UNSUPPORTED;
    if ((flags & GDR_PRO_L2NORM_QK) && !kda && gdr::prefill_bf16_split(kda, flags))
        return GDR_ERR_UNSUPPORTED;
    return GDR_OK;
}

int check_enums(int gate, int dtype) {
    if (gate != GDR_GATE_GDN && gate != GDR_GATE_KDA) return GDR_ERR_BAD_ENUM;
    if (dtype != GDR_DTYPE_F32 && dtype != GDR_DTYPE_BF16) return GDR_ERR_BAD_ENUM;
    return GDR_OK;
}

// Everything gdr_chunk_prefill_ex checks apart from the workspace, in order,
// after the enums, flags and sizes (done by the caller).
int prefill_pointer_checks(int gate, int B, int T, int H, int dk, int dv, const void* q,
                           const void* k, const void* v, const float* alpha, const float* beta,
                           const float* state_in, const float* state_out, const void* o) {
    if (!state_out) return GDR_ERR_NULL_PTR;
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !o)) return GDR_ERR_NULL_PTR;
    const int kda = gate == GDR_GATE_KDA;
    if (!aligned(state_out, 16) || (state_in && !aligned(state_in, 16))) return GDR_ERR_MISALIGNED;
    if (T > 0 && (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
                  !aligned(beta, 4) || !aligned(alpha, kda ? 16 : 4)))
        return GDR_ERR_MISALIGNED;
    if (state_in && state_in != state_out) {
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(state_in);
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(state_out);
        const uintptr_t len = static_cast<size_t>(B) * H * dk * dv * sizeof(float);
        if (a0 < b0 + len && b0 < a0 + len) return GDR_ERR_ALIAS;
    }
    return GDR_OK;
}

// Enums, flags, shapes and schedule of a chunked prefill call.
int prefill_arg_checks(int gate, int dtype, int flags, int B, int T, int H, int dk, int dv,
                       int chunk) {
    int st = check_enums(gate, dtype);
    if (st != GDR_OK) return st;
    if (!prefill_flags_ok(flags)) return GDR_ERR_BAD_ENUM;
    if (B < 0 || H < 0 || T < 0) return GDR_ERR_BAD_SHAPE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv) || chunk != 64) return GDR_ERR_UNSUPPORTED;
    if ((st = schedule_status(flags, gate, dtype)) != GDR_OK) return st;
    if (!sizes_ok(B, T, H, dk, dv)) return GDR_ERR_BAD_SHAPE;
    return GDR_OK;
}

// The launch of a validated prefill call (T == 0: the state copy).
int prefill_launch(int gate, int dtype, int flags, int B, int T, int H, int dk, int dv,
                   float scale, const void* q, const void* k, const void* v, const float* alpha,
                   const float* beta, const float* state_in, float* state_out, void* o,
                   void* workspace, size_t workspace_bytes, hipStream_t s) {
    const int kda = gate == GDR_GATE_KDA;
    gdr::Opts opt;
    opt.pro = flags & kProFlags;
    hipError_t e;
    if (T == 0) {
        e = gdr::launch_state_copy(state_in, state_out, static_cast<size_t>(B) * H * dk * dv, s);
    } else if (dtype == GDR_DTYPE_F32) {
        e = gdr::launch_prefill_f32(kda, B, T, H, dk, dv, scale, static_cast<const float*>(q),
                                    static_cast<const float*>(k), static_cast<const float*>(v),
                                    alpha, beta, state_in, state_out, static_cast<float*>(o), s, opt);
    } else {
        e = gdr::launch_prefill_bf16(kda, B, T, H, dk, dv, scale,
                                     static_cast<const gdr::bf16_t*>(q),
                                     static_cast<const gdr::bf16_t*>(k),
                                     static_cast<const gdr::bf16_t*>(v), alpha, beta, state_in,
                                     state_out, static_cast<gdr::bf16_t*>(o), workspace,
                                     workspace_bytes, s, flags, opt);
    }
    return status_of(e);
}

}  // namespace

extern "C" {

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

const char* gdr_status_string(int status) {
    switch (status) {
        case GDR_OK: return "GDR_OK: success";
        case GDR_ERR_NULL_PTR: return "GDR_ERR_NULL_PTR: a required pointer is NULL";
        case GDR_ERR_BAD_SHAPE: return "GDR_ERR_BAD_SHAPE: a size is negative or too large";
        case GDR_ERR_UNSUPPORTED:
            return "GDR_ERR_UNSUPPORTED: dk and dv must be 16, 32, 64 or 128 and chunk must be 64";
        case GDR_ERR_MISALIGNED:
            return "GDR_ERR_MISALIGNED: tensors need 16-byte alignment (beta and GDN alpha 4-byte)";
        case GDR_ERR_WORKSPACE: return "GDR_ERR_WORKSPACE: workspace missing or too small";
        case GDR_ERR_BAD_ENUM: return "GDR_ERR_BAD_ENUM: unknown gate mode, dtype or flag";
        case GDR_ERR_HIP: return "GDR_ERR_HIP: the HIP runtime rejected a launch";
        case GDR_ERR_ALIAS: return "GDR_ERR_ALIAS: two state buffers (partially) overlap";
        case GDR_ERR_SCRATCH:
            return "GDR_ERR_SCRATCH: one chunk of every head needs more than the 96 MiB fixed scratch of "
                   "gdr_chunk_prefill_noalloc";
        default: return "unknown gdr status";
    }
}

int gdr_decode_step(int gate, int dtype, int B, int H, int dk, int dv, float scale,
                    const void* q, const void* k, const void* v, const float* alpha,
                    const float* beta, float* state, void* o, void* stream) {
    return gdr_decode_step_ex(gate, dtype, 0, B, H, dk, dv, scale, q, k, v, alpha, beta, state, o,
                              stream);
}

int gdr_decode_step_ex(int gate, int dtype, int flags, int B, int H, int dk, int dv, float scale,
                       const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, float* state, void* o, void* stream) {
    int st = check_enums(gate, dtype);
    if (st != GDR_OK) return st;
    if (!flags_ok(flags)) return GDR_ERR_BAD_ENUM;
    if (B < 0 || H < 0) return GDR_ERR_BAD_SHAPE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return GDR_ERR_UNSUPPORTED;
    if (!sizes_ok(B, 1, H, dk, dv)) return GDR_ERR_BAD_SHAPE;
    if (B == 0 || H == 0) return GDR_OK;
    if (!q || !k || !v || !alpha || !beta || !state || !o) return GDR_ERR_NULL_PTR;
    const int kda = gate == GDR_GATE_KDA;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(state, 16) || !aligned(beta, 4) || !aligned(alpha, kda ? 16 : 4))
        return GDR_ERR_MISALIGNED;
    hipError_t e = gdr::launch_decode(kda, dtype, B, H, dk, dv, scale, q, k, v, alpha, beta,
                                      state, o, static_cast<hipStream_t>(stream), flags);
    return status_of(e);
}

int gdr_decode_multi(int gate, int dtype, int B, int T, int H, int dk, int dv, float scale,
                     const void* q, const void* k, const void* v, const float* alpha,
                     const float* beta, float* state, void* o, float* states, void* stream) {
    return gdr_decode_multi_ex(gate, dtype, 0, B, T, H, dk, dv, scale, q, k, v, alpha, beta, state,
                               o, states, stream);
}

int gdr_decode_multi_ex(int gate, int dtype, int flags, int B, int T, int H, int dk, int dv,
                        float scale, const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, float* state, void* o,
                        float* states, void* stream) {
    int st = check_enums(gate, dtype);
    if (st != GDR_OK) return st;
    if (!flags_ok(flags)) return GDR_ERR_BAD_ENUM;
    if (B < 0 || H < 0 || T < 0) return GDR_ERR_BAD_SHAPE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv) || T > kMaxMultiTokens) return GDR_ERR_UNSUPPORTED;
    if (!sizes_ok(B, T, H, dk, dv) || static_cast<long long>(B) * T * H * dk * dv > (1LL << 40))
        return GDR_ERR_BAD_SHAPE;
    if (B == 0 || H == 0 || T == 0) return GDR_OK;
    if (!q || !k || !v || !alpha || !beta || !state || !o) return GDR_ERR_NULL_PTR;
    const int kda = gate == GDR_GATE_KDA;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(state, 16) || (states && !aligned(states, 16)) || !aligned(beta, 4) ||
        !aligned(alpha, kda ? 16 : 4))
        return GDR_ERR_MISALIGNED;
    if (states) {
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(state);
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(states);
        const uintptr_t la = static_cast<uintptr_t>(B) * H * dk * dv * sizeof(float);
        const uintptr_t lb = la * static_cast<uintptr_t>(T);
        if (a0 < b0 + lb && b0 < a0 + la) return GDR_ERR_ALIAS;
    }
    hipError_t e = gdr::launch_decode_multi(kda, dtype, B, T, H, dk, dv, scale, q, k, v, alpha,
                                            beta, state, o, states, static_cast<hipStream_t>(stream),
                                            flags);
    return status_of(e);
}

size_t gdr_chunk_prefill_workspace_bytes(int gate, int dtype, int B, int T, int H, int dk,
                                         int dv, int chunk) {
    return gdr_chunk_prefill_workspace_bytes_ex(gate, dtype, 0, B, T, H, dk, dv, chunk);
}

size_t gdr_chunk_prefill_workspace_bytes_ex(int gate, int dtype, int flags, int B, int T, int H,
                                            int dk, int dv, int chunk) {
    if (check_enums(gate, dtype) != GDR_OK || !prefill_flags_ok(flags) ||
        schedule_status(flags, gate, dtype) != GDR_OK || chunk != 64 || B < 0 || H < 0 || T < 0 ||
        !head_dim_ok(dk) || !head_dim_ok(dv) || !sizes_ok(B, T, H, dk, dv))
        return 0;
    // The fp32 path keeps its intermediates on chip; the bf16 path's split
    // schedule stages per-chunk images of its chunk-local products.
    if (dtype != GDR_DTYPE_BF16) return 0;
    return gdr::prefill_bf16_workspace(gate == GDR_GATE_KDA, flags, B, T, H, dk);
}

int gdr_chunk_prefill(int gate, int dtype, int B, int T, int H, int dk, int dv, int chunk,
                      float scale, const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, const float* state_in,
                      float* state_out, void* o, void* workspace, size_t workspace_bytes,
                      void* stream) {
    return gdr_chunk_prefill_ex(gate, dtype, 0, B, T, H, dk, dv, chunk, scale, q, k, v, alpha,
                                beta, state_in, state_out, o, workspace, workspace_bytes, stream);
}

int gdr_chunk_prefill_ex(int gate, int dtype, int flags, int B, int T, int H, int dk, int dv,
                         int chunk, float scale, const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta, const float* state_in,
                         float* state_out, void* o, void* workspace, size_t workspace_bytes,
                         void* stream) {
    int st = prefill_arg_checks(gate, dtype, flags, B, T, H, dk, dv, chunk);
    if (st != GDR_OK) return st;
    const size_t need = gdr_chunk_prefill_workspace_bytes_ex(gate, dtype, flags, B, T, H, dk, dv, chunk);
    if (workspace_bytes < need || (need > 0 && !workspace)) return GDR_ERR_WORKSPACE;
    if (B == 0 || H == 0) return GDR_OK;
    if ((st = prefill_pointer_checks(gate, B, T, H, dk, dv, q, k, v, alpha, beta, state_in, state_out,
                                     o)) != GDR_OK)
        return st;
    return prefill_launch(gate, dtype, flags, B, T, H, dk, dv, scale, q, k, v, alpha, beta, state_in,
                          state_out, o, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int gdr_chunk_prefill_noalloc(int gate, int dtype, int flags, int B, int T, int H, int dk, int dv,
                              int chunk, float scale, const void* q, const void* k, const void* v,
                              const float* alpha, const float* beta, const float* state_in,
                              float* state_out, void* o, void* stream) {
    int st = prefill_arg_checks(gate, dtype, flags, B, T, H, dk, dv, chunk);
    if (st != GDR_OK) return st;
    if (B == 0 || H == 0) return GDR_OK;
    const bool split = dtype == GDR_DTYPE_BF16 && T > 0 && gdr::prefill_bf16_split(gate == GDR_GATE_KDA, flags);
    // the images of one chunk of every head have to fit the fixed scratch
    if (split && static_cast<size_t>(B) * H * gdr::prefill_bf16_image_bytes(gate == GDR_GATE_KDA, dk) >
                     gdr::kNoallocScratchBytes)
        return GDR_ERR_SCRATCH;
    if ((st = prefill_pointer_checks(gate, B, T, H, dk, dv, q, k, v, alpha, beta, state_in, state_out,
                                     o)) != GDR_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* scratch = nullptr;
    if (split && gdr::noalloc_scratch(s, &scratch) != hipSuccess) return GDR_ERR_HIP;
    return prefill_launch(gate, dtype, flags, B, T, H, dk, dv, scale, q, k, v, alpha, beta, state_in,
                          state_out, o, scratch, split ? gdr::kNoallocScratchBytes : 0, s);
}

size_t gdr_chunk_prefill_varlen_workspace_bytes(int gate, int dtype, int N, int max_T, int H,
                                                int dk, int dv, int chunk) {
    return gdr_chunk_prefill_workspace_bytes_ex(gate, dtype, 0, N, max_T, H, dk, dv, chunk);
}

size_t gdr_chunk_prefill_varlen_workspace_bytes_ex(int gate, int dtype, int flags, int N,
                                                   int max_T, int H, int dk, int dv, int chunk) {
    return gdr_chunk_prefill_workspace_bytes_ex(gate, dtype, flags, N, max_T, H, dk, dv, chunk);
}

int gdr_chunk_prefill_varlen(int gate, int dtype, int N, int total_T, int max_T, int H, int dk,
                             int dv, int chunk, float scale, const void* q, const void* k,
                             const void* v, const float* alpha, const float* beta,
                             const int* cu_seqlens, const int* state_slots, const int* has_state,
                             float* states, int n_slots, void* o, void* workspace,
                             size_t workspace_bytes, void* stream) {
    return gdr_chunk_prefill_varlen_ex(gate, dtype, 0, N, total_T, max_T, H, dk, dv, chunk, scale, q,
                                       k, v, alpha, beta, cu_seqlens, state_slots, has_state, states,
                                       n_slots, o, workspace, workspace_bytes, stream);
}

int gdr_chunk_prefill_varlen_ex(int gate, int dtype, int flags, int N, int total_T, int max_T,
                                int H, int dk, int dv, int chunk, float scale, const void* q,
                                const void* k, const void* v, const float* alpha,
                                const float* beta, const int* cu_seqlens, const int* state_slots,
                                const int* has_state, float* states, int n_slots, void* o,
                                void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_enums(gate, dtype);
    if (st != GDR_OK) return st;
    if (!prefill_flags_ok(flags)) return GDR_ERR_BAD_ENUM;
    if (N < 0 || total_T < 0 || max_T < 0 || H < 0 || n_slots < 0) return GDR_ERR_BAD_SHAPE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv) || chunk != 64) return GDR_ERR_UNSUPPORTED;
    if ((st = schedule_status(flags, gate, dtype)) != GDR_OK) return st;
    if (!sizes_ok(1, total_T, H, dk, dv) || !sizes_ok(N, max_T, H, dk, dv) ||
        !sizes_ok(n_slots, 1, H, dk, dv))
        return GDR_ERR_BAD_SHAPE;
    const size_t need =
        gdr_chunk_prefill_varlen_workspace_bytes_ex(gate, dtype, flags, N, max_T, H, dk, dv, chunk);
    if (workspace_bytes < need || (need > 0 && !workspace)) return GDR_ERR_WORKSPACE;
    if (N == 0 || H == 0) return GDR_OK;
    if (!cu_seqlens || !state_slots || !states) return GDR_ERR_NULL_PTR;
    if (total_T > 0 && (!q || !k || !v || !alpha || !beta || !o)) return GDR_ERR_NULL_PTR;
    const int kda = gate == GDR_GATE_KDA;
    if (!aligned(states, 16) || !aligned(cu_seqlens, 4) || !aligned(state_slots, 4) ||
        (has_state && !aligned(has_state, 4)))
        return GDR_ERR_MISALIGNED;
    if (total_T > 0 && (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
                        !aligned(beta, 4) || !aligned(alpha, kda ? 16 : 4)))
        return GDR_ERR_MISALIGNED;
    gdr::Opts vl;
    vl.cu = cu_seqlens;
    vl.slot = state_slots;
    vl.has = has_state;
    vl.n_slots = n_slots;
    vl.total = total_T;
    vl.pro = flags & kProFlags;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dtype == GDR_DTYPE_F32) {
        e = gdr::launch_prefill_f32(kda, N, max_T, H, dk, dv, scale, static_cast<const float*>(q),
                                    static_cast<const float*>(k), static_cast<const float*>(v),
                                    alpha, beta, states, states, static_cast<float*>(o), s, vl);
    } else {
        e = gdr::launch_prefill_bf16(kda, N, max_T, H, dk, dv, scale,
                                     static_cast<const gdr::bf16_t*>(q),
                                     static_cast<const gdr::bf16_t*>(k),
                                     static_cast<const gdr::bf16_t*>(v), alpha, beta, states,
                                     states, static_cast<gdr::bf16_t*>(o), workspace, workspace_bytes,
                                     s, flags, vl);
    }
    return status_of(e);
}

size_t gdr_chunk_backward_workspace_bytes(int gate, int dtype, int B, int T, int H, int dk,
                                          int dv, int chunk) {
    if (check_enums(gate, dtype) != GDR_OK || chunk != 64 || B < 0 || H < 0 || T < 0 ||
        !head_dim_ok(dk) || !head_dim_ok(dv) || !sizes_ok(B, T, H, dk, dv) ||
        !backward_grid_ok(B, T, H, dv))
        return 0;
    if (B == 0 || H == 0 || T == 0) return 0;
    return gdr::backward_workspace_floats(B, T, H, dk, dv) * sizeof(float);
}

size_t gdr_chunk_backward_workspace_bytes_ranged(int gate, int dtype, int B, int T, int H, int dk,
                                                 int dv, int chunk, int range_chunks) {
    if (range_chunks < 1) return 0;
    if (gdr_chunk_backward_workspace_bytes(gate, dtype, B, T, H, dk, dv, chunk) == 0) return 0;
    return gdr::backward_workspace_floats_ranged(B, T, H, dk, dv, range_chunks) * sizeof(float);
}

int gdr_chunk_backward(int gate, int dtype, int B, int T, int H, int dk, int dv, int chunk,
                       float scale, const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, const float* state_in,
                       const void* grad_o, const float* grad_state_out, void* grad_q,
                       void* grad_k, void* grad_v, float* grad_alpha, float* grad_beta,
                       float* grad_state_in, void* workspace, size_t workspace_bytes,
                       void* stream) {
    int st = check_enums(gate, dtype);
    if (st != GDR_OK) return st;
    if (B < 0 || H < 0 || T < 0) return GDR_ERR_BAD_SHAPE;
    if (!head_dim_ok(dk) || !head_dim_ok(dv) || chunk != 64) return GDR_ERR_UNSUPPORTED;
    if (!sizes_ok(B, T, H, dk, dv)) return GDR_ERR_BAD_SHAPE;
    if (!backward_grid_ok(B, T, H, dv)) return GDR_ERR_BAD_SHAPE;
    // the smallest workspace: ranges of one chunk (the whole sequence runs at
    // once from gdr_chunk_backward_workspace_bytes on)
    const size_t need = gdr_chunk_backward_workspace_bytes_ranged(gate, dtype, B, T, H, dk, dv, chunk, 1);
    if (workspace_bytes < need || (need > 0 && !workspace)) return GDR_ERR_WORKSPACE;
    if (B == 0 || H == 0) return GDR_OK;
    const int kda = gate == GDR_GATE_KDA;
    if (T > 0 && (!q || !k || !v || !alpha || !beta || !grad_o || !grad_q || !grad_k || !grad_v ||
                  !grad_alpha || !grad_beta))
        return GDR_ERR_NULL_PTR;
    if ((state_in && !aligned(state_in, 16)) || (grad_state_out && !aligned(grad_state_out, 16)) ||
        (grad_state_in && !aligned(grad_state_in, 16)) || (workspace && !aligned(workspace, 16)))
        return GDR_ERR_MISALIGNED;
    if (T > 0 && (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(grad_o, 16) ||
                  !aligned(grad_q, 16) || !aligned(grad_k, 16) || !aligned(grad_v, 16) ||
                  !aligned(beta, 4) || !aligned(grad_beta, 4) || !aligned(alpha, kda ? 16 : 4) ||
                  !aligned(grad_alpha, kda ? 16 : 4)))
        return GDR_ERR_MISALIGNED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (T == 0) {
        e = grad_state_in ? gdr::launch_state_copy(grad_state_out, grad_state_in,
                                                    static_cast<size_t>(B) * H * dk * dv, s)
                          : hipSuccess;
    } else {
        e = gdr::launch_backward(kda, dtype, B, T, H, dk, dv, scale, q, k, v, alpha, beta, state_in,
                                 grad_o, grad_state_out, grad_q, grad_k, grad_v, grad_alpha,
                                 grad_beta, grad_state_in, static_cast<float*>(workspace),
                                 workspace_bytes / sizeof(float), s);
    }
    return status_of(e);
}

}  // extern "C"
