// Internal declarations shared by the translation units of libgdr.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr.h"

namespace gdr {

// bfloat16 is carried as its 16-bit pattern.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round to nearest even; NaN is kept a (quiet) NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static void store(float* p, float x) { *p = x; }
};
template <> struct Elem<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
    __device__ __forceinline__ static void store(bf16_t* p, float x) { *p = f32_to_bf16(x); }
};

// Per-launch options of the prefill kernels.
//  Packed variable-length sequences (all pointers device memory; all null for
//  the uniform [B, T, H, .] layout): sequence b holds tokens cu[b] .. cu[b+1]-1
//  of the packed token tensors and its state is row slot[b] of the state pool;
//  has[b] == 0 starts it from zeros.  A kernel skips (writes nothing for) a
//  sequence whose offsets or slot are out of range.
//  pro: input prologue flags (GDR_PRO_*), applied where q, k and the gates are
//  loaded.
struct Opts {
    const int* cu = nullptr;
    const int* slot = nullptr;
    const int* has = nullptr;
    int n_slots = 0;  // rows of the state pool
    int total = 0;    // tokens of the packed tensors
    int pro = 0;
};

// Input prologue helpers (fp32).  A row is divided by max(||x||, 1e-12), i.e.
// multiplied by rsqrt(max(sum x^2, 1e-24)); sigmoid and log2(sigmoid) in a
// form that neither overflows nor loses the small-gate end.
constexpr float kNormEps2 = 1e-24f;
__device__ __forceinline__ float inv_norm(float sumsq) { return rsqrtf(fmaxf(sumsq, kNormEps2)); }
__device__ __forceinline__ float sigmoid_f(float z) { return 1.f / (1.f + __expf(-z)); }
__device__ __forceinline__ float log2_sigmoid(float z) {
    // log2 sigma(z) = -(max(-z, 0) log2 e + log2(1 + 2^(-|z| log2 e)))
    constexpr float kLog2e = 1.4426950408889634f;
    return -(fmaxf(-z, 0.f) * kLog2e + __log2f(1.f + exp2f(-fabsf(z) * kLog2e)));
}

// A dispatch's work-item count (workgroups x threads) has to fit 32 bits.
// Launchers check their grids with this before any HIP call and return
// hipErrorInvalidConfiguration for a shape that would exceed it.
inline bool grid_fits(unsigned long long blocks, unsigned long long threads) {
    return blocks * threads <= 0xFFFFFFFFull;
}

// Launchers, one per kernel family.  They assume validated arguments and
// return the hipError_t of the launch.
// pro: input prologue flags (GDR_PRO_*).
hipError_t launch_decode(int kda, int dtype, int B, int H, int dk, int dv, float scale,
                         const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, float* state, void* o, hipStream_t s, int pro = 0);
// T decode steps per head; token tensors [B, T, H, .]; states (optional)
// receives the state after every token, [B, T, H, dk, dv].
hipError_t launch_decode_multi(int kda, int dtype, int B, int T, int H, int dk, int dv,
                               float scale, const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta, float* state, void* o,
                               float* states, hipStream_t s, int pro = 0);

hipError_t launch_prefill_f32(int kda, int B, int T, int H, int dk, int dv, float scale,
                              const float* q, const float* k, const float* v,
                              const float* alpha, const float* beta, const float* state_in,
                              float* state_out, float* o, hipStream_t s, const Opts& vl = Opts());

// The bf16 prefill runs its split schedule (chunk-local kernel, then chain
// kernel, `workspace` of at least prefill_bf16_workspace(...) bytes) when
// prefill_bf16_split(kda, flags) holds, else the fused kernel (no
// workspace).  flags: the GDR_SCHED_* bits of the call (validated).
// workspace_bytes caps the split schedule's ranges of chunks (each range's
// images must fit); at least prefill_bf16_workspace(...) or B*H image bytes.
hipError_t launch_prefill_bf16(int kda, int B, int T, int H, int dk, int dv, float scale,
                               const bf16_t* q, const bf16_t* k, const bf16_t* v,
                               const float* alpha, const float* beta, const float* state_in,
                               float* state_out, bf16_t* o, void* workspace, size_t workspace_bytes,
                               hipStream_t s, int flags, const Opts& vl = Opts());
bool prefill_bf16_split(int kda, int flags);
size_t prefill_bf16_workspace(int kda, int flags, int B, int T, int H, int dk);
// Bytes of one (head, chunk) image of the split schedule.
size_t prefill_bf16_image_bytes(int kda, int dk);

// Fixed scratch of gdr_chunk_prefill_noalloc: a file-scope device array per
// GPU (noalloc.hip).  noalloc_scratch returns its address on the device of
// `stream` (the current device for the null stream), looked up on first use.
constexpr size_t kNoallocScratchBytes = size_t(96) << 20;
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

// Backward of the chunked recurrence (fp32 arithmetic; q, k, v, d_o, dq, dk,
// dv in the element type `dtype`).  ws: ws_floats floats, at least
// backward_workspace_floats_ranged(..., 1); with backward_workspace_floats(...)
// the whole sequence runs at once, with less it runs in the widest chunk
// ranges that fit (a forward pass for the range start states, then the
// ranges from the last).
size_t backward_workspace_floats(int B, int T, int H, int dk, int dv);
size_t backward_workspace_floats_ranged(int B, int T, int H, int dk, int dv, int range_chunks);
hipError_t launch_backward(int kda, int dtype, int B, int T, int H, int dk, int dv, float scale,
                           const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* state_in, const void* d_o,
                           const float* d_state_out, void* dq, void* dkk, void* dvv, float* dalpha,
                           float* dbeta, float* d_state_in, float* ws, size_t ws_floats, hipStream_t s);

// state_out <- state_in (or zeros when state_in is NULL), n floats.
hipError_t launch_state_copy(const float* state_in, float* state_out, size_t n, hipStream_t s);

}  // namespace gdr
