/*
 * gdr.h -- C ABI of the gated delta-rule token mixer for AMD MI355X (gfx950).
 *
 * The mixer.  "Super Apriel: One Checkpoint, Many Speeds"
 * (gist.science/paper/2604.19877), §2.A "The Supernet Architecture", lists
 * two recurrent token mixers with a fixed-size state and O(n) time: Gated
 * DeltaNet (GDN), a delta rule with a scalar gate, and Kimi Delta Attention
 * (KDA), delta attention with a channel-wise gate; §2.D "Inference &
 * Serving" runs them in decode (including an all-GDN speculative draft).
 * The pages print no update rule; this library computes the gated delta rule
 * in its usual form, per batch entry b and head h, with an fp32 state
 * S in R^{dk x dv} (row i = key channel, column j = value channel):
 *
 *     S_t = (I - beta_t k_t k_t^T) D_t S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * D_t = alpha_t I for GDN (one scalar gate per token and head) and
 * D_t = diag(alpha_t) for KDA (alpha_t in R^dk, acting on the key axis).
 * The gate is applied before the delta correction; the output reads the
 * post-update state.  alpha and beta are given in linear space (already
 * passed through their activations); alpha is expected in [0, 1].
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer to a dense, row-major buffer
 *    owned by the caller.  The library allocates and frees nothing and keeps
 *    no mutable global state (apart from gdr_chunk_prefill_noalloc's fixed
 *    scratch, see there); concurrent calls on different streams are safe as
 *    long as their output buffers do not overlap.
 *  - q, k, v, o share one element type, selected by `dtype`: GDR_DTYPE_F32
 *    (IEEE fp32) or GDR_DTYPE_BF16 (bfloat16, outputs rounded to nearest
 *    even).  alpha, beta and the state are always fp32.
 *  - Supported head sizes: dk, dv in {16, 32, 64, 128}.  The chunk size of
 *    the prefill is 64.
 *  - Alignment: q, k, v, o, the state buffers and KDA alpha must be 16-byte
 *    aligned; beta and GDN alpha 4-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued on it; no call synchronises the host.
 *  - Arguments are validated completely before any HIP call, so an invalid
 *    call returns an error without touching the device.  Faults inside a
 *    kernel surface at the caller's next synchronisation; launch failures
 *    return GDR_ERR_HIP.
 *  - Zero-sized problems (B == 0 or H == 0) are no-ops that return GDR_OK;
 *    their pointers may then be NULL.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 2

/* Gate mode: scalar gate (Gated DeltaNet) or channel-wise gate (Kimi Delta
 * Attention), the two mixers of the pages' §2.A. */
typedef enum { GDR_GATE_GDN = 0, GDR_GATE_KDA = 1 } gdr_gate_t;

/* Element type of q, k, v and o. */
typedef enum { GDR_DTYPE_F32 = 0, GDR_DTYPE_BF16 = 1 } gdr_dtype_t;

/* Status codes.  0 is success; errors are negative. */
enum {
    GDR_OK = 0,
    GDR_ERR_NULL_PTR = -1,    /* a required pointer is NULL                 */
    GDR_ERR_BAD_SHAPE = -2,   /* a size is negative or overflows (also: a
                                 launch would exceed 2^32 work-items)       */
    GDR_ERR_UNSUPPORTED = -3, /* dk, dv or chunk outside the supported set  */
    GDR_ERR_MISALIGNED = -4,  /* a pointer violates the alignment rule      */
    GDR_ERR_WORKSPACE = -5,   /* workspace missing or too small             */
    GDR_ERR_BAD_ENUM = -6,    /* gate, dtype or flags not known             */
    GDR_ERR_HIP = -7,         /* the HIP runtime rejected a launch          */
    GDR_ERR_ALIAS = -8,       /* two state buffers (partially) overlap      */
    GDR_ERR_SCRATCH = -9      /* gdr_chunk_prefill_noalloc: the problem
                                 needs more than its fixed scratch          */
};

/*
 * One decode step for B x H independent heads, updating the state in place
 * (the per-token step of §2.D's decode; one token per head).
 *
 *   q, k   [B, H, dk]   dtype         v, o   [B, H, dv]   dtype
 *   alpha  [B, H] (GDN) or [B, H, dk] (KDA), fp32
 *   beta   [B, H], fp32
 *   state  [B, H, dk, dv], fp32, read and overwritten with S_t
 *
 * o may not overlap any input.  Returns a GDR_* status.
 */
int gdr_decode_step(int gate, int dtype, int B, int H, int dk, int dv, float scale,
                    const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta,
                    float* state, void* o, void* stream);

/*
 * Input prologue flags of the *_ex entry points (bitwise OR; 0 = none).  The
 * mixers' inputs usually come out of a projection followed by two cheap
 * transforms; these flags run them inside the kernels, where q, k and the
 * gates are loaded, instead of as separate passes over HBM:
 *   GDR_PRO_L2NORM_QK   q and k are raw: each dk-vector q[b,t,h,:] and
 *                       k[b,t,h,:] is divided by max(||x||_2, 1e-12) in fp32
 *                       (bf16 inputs: the normalised values feed the bf16
 *                       matrix products rounded to bf16 again).
 *   GDR_PRO_SIGMOID     alpha and beta are logits: the kernels use
 *                       sigmoid(alpha) and sigmoid(beta) (the chunked paths
 *                       take log2 sigmoid(alpha) directly, so very negative
 *                       logits keep their size instead of underflowing).
 * Other bits (apart from the prefill calls' GDR_SCHED_* bits below) return
 * GDR_ERR_BAD_ENUM.
 */
enum { GDR_PRO_L2NORM_QK = 1, GDR_PRO_SIGMOID = 2 };

/*
 * Schedule flags of the bf16 chunked prefill (gdr_chunk_prefill_ex,
 * gdr_chunk_prefill_varlen_ex and their workspace queries; OR-ed with the
 * GDR_PRO_* bits).  With dtype BF16 the prefill has two schedules:
 *   GDR_SCHED_FUSED  one kernel per (head, value slice) that forms each
 *                    chunk's local products itself while it advances the
 *                    state; no workspace.  GDN only.
 *   GDR_SCHED_SPLIT  a chunk-local kernel per (head, chunk) writes each
 *                    chunk's products to the workspace, then a chain kernel
 *                    per (head, value slice) runs the state through them.
 * Neither bit: the default, FUSED for GDN and SPLIT for KDA (the channel
 * gate makes the chunk-local work the expensive part, which the fused kernel
 * would repeat for every value slice).  Prologue support: GDR_PRO_SIGMOID
 * runs in both schedules; GDR_PRO_L2NORM_QK runs in GDN FUSED and KDA SPLIT
 * (where the kernel that forms the chunk-local products stages q and k
 * itself) and returns GDR_ERR_UNSUPPORTED with GDN SPLIT.  Both bits set is
 * GDR_ERR_BAD_ENUM; GDR_SCHED_FUSED with KDA, or either bit with dtype F32
 * (one schedule), is GDR_ERR_UNSUPPORTED.  The decode calls take no schedule
 * bits (GDR_ERR_BAD_ENUM).
 */
enum { GDR_SCHED_FUSED = 4, GDR_SCHED_SPLIT = 8 };

/*
 * gdr_decode_step with an input prologue (flags: GDR_PRO_*): the same step
 * on normalised q, k and sigmoid gates.  flags == 0 is gdr_decode_step
 * exactly (the same kernel and arithmetic).
 */
int gdr_decode_step_ex(int gate, int dtype, int flags, int B, int H, int dk, int dv, float scale,
                       const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta,
                       float* state, void* o, void* stream);

/*
 * T consecutive decode steps per head in one call, the verify step of
 * speculative decoding (§2.D of the pages runs an all-GDN draft whose tokens
 * the target then checks): the T draft tokens go through the recurrence in
 * order, and the state after every token can be kept so that the caller can
 * roll back to any accepted prefix.
 *
 *   q, k    [B, T, H, dk]   dtype        v, o   [B, T, H, dv]   dtype
 *   alpha   [B, T, H] (GDN) or [B, T, H, dk] (KDA), fp32
 *   beta    [B, T, H], fp32
 *   state   [B, H, dk, dv], fp32, read as S_0 and overwritten with S_T
 *   states  [B, T, H, dk, dv], fp32, or NULL: receives S_t, the state after
 *           token t (t = 1 .. T at index t - 1); accepting the first a
 *           tokens means continuing from states[:, a - 1]
 *
 * o_t and every S_t are exactly what T calls of gdr_decode_step would give
 * (same arithmetic, same order); the state is read and written once.
 * 0 <= T <= 64 (longer runs belong to gdr_chunk_prefill; larger T returns
 * GDR_ERR_UNSUPPORTED); T == 0 is a no-op.  o and states may not overlap any
 * input, and states may not overlap state (GDR_ERR_ALIAS).  Returns a GDR_*
 * status.
 */
int gdr_decode_multi(int gate, int dtype, int B, int T, int H, int dk, int dv, float scale,
                     const void* q, const void* k, const void* v,
                     const float* alpha, const float* beta,
                     float* state, void* o, float* states, void* stream);

/*
 * gdr_decode_multi with an input prologue (flags: GDR_PRO_*), applied to
 * every token.  flags == 0 is gdr_decode_multi exactly.
 */
int gdr_decode_multi_ex(int gate, int dtype, int flags, int B, int T, int H, int dk, int dv,
                        float scale, const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta,
                        float* state, void* o, float* states, void* stream);

/*
 * Chunked prefill of T tokens for B x H independent heads (the prompt pass
 * of the same recurrence), in chunks of `chunk` = 64 tokens; T need not be a
 * multiple of the chunk.
 *
 *   q, k      [B, T, H, dk]   dtype     v, o   [B, T, H, dv]   dtype
 *   alpha     [B, T, H] (GDN) or [B, T, H, dk] (KDA), fp32
 *   beta      [B, T, H], fp32
 *   state_in  [B, H, dk, dv] fp32, or NULL for a zero initial state
 *   state_out [B, H, dk, dv] fp32, receives S_T; may equal state_in (in
 *             place) but may not partially overlap it
 *   workspace device scratch of at least
 *             gdr_chunk_prefill_workspace_bytes(...) bytes (NULL if that is 0)
 *
 * T == 0 copies state_in (or zeros) to state_out.  With dtype BF16 the
 * contractions run on bf16 matrix cores with fp32 accumulation and an fp32
 * state; with dtype F32 every operation is fp32.  Any gate in [0, 1] is
 * valid.  Gates near zero are raised to a floor per token (and channel):
 * KDA with BF16 to 2^-15, which changes a state or output by at most 2^-15
 * of the state's magnitude, below the bf16 rounding of the operands; GDN
 * with BF16 to e^-80 and the F32 path to e^-40 (no visible change).
 * Returns a GDR_* status.
 */
int gdr_chunk_prefill(int gate, int dtype, int B, int T, int H, int dk, int dv, int chunk,
                      float scale,
                      const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta,
                      const float* state_in, float* state_out, void* o,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace gdr_chunk_prefill needs for these arguments (0 when the
 * arguments are invalid or no scratch is needed). */
size_t gdr_chunk_prefill_workspace_bytes(int gate, int dtype, int B, int T, int H,
                                         int dk, int dv, int chunk);

/* Bytes of workspace gdr_chunk_prefill_ex needs with these flags (0 when the
 * arguments or flags are invalid, or no scratch is needed). */
size_t gdr_chunk_prefill_workspace_bytes_ex(int gate, int dtype, int flags, int B, int T, int H,
                                            int dk, int dv, int chunk);

/*
 * gdr_chunk_prefill with an input prologue and a schedule choice (flags:
 * GDR_PRO_* | GDR_SCHED_*), taking a workspace of at least
 * gdr_chunk_prefill_workspace_bytes_ex(..., flags, ...) bytes.  flags == 0
 * is gdr_chunk_prefill exactly.  Both prologue flags run in the fp32 path;
 * the bf16 schedules support them as listed with GDR_SCHED_*.
 */
int gdr_chunk_prefill_ex(int gate, int dtype, int flags, int B, int T, int H, int dk, int dv,
                         int chunk, float scale,
                         const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta,
                         const float* state_in, float* state_out, void* o,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdr_chunk_prefill_ex without a workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, flags, support and results as
 * gdr_chunk_prefill_ex (bitwise: the same kernels and arithmetic).  The split
 * schedule's chunk images go to a fixed scratch buffer of 96 MiB that the
 * library holds as a device array, one per GPU: it is set up on the first
 * call on a device (the address lookup loads it there) and kept until the
 * process ends; the call itself allocates and frees nothing.  Ranges of
 * chunks are sized so one range's images fit the buffer; a problem whose
 * single chunk of all B * H heads does not fit (B * H * 68 KiB > 96 MiB for
 * KDA at dk = 128, i.e. more than 1445 heads) returns GDR_ERR_SCRATCH before
 * any device work.  Every call on a GPU shares that GPU's buffer, so calls
 * that overlap in time on one GPU (on different streams, or from different
 * host threads) race; calls ordered on one stream do not.  Nothing in the
 * buffer needs to start at zero (each range writes its images before reading
 * them).  The stream's device (the current device for the null stream) must
 * be one of the first 64.  Returns a GDR_* status.
 */
int gdr_chunk_prefill_noalloc(int gate, int dtype, int flags, int B, int T, int H, int dk, int dv,
                              int chunk, float scale, const void* q, const void* k, const void* v,
                              const float* alpha, const float* beta, const float* state_in,
                              float* state_out, void* o, void* stream);

/*
 * Chunked prefill of N packed variable-length sequences whose states live in
 * a pool of state rows (the call a serving engine makes for a batch of
 * prompts of different lengths; the pages' §2.D serves the mixers through
 * such an engine).  Sequence n holds tokens cu_seqlens[n] .. cu_seqlens[n+1]-1
 * of the packed token tensors; its initial state is row state_slots[n] of
 * `states` (or zeros where has_state[n] == 0), and its final state is written
 * back to the same row.  The same kernels as gdr_chunk_prefill run every
 * sequence independently.
 *
 *   q, k         [total_T, H, dk]   dtype    v, o   [total_T, H, dv]   dtype
 *   alpha        [total_T, H] (GDN) or [total_T, H, dk] (KDA), fp32
 *   beta         [total_T, H], fp32
 *   cu_seqlens   [N + 1] int32, DEVICE: non-decreasing token offsets
 *   state_slots  [N] int32, DEVICE: distinct rows of `states`
 *   has_state    [N] int32, DEVICE, or NULL (every sequence reads its row)
 *   states       [n_slots, H, dk, dv] fp32, DEVICE, read and written in place
 *   max_T        an upper bound of every sequence length (sizes the launch
 *                and the workspace, gdr_chunk_prefill_varlen_workspace_bytes)
 *
 * The offsets and slots are device data the host does not read: a sequence
 * whose offsets are out of order, longer than max_T or beyond total_T, or
 * whose slot is outside [0, n_slots), is skipped (nothing of it is written);
 * a sequence of length 0 leaves its row untouched.  Two sequences with the
 * same slot race.  Returns a GDR_* status.
 */
int gdr_chunk_prefill_varlen(int gate, int dtype, int N, int total_T, int max_T, int H, int dk,
                             int dv, int chunk, float scale,
                             const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta,
                             const int* cu_seqlens, const int* state_slots, const int* has_state,
                             float* states, int n_slots, void* o,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdr_chunk_prefill_varlen with an input prologue and a schedule choice
 * (flags: GDR_PRO_* | GDR_SCHED_*), with the same support as
 * gdr_chunk_prefill_ex and a workspace of at least
 * gdr_chunk_prefill_varlen_workspace_bytes_ex(..., flags, ...) bytes.
 * flags == 0 is gdr_chunk_prefill_varlen exactly.
 */
int gdr_chunk_prefill_varlen_ex(int gate, int dtype, int flags, int N, int total_T, int max_T,
                                int H, int dk, int dv, int chunk, float scale,
                                const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta,
                                const int* cu_seqlens, const int* state_slots,
                                const int* has_state, float* states, int n_slots, void* o,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace gdr_chunk_prefill_varlen needs (0 when the arguments are
 * invalid or no scratch is needed). */
size_t gdr_chunk_prefill_varlen_workspace_bytes(int gate, int dtype, int N, int max_T, int H,
                                                int dk, int dv, int chunk);

/* Bytes of workspace gdr_chunk_prefill_varlen_ex needs with these flags (0
 * when the arguments or flags are invalid, or no scratch is needed). */
size_t gdr_chunk_prefill_varlen_workspace_bytes_ex(int gate, int dtype, int flags, int N,
                                                   int max_T, int H, int dk, int dv, int chunk);

/*
 * Backward pass of the chunked prefill (the training step of the mixers; the
 * pages' §2.B trains the supernet's mixers in its distillation stages):
 * gradients of L = sum(grad_o * o) + sum(grad_state_out * S_T) with respect
 * to every input of gdr_chunk_prefill, same shapes and layouts.
 *
 *   inputs     q, k, v, alpha, beta, state_in (NULL = zeros): as given to
 *              the forward (alpha, beta in linear space)
 *   grad_o     [B, T, H, dv]    dtype
 *   grad_state_out [B, H, dk, dv] fp32, or NULL (S_T unused by the loss)
 *   grad_q, grad_k [B, T, H, dk] dtype;  grad_v [B, T, H, dv] dtype
 *   grad_alpha [B, T, H] (GDN) or [B, T, H, dk] (KDA) fp32
 *   grad_beta  [B, T, H] fp32
 *   grad_state_in [B, H, dk, dv] fp32, or NULL (not wanted)
 *   workspace  device scratch: gdr_chunk_backward_workspace_bytes runs the
 *              sequence in one pass, down to
 *              gdr_chunk_backward_workspace_bytes_ranged(..., 1) it runs in
 *              chunk ranges (below); less is GDR_ERR_WORKSPACE
 *
 * Every product runs in fp32 (bf16 inputs are widened, bf16 gradients rounded
 * to nearest even).  The gate enters through log(alpha), floored at -40 per
 * token as in the fp32 forward; where the floor is active (alpha <= e^-40,
 * alpha = 0 included) grad_alpha is formed from the terms that carry alpha
 * as a factor, i.e. its value at alpha = 0 up to terms of order e^-40.
 * Every sum runs in a fixed order: repeated calls give identical gradients.
 * T == 0 copies grad_state_out (or zeros) to grad_state_in.  Outputs may not
 * overlap inputs.  B * H * ceil(T / 64) and ceil(B * H / 8) * 8 * dv / 16
 * must stay below 2^22 (1024-thread workgroups per chunk and head, and per 16
 * value columns of each head), else GDR_ERR_BAD_SHAPE.  Returns a GDR_*
 * status.
 */
int gdr_chunk_backward(int gate, int dtype, int B, int T, int H, int dk, int dv, int chunk,
                       float scale,
                       const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, const float* state_in,
                       const void* grad_o, const float* grad_state_out,
                       void* grad_q, void* grad_k, void* grad_v,
                       float* grad_alpha, float* grad_beta, float* grad_state_in,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace with which gdr_chunk_backward runs the whole sequence
 * at once (0 when the arguments are invalid). */
size_t gdr_chunk_backward_workspace_bytes(int gate, int dtype, int B, int T, int H, int dk,
                                          int dv, int chunk);

/* Bytes of workspace with which gdr_chunk_backward runs the sequence in
 * ranges of range_chunks chunks of 64 tokens (0 when the arguments are
 * invalid or range_chunks < 1; the whole-sequence size when range_chunks
 * covers the sequence).  A range holds every head's chunk images, states and
 * per-token terms of its chunks; the rest is one state per range start and
 * one state gradient.  gdr_chunk_backward accepts any workspace of at least
 * the one-chunk size: it takes the widest ranges that fit.  In ranges it
 * runs a forward pass that keeps only each range's start state, then the
 * ranges from the last, each from its start state (the chunk-local forward
 * work of every range but the last runs twice); the gradients are bitwise
 * the same as in one pass. */
size_t gdr_chunk_backward_workspace_bytes_ranged(int gate, int dtype, int B, int T, int H, int dk,
                                                 int dv, int chunk, int range_chunks);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* gdr_status_string(int status);

/* GDR_ABI_VERSION of the loaded library. */
int gdr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
