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
// scale their outputs; log2(alpha) is floored at -115.4 (alpha ~ e^-80), so
// alpha == 0 is legal.  KDA: the decay differs per channel, so it has to sit
// inside the operands.  The state-side operands carry factors <= 1 only:
// Khat_t = k_t 2^G_t, Qhat_t = q_t 2^G_t, Ktil_t = k_t 2^(G_end - G_t).  A and
// P factor every pair through the middle of the 16-token block of row t,
// m_r = G at token 16 r + 7 of the chunk:
//     2^(G_t - G_j) = 2^(G_t - m_r) 2^(m_r - G_j),
// with left rows k_t 2^(G_t - m_r) (q_t for P) and, per row block r, right
// rows k_j 2^(m_r - G_j) for every j up to the end of block r.  alpha is
// raised to at least 2^-15 per token and channel, so a factor is at most
// 2^(15 * 8) = 2^120 (t or j at most 8 tokens from the middle of its block)
// and nothing overflows for any gate; for j before block r the right factor
// is <= 1, and where it underflows the exact product is below 2^-21.  The
// floor changes each step's decay by at most 2^-15 of the state (alpha = 0
// forgets all but 3e-5 of it), below the bf16 rounding of the operands.
//
// Mapping.  One workgroup per (b, h, slice of 16*NSW value columns); the value
// columns of S are independent, so the slices of a head run on different CUs
// (their block ids are congruent mod 8: one XCD, shared L2).  Waves 0..3 are
// "prep" waves, waves 4.. are "serial" waves owning 16 value columns each.
// GDN (kFused), one workgroup barrier per step: in step i the prep waves gate
// chunk i+2 and form A, P and the D_r^{-1} of chunk i+1 while the serial waves
// compute Khat S, X, U, O and the new S of chunk i, so LDS holds three sets
// of gated operands and two sets of tiles.  KDA runs the same prep work once
// per (head, chunk) in kPrep and the serial work in kChain (below).  The
// serial chain keeps S, X and U in
// MFMA registers: an fp32 accumulator tile holds rows 4g..4g+3 of column l%16
// in lane l (g = l/16), so two row tiles together are the B operand of a
// K=32 step whose k order is {4g..4g+3, 16+4g..16+4g+3}; the LDS operand of
// that step is read in the same k order, which keeps every product exact
// without any register shuffle.
#include <algorithm>
#include <numeric>
#include <type_traits>

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

// One kernel body, three launch modes:
//   kFused  one workgroup per (b, h, value slice); prep waves form chunk i+1
//           in LDS while the serial waves advance the state through chunk i;
//   kPrep   one workgroup per (b, h, chunk): only the prep work, writing the
//           chunk's LDS buffer image (gated operands, A, P, D_r^{-1}, gates)
//           to a workspace;
//   kChain  one workgroup per (b, h, value slice): a loader wave copies the
//           images into two LDS buffers (direct global-to-LDS loads) while the
//           serial waves run the state recurrence.
// kPrep + kChain do the chunk-local work once per (head, chunk) instead of
// once per value slice, and run it at full occupancy.
enum : int { kFused = 0, kPrep = 1, kChain = 2 };
constexpr float kLog2Floor = -115.4f;  // GDN: log2(alpha) floor, alpha ~ e^-80
constexpr float kKdaMinGate = 3.0517578125e-05f;  // KDA: alpha floor 2^-15 (factors within 2^+-120)
constexpr int kRR = 160;  // KDA right-operand rows: block r keeps rows 0 .. 16 r + 15 (16 + 32 + 48 + 64)
__device__ __forceinline__ constexpr int rr_row0(int r) { return 8 * r * (r + 1); }  // first row of block r's set
// KDA chunk-local rows in LDS (left rows, right rows): the 16-byte unit j of
// row R sits at unit j ^ ((R / 8) mod U) (U units per row).  A gating store
// writes 16 rows four apart at one unit, which would otherwise meet on two
// bank groups; the matrix-core reads apply the same map.
template <int U>
__device__ __forceinline__ int kswz(int row, int unit) { return unit ^ ((row >> 3) & (U - 1)); }

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
// Channel-permuted rows: channel 16 h + 4 g + i of each 32-channel group sits
// at position 8 g + 4 h + i, so the k order {4g..4g+3, 16+4g..16+4g+3} of a
// fragment is 8 contiguous elements (one 16-byte read).
__device__ __forceinline__ constexpr int perm_pos(int c) {
    return (c & ~31) + 8 * ((c >> 2) & 3) + 4 * ((c >> 4) & 1) + (c & 3);
}
__device__ __forceinline__ void st4(bf16_t* p, const f32x4& x) {
    *reinterpret_cast<uint2*>(p) = __builtin_bit_cast(uint2, cvt4(x));
}
__device__ __forceinline__ uint32_t bf_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
// Hardware 2^x and log2 (v_exp_f32 / v_log_f32).  Every exponent here is a
// difference of cumulative log-gates bounded by the chunk's total decay, so
// the plain instructions suffice (results below 2^-126 may flush to zero,
// which is the intended limit of a vanishing decay).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
// 16-bit element e (0..7) of eight packed bf16
__device__ __forceinline__ uint32_t bf16_half(const uint4& w, int e) {
    const uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
    return (e & 1) ? (x >> 16) : (x & 0xffffu);
}
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Input prologue on eight packed bf16: sum of squares, and the values scaled
// by s and rounded to bf16 again.
__device__ __forceinline__ float sumsq8(const uint4& w) {
    float a = bf_lo(w.x) * bf_lo(w.x) + bf_hi(w.x) * bf_hi(w.x);
    float b = bf_lo(w.y) * bf_lo(w.y) + bf_hi(w.y) * bf_hi(w.y);
    a += bf_lo(w.z) * bf_lo(w.z) + bf_hi(w.z) * bf_hi(w.z);
    b += bf_lo(w.w) * bf_lo(w.w) + bf_hi(w.w) * bf_hi(w.w);
    return a + b;
}
__device__ __forceinline__ uint4 scale8(const uint4& w, float s) {
    auto sc = [&](uint32_t x) {
        return static_cast<uint32_t>(bf_bits(bf_lo(x) * s)) | (static_cast<uint32_t>(bf_bits(bf_hi(x) * s)) << 16);
    };
    return make_uint4(sc(w.x), sc(w.y), sc(w.z), sc(w.w));
}
// Sum over each group of N adjacent lanes (N = 2, 4, 8, 16), by DPP moves:
// quad permutations, then the half-row and row mirrors.  Every lane of a
// group ends with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Value of lane N of this lane's DPP row (row_share).
template <int N>
__device__ __forceinline__ float row_share(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + N, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float lane_group_sum(float x) {
    x += dpp_f<0xB1>(x);                         // quad_perm [1, 0, 3, 2]
    if constexpr (N >= 4) x += dpp_f<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    if constexpr (N >= 8) x += dpp_f<0x141>(x);  // row_half_mirror
    if constexpr (N >= 16) x += dpp_f<0x140>(x); // row_mirror
    return x;
}

// Raw buffer access (SGPR base and range, 32-bit lane offsets).  Loads beyond
// the range return zero and stores beyond it are dropped, so the rows past the
// end of a ragged chunk need neither clamped addresses nor branches (and the
// memory-counter waits stay exact).
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr uint32_t kOOB = 0x80000000u;  // a lane offset past every range used here
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

template <int DK, int NSW, bool KDA>
struct Layout {
    static constexpr int DKP = DK < 32 ? 32 : DK;  // contraction pad (dk = 16)
    // pitch of [token][channel] tiles (bf16).  KDA reads row fragments as
    // two 8-byte pieces (conflict-free at DKP + 8); GDN reads them as one
    // 16-byte piece, and 16-byte reads of lanes 8b..8b+7 share an LDS cycle
    // with lanes 8(b^7)..: a pitch of DKP + 16 puts rows r and r + 8 on
    // disjoint banks (and halves the conflicts of the transposing reads).
    static constexpr int PK = DKP + (KDA ? 8 : 16);
    static constexpr int PT = kC + 4;              // pitch of [channel][token] tiles (bf16)
    static constexpr int PD = 16 + 8;              // pitch of packed 16x16 tiles (bf16)
    static constexpr int TILE = 16 * PD * 2;       // bytes of one packed tile
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
    static constexpr int BUF = ((oGend + DK * 4) + 15) / 16 * 16;
    static constexpr int IMG = (BUF + 1023) / 1024 * 1024;  // image stride (1 KB per copy instruction)
    // prep-private
    static constexpr int oKc = 2 * BUF;                   // KDA Kcheck [64][PK]
    static constexpr int oG = oKc + (KDA ? kC * PK * 2 : 0);  // GDN G_t [64]
    static constexpr int PS = 20;                         // pitch of the fp32 scratch tiles
    static constexpr int oScr = oG + kC * 4;              // fp32 diagonal tiles [4][16][PS]
    static constexpr int bytes = oScr + kPrepWaves * 16 * PS * 4;
    static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
    // kPrep: only what the A/P products and the inverses read stays in LDS.
    // KDA: pKh / pQh hold the left rows k_t 2^(G_t - m_r), q_t 2^(G_t - m_r)
    // and pKc the right rows of the four row blocks (kRR rows; the image gets
    // Khat and Qhat instead).
    static constexpr int pKh = 0;
    static constexpr int pQh = kC * PK * 2;
    static constexpr int pBeta = 2 * kC * PK * 2;
    static constexpr int pKc = pBeta + kC * 4;
    static constexpr int pG = pKc + (KDA ? kRR * PK * 2 : 0);
    static constexpr int pScr = pG + kC * 4;
    static constexpr int pA = pScr + kPrepWaves * 16 * PS * 4;  // -A_rk tiles (6)
    static constexpr int pD = pA + 6 * TILE;                     // D_r^{-1} tiles (4)
    static constexpr int pT = pD + 4 * TILE;                     // T_rk tiles, k < r (6)
    static constexpr int pNrm = pT + 6 * TILE;  // KDA prologue: per-wave sums of squares [4][64][2]
    static constexpr int pBytes = pNrm + (KDA ? kPrepWaves * kC * 2 * 4 : 0);
    // GDN kFused, one barrier per chunk: three operand sets (Khat, Qhat and
    // the per-token scalars: prep gates chunk i+2 while the serial waves read
    // chunk i) and two tile sets (P, -A, D_r^{-1}: prep forms chunk i+1).
    // The serial waves read K^T through transposing LDS reads of Khat (GDN
    // contracts raw k), so there is no K^T copy.
    static constexpr int uKh = 0;
    static constexpr int uQh = kC * PK * 2;
    static constexpr int uBeta = 2 * kC * PK * 2;
    static constexpr int uEg = uBeta + kC * 4;
    static constexpr int uEk = uEg + kC * 4;
    static constexpr int uG = uEk + kC * 4;
    static constexpr int uGend = uG + kC * 4;
    // factors of 2^(G_t - G_j) for t, j in different 16-token blocks:
    // 2^(G_t - Gb_{b(t)-1}) 2^(Gb_{b(t)-1} - Gb_{b(j)}) 2^(Gb_{b(j)} - G_j),
    // Gb_b = G at the last token of block b (each factor <= 1)
    static constexpr int uU = uGend + 16;   // [64] row factors
    static constexpr int uW = uU + kC * 4;  // [64] column factors
    static constexpr int uC = uW + kC * 4;  // [4][4] block-pair factors (r > c)
    static constexpr int uEs = uC + 64;     // [64] scale 2^G_t (the output's row factor)
    static constexpr int OPS = (uEs + kC * 4 + 15) / 16 * 16;  // operand set stride
    static constexpr int uTB = 3 * OPS;                      // first tile set
    static constexpr int TLS = 20 * TILE;                    // tile set: P (10), -A (6), D (4)
    static constexpr int uScr = uTB + 2 * TLS;
    static constexpr int ubytes = uScr + kPrepWaves * 16 * PS * 4;
    static_assert(ubytes <= 160 * 1024, "LDS budget exceeded");
    // kChain: two image buffers
    static constexpr int cBytes = 2 * IMG;
    static_assert(cBytes <= 160 * 1024, "LDS budget exceeded");
    // GDN split: the image holds only the tiles and gate factors (the BUF
    // range from oP on); the chain stages raw k and q rows itself, in rows of
    // DKP bf16 whose 16-byte units are permuted by a row-dependent XOR (swz)
    // so that 16 rows read at one column hit distinct LDS banks.
    static constexpr int TIMG = ((BUF - oP) + 15) / 16 * 16;
    static constexpr int lK = 0;
    static constexpr int lQ = kC * DKP * 2;
    static constexpr int lT = 2 * kC * DKP * 2;
    static constexpr int lBUF = ((lT + TIMG) + 15) / 16 * 16;
    static constexpr int lBytes = 2 * lBUF;
    static_assert(lBytes <= 160 * 1024, "LDS budget exceeded");
    static constexpr int U = DKP / 8;  // 16-byte units per staged row
    // Per serial wave, a 2 KiB tile of the chunk's v (64 rows x 16 columns),
    // after the mode's other LDS, when it fits: v then arrives with two
    // 16-byte loads per lane and is transposed by an LDS read.
    static constexpr int VST = kC * 16 * 2;
    // LDS of the fused mode before the v tiles (GDN: the one-barrier layout)
    static constexpr int fBytes(bool kda) { return kda ? bytes : ubytes; }
    static constexpr bool vstage(int mode, bool kda) {
        return (mode == 0 ? fBytes(kda) : mode == 2 ? (kda ? cBytes : lBytes) : 0) + NSW * VST <= 160 * 1024 &&
               mode != 1;
    }
    static constexpr int vbase(int mode, bool kda) { return mode == 0 ? fBytes(kda) : kda ? cBytes : lBytes; }
};
// Unit permutation of staged row r (see Layout): position = unit ^ swz(r).
template <int U>
__device__ __forceinline__ int swz(int r) { return ((2 * r) | ((r >> 3) & 1)) & (U - 1); }

// Chain kernel: waves that copy chunk images into LDS (they fill the SIMDs
// the serial waves leave free; the copies of one chunk are split among them).
// (KDA: the image holds everything; GDN ("lite"): the serial waves stage
// the raw rows and the small tile image through their registers instead.)
template <int NSW, bool KDA>
constexpr int load_waves() { return !KDA ? 0 : NSW >= 4 ? 1 : 4 - NSW; }
template <int NSW, bool KDA, int MODE>
constexpr int block_threads() {
    return 64 * (MODE == kPrep ? kPrepWaves
                 : MODE == kChain ? load_waves<NSW, KDA>() + NSW : kPrepWaves + NSW);
}
// Waves per SIMD the register allocation is sized for: a chain workgroup of
// at most four waves has a SIMD per wave (its LDS keeps it alone on the CU),
// so each wave may use the whole register file.
template <int NSW, bool KDA, int MODE>
constexpr int waves_per_simd() {
    // (KDA's chunk-local kernel: its LDS keeps it at one workgroup per CU,
    // one wave per SIMD, so it may use the whole register file too)
    return (MODE == kChain && load_waves<NSW, KDA>() + NSW <= 4) || (MODE == kPrep && KDA) ? 1 : 2;
}

__device__ __forceinline__ int ptile(int rt, int ct) { return rt * (rt + 1) / 2 + ct; }  // ct <= rt
__device__ __forceinline__ int atile(int rt, int ct) { return rt * (rt - 1) / 2 + ct; }  // ct < rt
// A compile-time list of A/P tiles: code = 16 isP + 4 row + column (column <= row).
template <int... T>
struct Tiles {
    static constexpr int n = sizeof...(T);
    static constexpr int code[n] = {T...};
};
constexpr int tA(int r, int c) { return 4 * r + c; }
constexpr int tP(int r, int c) { return 16 + 4 * r + c; }

template <int DK, int NSW, bool KDA, int MODE>
__global__ __launch_bounds__((block_threads<NSW, KDA, MODE>()))
__attribute__((amdgpu_waves_per_eu(waves_per_simd<NSW, KDA, MODE>(), waves_per_simd<NSW, KDA, MODE>()))) void prefill_bf16_kernel(
    int B, int Tmax, int H, int DV, int NS, float scale, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, const float* __restrict__ state_in,
    float* __restrict__ state_out, bf16_t* __restrict__ o, unsigned char* __restrict__ img,
    int c0, int c1, Opts vl) {
    // Chunks c0 .. c1-1 of every sequence (the split schedule runs a long
    // sequence as consecutive ranges, chaining the state through state_in /
    // state_out, so that one range's images stay cache resident).  Packed
    // variable-length sequences (vl.cu) end at their own chunk count.
    using L = Layout<DK, NSW, KDA>;
    constexpr int DVS = 16 * NSW;
    constexpr int NRT = DK / 16;          // 16-row tiles of S
    constexpr int NKS = L::DKP / 32;      // K=32 steps over dk

    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int lr = lane & 15, lg = lane >> 4;

    const int BH = B * H;
    int bh, slice = 0, g = 0;
    if constexpr (MODE == kPrep) {
        g = static_cast<int>(blockIdx.x) / BH;  // NS = chunks per workgroup
        bh = static_cast<int>(blockIdx.x) - g * BH;
    } else {
        const int grp = blockIdx.x / (8 * NS);
        const int rem = blockIdx.x - grp * 8 * NS;
        bh = grp * 8 + (rem & 7);
        slice = rem >> 3;
        if (bh >= BH) return;  // whole block exits before any barrier
    }
    const int b = bh / H, h = bh - b * H;
    // This sequence: its length, first token row, state row, and whether it
    // reads an initial state (later ranges of the split schedule always read
    // the state carried from the previous range).
    int T = Tmax;
    size_t tseq = static_cast<size_t>(b) * Tmax;
    int srow = bh;
    bool init = state_in != nullptr;
    if (vl.cu) {
        const int s0 = vl.cu[b], s1 = vl.cu[b + 1];
        if (s0 < 0 || s1 < s0 || s1 - s0 > Tmax || s1 > vl.total) return;  // whole block, no barrier yet
        T = s1 - s0;
        tseq = static_cast<size_t>(s0);
        if (T == 0) return;  // an empty sequence leaves its state row untouched
    }
    if (vl.slot) {
        const int r = vl.slot[b];
        if (r < 0 || r >= vl.n_slots) return;
        srow = r * H + h;
    }
    if (vl.has && c0 == 0 && vl.has[b] == 0) init = false;
    const int nch = min(c1, (T + kC - 1) / kC);  // chunks run by this launch: c0 .. nch-1
    int pc = 0, pc_end = 0;                       // kPrep: chunks pc .. pc_end-1 of one head
    if constexpr (MODE == kPrep) {
        pc = c0 + g * NS;
        pc_end = min(nch, pc + NS);
    }
    constexpr int kLoad = load_waves<NSW, KDA>();
    constexpr bool LITE = !KDA && MODE != kFused;  // GDN split
    constexpr int kLead = MODE == kChain ? kLoad : kPrepWaves;  // waves before the serial ones
    const bool prep = MODE == kPrep || (MODE == kFused && wave < kPrepWaves);

    // Chunk buffers: kFused / kChain keep two in LDS (chunk c uses c & 1).
    constexpr int kStride = MODE == kChain ? (LITE ? L::lBUF : L::IMG) : L::BUF;
    // LITE chain buffers keep the tile image at lT (image offset = BUF offset - oP)
    constexpr int kTileShift = (LITE && MODE == kChain) ? L::lT - L::oP : 0;
    // GDN kFused: one barrier per chunk (three operand sets, two tile sets);
    // the buffer offsets (BUF layout) are mapped to the set holding them.
    constexpr bool ONEBAR = MODE == kFused && !KDA;
    auto at = [&](int c, int off) -> unsigned char* {
        if constexpr (ONEBAR) {
            unsigned char* ops = smem + (c % 3) * L::OPS;
            if (off == L::oKh) return ops + L::uKh;
            if (off == L::oQh) return ops + L::uQh;
            if (off == L::oBeta) return ops + L::uBeta;
            if (off == L::oEg) return ops + L::uEg;
            if (off == L::oEk) return ops + L::uEk;
            if (off == L::oGend) return ops + L::uGend;
            return smem + L::uTB + (c & 1) * L::TLS + (off - L::oP);  // P, -A, D_r^{-1}
        } else {
            return smem + (c & 1) * kStride + off + kTileShift;
        }
    };
    auto bfp = [&](int c, int off) { return reinterpret_cast<bf16_t*>(at(c, off)); };
    auto f32p = [&](int c, int off) { return reinterpret_cast<float*>(at(c, off)); };
    // The image of chunk c of this head (kPrep writes it, kChain reads it).
    constexpr int kImg = LITE ? L::TIMG : L::IMG;  // image bytes per (head, chunk)
    auto imgp = [&](int c) { return img + (static_cast<size_t>(bh) * (c1 - c0) + (c - c0)) * kImg; };
    // Where the prep work reads and writes.  kFused: the LDS buffer of the
    // chunk.  kPrep: what the A/P products and the inverses read sits in LDS
    // (and Khat, Qhat, beta are also written to the image); everything else
    // goes to the image only.
    auto prep_lds_b = [&](int c, int off_fused, int off_prep) {
        if constexpr (MODE == kPrep) return reinterpret_cast<bf16_t*>(smem + off_prep);
        else return bfp(c, off_fused);
    };
    auto prep_out_b = [&](int c, int off) {
        if constexpr (MODE == kPrep) return reinterpret_cast<bf16_t*>(imgp(c) + off - (LITE ? L::oP : 0));
        else return bfp(c, off);
    };
    auto prep_out_f = [&](int c, int off) {
        if constexpr (MODE == kPrep) return reinterpret_cast<float*>(imgp(c) + off - (LITE ? L::oP : 0));
        else return f32p(c, off);
    };
    bf16_t* Kc = reinterpret_cast<bf16_t*>(smem + (MODE == kPrep ? L::pKc : L::oKc));  // KDA right rows
    // G_t of the chunk being gated / formed (ONEBAR: one per operand set)
    auto sGp = [&](int c) {
        if constexpr (ONEBAR) return reinterpret_cast<float*>(smem + (c % 3) * L::OPS + L::uG);
        else return reinterpret_cast<float*>(smem + (MODE == kPrep ? L::pG : L::oG));
    };
    float* scr0 = reinterpret_cast<float*>(smem + (MODE == kPrep ? L::pScr : ONEBAR ? L::uScr : L::oScr));

    // KDA chunk-local rows: element position of (row, col) under the unit map
    constexpr bool KSW = KDA && MODE == kPrep;
    auto kpos = [](int row, int col) {
        return KSW ? (kswz<L::DKP / 8>(row, col >> 3) << 3) | (col & 7) : col;
    };
    if constexpr (L::DKP != DK && MODE != kChain) {  // zero the contraction padding
        constexpr int W = L::DKP - DK;
        constexpr int NB = MODE == kPrep ? 1 : ONEBAR ? 3 : 2;
        for (int idx = tid; idx < NB * kC * W; idx += blockDim.x) {
            const int c = idx / (kC * W), r = idx % (kC * W);
            const int t = r / W, col = ONEBAR ? perm_pos(DK + r % W) : kpos(r / W, DK + r % W);
            prep_lds_b(c, L::oKh, L::pKh)[t * L::PK + col] = 0;
            prep_lds_b(c, L::oQh, L::pQh)[t * L::PK + col] = 0;
        }
        if constexpr (KSW) {
            for (int idx = tid; idx < kRR * W; idx += blockDim.x)
                Kc[(idx / W) * L::PK + kpos(idx / W, DK + idx % W)] = 0;
        }
    }
    // kPrep: the same padding in the image of chunk c, which the chain reads
    auto zero_image_pad = [&](int c) {
        if constexpr (L::DKP != DK && MODE == kPrep && !LITE) {
            constexpr int W = L::DKP - DK;
            for (int idx = tid; idx < kC * W; idx += blockDim.x) {
                const int t = idx / W, col = DK + idx % W;
                reinterpret_cast<bf16_t*>(imgp(c) + L::oKh)[t * L::PK + col] = 0;
                reinterpret_cast<bf16_t*>(imgp(c) + L::oQh)[t * L::PK + col] = 0;
            }
        }
    };

    // ================= prep-wave work =================
    // Lane layout for q and k: lane = (channel octet oct, run of 4 tokens
    // tg); loads and LDS writes are 16 bytes (8 channels).
    //  KDA: the 16 lanes of an octet are one DPP row, so each channel's
    //       cumulative log-gate over the chunk is an in-row scan.
    //  GDN: the octets of a row are adjacent lanes (a wave load instruction
    //       reads whole 256-byte rows); the scalar gates of the 64 tokens are
    //       scanned by one wave alone, one token per lane.
    constexpr int OPR = DK / 8;  // octets per row
    const int oct = KDA ? tid >> 4 : tid % OPR;
    const int tg = KDA ? tid & 15 : tid / OPR;
    // DK/8 octets x 16 token runs (GDN kFused, dk = 128: every prep lane)
    const bool gater = (ONEBAR && 2 * DK >= kPrepWaves * 64) || tid < 2 * DK;
    const int c8 = 8 * oct;           // first channel of this lane's octet
    constexpr int NA = KDA ? 32 : 4;  // gate values per lane
    // GDN: the wave that scans the scalar gates (kFused: one that inverts no
    // diagonal block; see the tile lists of prep_ap)
    constexpr int kScanWave = ONEBAR ? 3 : 1;
    struct PrepIn {
        uint4 kr[4], qr[4];
        float a[NA];
        float bt[4];
    };
    const size_t tok0 = tseq * H + h;  // token (b, 0, h)
    auto prep_load = [&](int c, PrepIn& R) {
        // ONEBAR: R was gated this step; the other register set's 10 loads
        // (one step younger) may still be in flight.  Every older load has
        // landed, which the wait states explicitly: otherwise the register
        // reuse below is guarded by waits that also drain the younger set.
        if constexpr (ONEBAR) __builtin_amdgcn_s_waitcnt(0x0F7A);  // vmcnt(10)
        const int t0 = c * kC, nn = min(kC, T - t0);
        const size_t rb = tok0 + static_cast<size_t>(t0) * H;  // row of token t0 (uniform)
        const bf16_t* kb = k + rb * DK;
        const bf16_t* qb = q + rb * DK;
        const float* ab = KDA ? alpha + rb * DK : alpha + rb;
        const float* bb = beta + rb;
        if constexpr (ONEBAR) {
            // range-checked loads: rows past the chunk's end (and every row
            // of a chunk past the sequence's end) read zero
            const uint32_t nr = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(max(nn, 0)));  // uniform
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, nr * H * DK * 2);
            const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, nr * H * DK * 2);
            if (gater) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t off = static_cast<uint32_t>(((4 * tg + u) * H * DK + c8) * 2);
                    R.kr[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
                    R.qr[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
                }
            }
            // gates, token = lane (used by the scan wave; every wave loads
            // them, so every wave has the same 10 loads in flight per set)
            const uint32_t off = static_cast<uint32_t>(lane * H * 4);
            R.a[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(ab, nr * H * 4), off, 0, 0));
            R.bt[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(bb, nr * H * 4), off, 0, 0));
            return;
        }
        if (gater) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int tc = nn == kC ? 4 * tg + u : min(4 * tg + u, nn - 1);
            const unsigned ro = static_cast<unsigned>(tc * H);  // row offset inside the chunk
            R.kr[u] = *reinterpret_cast<const uint4*>(kb + (ro * DK + c8));
            R.qr[u] = *reinterpret_cast<const uint4*>(qb + (ro * DK + c8));
            if constexpr (KDA) {
                const float4 x0 = *reinterpret_cast<const float4*>(ab + (ro * DK + c8));
                const float4 x1 = *reinterpret_cast<const float4*>(ab + (ro * DK + c8 + 4));
                R.a[8 * u + 0] = x0.x; R.a[8 * u + 1] = x0.y; R.a[8 * u + 2] = x0.z; R.a[8 * u + 3] = x0.w;
                R.a[8 * u + 4] = x1.x; R.a[8 * u + 5] = x1.y; R.a[8 * u + 6] = x1.z; R.a[8 * u + 7] = x1.w;
                R.bt[u] = bb[ro];
            }
        }
        }
        if constexpr (!KDA) {
            if (wave == kScanWave) {  // token = lane
                const int tc = nn == kC ? lane : min(lane, nn - 1);
                const unsigned ro = static_cast<unsigned>(tc * H);
                R.a[0] = ab[ro];
                R.bt[0] = bb[ro];
            }
        }
    };
    // inclusive scan over the 16 lanes of a DPP row (row_shr by 1, 2, 4, 8)
    auto row_scan = [](float x) {
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
        return x;
    };
    auto bf_at = [](const uint4& w, int e) {  // element e of 8 packed bf16
        const uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
        return (e & 1) ? bf_hi(x) : bf_lo(x);
    };

    // Gates and gated operands of chunk c into buffer c & 1.
    auto prep_gate = [&](int c, const PrepIn& R) {
        const int n = min(kC, T - c * kC);
        bf16_t* Kh = prep_lds_b(c, L::oKh, L::pKh);
        bf16_t* Qh = prep_lds_b(c, L::oQh, L::pQh);
        bf16_t* Kt = (LITE || ONEBAR) ? nullptr : prep_out_b(c, L::oKt);  // lite image / ONEBAR: no K^T
        float* sBeta = reinterpret_cast<float*>(prep_lds_b(c, L::oBeta, L::pBeta));
        // kPrep: copies of Khat, Qhat and beta for the image
        bf16_t* KhI = reinterpret_cast<bf16_t*>(MODE == kPrep && !LITE ? imgp(c) + L::oKh : nullptr);
        bf16_t* QhI = reinterpret_cast<bf16_t*>(MODE == kPrep && !LITE ? imgp(c) + L::oQh : nullptr);
        // Input prologue.  Sigmoid gates (logits given); inverse norms of the
        // raw q, k rows, nk[u], nq[u] for token 4 tg + u.  GDN: a row is OPR
        // adjacent lanes (a DPP sum).  KDA (chunk-local kernel): a row is the
        // lanes tg, tg+16, tg+32, tg+48 of every wave, so the per-wave sums
        // meet in LDS behind one barrier, which every wave reaches.
        const bool sig = (vl.pro & GDR_PRO_SIGMOID) != 0;
        const bool nrm = (vl.pro & GDR_PRO_L2NORM_QK) != 0;
        float nk[4] = {1.f, 1.f, 1.f, 1.f}, nq[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (KDA && MODE == kPrep) {
            if (nrm) {
                float* part = reinterpret_cast<float*>(smem + L::pNrm);  // [wave][token][k, q]
                float sk[4], sq[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    sk[u] = gater ? sumsq8(R.kr[u]) : 0.f;
                    sq[u] = gater ? sumsq8(R.qr[u]) : 0.f;
                    sk[u] += __shfl_xor(sk[u], 16);
                    sq[u] += __shfl_xor(sq[u], 16);
                    sk[u] += __shfl_xor(sk[u], 32);
                    sq[u] += __shfl_xor(sq[u], 32);
                }
                if (lane < 16) {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        *reinterpret_cast<float2*>(part + 2 * (wave * kC + 4 * tg + u)) = make_float2(sk[u], sq[u]);
                }
                lds_barrier();
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float a = 0.f, bq = 0.f;
#pragma unroll
                    for (int w = 0; w < kPrepWaves; ++w) {
                        const float2 x = *reinterpret_cast<const float2*>(part + 2 * (w * kC + 4 * tg + u));
                        a += x.x;
                        bq += x.y;
                    }
                    nk[u] = inv_norm(a);
                    nq[u] = inv_norm(bq);
                }
            }
        }
        if (KDA && !gater) return;
        // a full chunk (every chunk but a ragged last one) needs no row masks;
        // KDA full chunks without the norm prologue skip the unit factors
        auto body = [&](auto full_tag, auto nrm_tag) {
            constexpr bool FULL = decltype(full_tag)::value;
            constexpr bool NRM = decltype(nrm_tag)::value;  // false: nk = nq = 1
            bool valid[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) valid[u] = FULL || 4 * tg + u < n;
            if (KDA && oct == 0) {
                auto bt = [&](int u) { return valid[u] ? (sig ? sigmoid_f(R.bt[u]) : R.bt[u]) : 0.f; };
                float4 b4;
                b4.x = bt(0); b4.y = bt(1); b4.z = bt(2); b4.w = bt(3);
                *reinterpret_cast<float4*>(sBeta + 4 * tg) = b4;
                if constexpr (MODE == kPrep) *reinterpret_cast<float4*>(prep_out_f(c, L::oBeta) + 4 * tg) = b4;
            }
            uint4 kz[4], qz[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                kz[u] = valid[u] ? R.kr[u] : make_uint4(0, 0, 0, 0);
                qz[u] = valid[u] ? R.qr[u] : make_uint4(0, 0, 0, 0);
            }
            if constexpr (KDA) {
                // Lane = one 4-token group (tokens 4 tg .. 4 tg + 3) of 8
                // channels; the 16 groups of the chunk are one DPP row.
                // Pass 1, per channel: the product of the lane's 4 gates, its
                // log2 scanned across the row (G at each group's end, inc),
                // and the lane's factors from X = inc - log2(product) (G
                // before the group): 2^X, 2^(X - m_b) (b = the lane's block),
                // 2^(G_end - inc) and 2^(m_r - inc) for the blocks r >= b.
                // Pass 2 walks the tokens forward with the running product
                // 2^(G_t - X) (Khat, Qhat, left rows), pass 3 backward with
                // 2^(inc - G_t) (Ktil, right rows).  Every factor lies within
                // 2^+-120 (see the file header).
                const int blk = tg >> 2;
                float ga[NA], cK[8], cD[8], cT[8], cR[4][8];
#pragma unroll
                for (int i = 0; i < NA; ++i)
                    ga[i] = valid[i >> 3] ? fmaxf(sig ? sigmoid_f(R.a[i]) : R.a[i], kKdaMinGate) : 1.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float tot = lg2(ga[e] * ga[8 + e] * ga[16 + e] * ga[24 + e]);
                    const float inc = row_scan(tot);
                    const float X = inc - tot;
                    const float gend = row_share<15>(inc);
                    const float m0 = row_share<1>(inc), m1 = row_share<5>(inc);
                    const float m2 = row_share<9>(inc), m3 = row_share<13>(inc);
                    const float mb = blk == 0 ? m0 : blk == 1 ? m1 : blk == 2 ? m2 : m3;
                    cK[e] = ex2(X);
                    cD[e] = ex2(X - mb);
                    cT[e] = ex2(gend - inc);
                    cR[0][e] = blk == 0 ? ex2(m0 - inc) : 0.f;
                    cR[1][e] = blk <= 1 ? ex2(m1 - inc) : 0.f;
                    cR[2][e] = blk <= 2 ? ex2(m2 - inc) : 0.f;
                    cR[3][e] = ex2(m3 - inc);
                    if (tg == 0) prep_out_f(c, L::oGend)[c8 + e] = ex2(gend);
                }
                float run[8];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int t = 4 * tg + u;
                    bf16x8 kh, qh, dl, dq;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        run[e] = u == 0 ? ga[e] : run[e] * ga[8 * u + e];  // 2^(G_t - X)
                        const float kp = bf_at(kz[u], e) * (NRM ? nk[u] : 1.f) * run[e];
                        const float qp = bf_at(qz[u], e) * (NRM ? nq[u] : 1.f) * run[e];
                        kh[e] = static_cast<__bf16>(kp * cK[e]);
                        qh[e] = static_cast<__bf16>(qp * cK[e]);
                        dl[e] = static_cast<__bf16>(kp * cD[e]);
                        dq[e] = static_cast<__bf16>(qp * cD[e]);
                    }
                    const int pos = kpos(t, c8);
                    *reinterpret_cast<bf16x8*>(Kh + t * L::PK + pos) = dl;
                    *reinterpret_cast<bf16x8*>(Qh + t * L::PK + pos) = dq;
                    *reinterpret_cast<bf16x8*>(KhI + t * L::PK + c8) = kh;
                    *reinterpret_cast<bf16x8*>(QhI + t * L::PK + c8) = qh;
                }
                uint32_t ktw[8][2];
                float rev[8];
#pragma unroll
                for (int u = 3; u >= 0; --u) {
                    const int t = 4 * tg + u;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        bf16x8 rr;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            if (r == 0) rev[e] = u == 3 ? 1.f : rev[e] * ga[8 * (u + 1) + e];  // 2^(inc - G_t)
                            const float ks = bf_at(kz[u], e) * (NRM ? nk[u] : 1.f) * rev[e];
                            if (r == 0) {
                                const uint32_t kt = bf_bits(ks * cT[e]);
                                if (u & 1) ktw[e][u >> 1] = kt << 16;
                                else ktw[e][u >> 1] |= kt;
                            }
                            rr[e] = static_cast<__bf16>(ks * cR[r][e]);
                        }
                        const int row = rr_row0(r) + t;
                        if (r >= blk) *reinterpret_cast<bf16x8*>(Kc + row * L::PK + kpos(row, c8)) = rr;
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *reinterpret_cast<uint2*>(Kt + (c8 + e) * L::PT + 4 * tg) = make_uint2(ktw[e][0], ktw[e][1]);
            } else {
                if (wave == kScanWave) {
                    // scalar gates: token t = lane; inclusive scan of log2 alpha
                    // over the wave (in-row DPP scan, then the row totals,
                    // read into scalar registers)
                    const bool vt = FULL || lane < n;
                    float x = vt ? fmaxf(sig ? log2_sigmoid(R.a[0]) : lg2(R.a[0]), kLog2Floor) : 0.f;
                    x = row_scan(x);
                    auto lane_at = [](float y, int l) {
                        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(y), l));
                    };
                    const float r0 = lane_at(x, 15), r1 = lane_at(x, 31), r2 = lane_at(x, 47);
                    const int row = lane >> 4;
                    x += (row >= 1 ? r0 : 0.f) + (row >= 2 ? r1 : 0.f) + (row >= 3 ? r2 : 0.f);
                    const float end = lane_at(x, 63);
                    if constexpr (ONEBAR) {
                        // block-factored gate products (each factor <= 1)
                        const float gb0 = r0, gb1 = r0 + r1, gb2 = r0 + r1 + r2;
                        auto gb = [&](int bb) { return bb == 0 ? gb0 : bb == 1 ? gb1 : bb == 2 ? gb2 : end; };
                        float* ops = reinterpret_cast<float*>(smem + (c % 3) * L::OPS);
                        ops[L::uU / 4 + lane] = ex2(x - (row == 0 ? 0.f : gb(row - 1)));
                        ops[L::uW / 4 + lane] = ex2(gb(row) - x);
                        if (lane < 16) {
                            const int br = lane >> 2, bc = lane & 3;
                            ops[L::uC / 4 + lane] = br > bc ? ex2(gb(br - 1) - gb(bc)) : 0.f;
                        }
                        ops[L::uEs / 4 + lane] = ex2(x) * scale;
                    }
                    sGp(c)[lane] = x;
                    prep_out_f(c, L::oEg)[lane] = ex2(x);
                    prep_out_f(c, L::oEk)[lane] = ex2(end - x);
                    const float bv = vt ? (sig ? sigmoid_f(R.bt[0]) : R.bt[0]) : 0.f;
                    sBeta[lane] = bv;
                    if constexpr (MODE == kPrep) prep_out_f(c, L::oBeta)[lane] = bv;
                    if (lane == 0) prep_out_f(c, L::oGend)[0] = ex2(end);
                }
                if (!gater) return;
                if (MODE == kFused && nrm) {  // a row is the OPR adjacent lanes of one token run
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        kz[u] = scale8(kz[u], inv_norm(lane_group_sum<OPR>(sumsq8(kz[u]))));
                        qz[u] = scale8(qz[u], inv_norm(lane_group_sum<OPR>(sumsq8(qz[u]))));
                    }
                }
                if constexpr (ONEBAR && DK >= 32) {
                    // channel-permuted rows (see perm_pos).  Octets o and o^2
                    // of a 32-channel group (lanes of one DPP quad) swap one
                    // 8-byte half, after which each lane holds 16 contiguous
                    // bytes of the permuted row: octet 4j + o4 writes
                    // positions 32 j + 16 (o4 & 1) + 8 (o4 >> 1) .. + 7 (the
                    // same 256 bytes per row as unpermuted 16-byte stores)
                    const int o4 = oct & 3;
                    const bool up = o4 >= 2;  // keeps its high half, receives the partner's
                    bf16_t* kr0 = Kh + 32 * (oct >> 2) + 16 * (o4 & 1) + 8 * (o4 >> 1);
                    bf16_t* qr0 = Qh + 32 * (oct >> 2) + 16 * (o4 & 1) + 8 * (o4 >> 1);
                    auto xch = [&](uint32_t x) {  // value of quad lane o4 ^ 2
                        return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0x4E, 0xF, 0xF, false));
                    };
                    auto perm16 = [&](const uint4& w) {
                        const uint32_t s0 = up ? w.x : w.z, s1 = up ? w.y : w.w;  // half sent to the partner
                        const uint32_t r0 = xch(s0), r1 = xch(s1);
                        return up ? make_uint4(r0, r1, w.z, w.w) : make_uint4(w.x, w.y, r0, r1);
                    };
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int t = 4 * tg + u;
                        *reinterpret_cast<uint4*>(kr0 + t * L::PK) = perm16(kz[u]);
                        *reinterpret_cast<uint4*>(qr0 + t * L::PK) = perm16(qz[u]);
                    }
                    return;
                } else if constexpr (ONEBAR) {
                    // dk = 16 (one octet pair per row): the two halves go to
                    // positions p0 and p0 + 8 (p0 = perm_pos of the octet)
                    const int p0 = perm_pos(c8);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int t = 4 * tg + u;
                        *reinterpret_cast<uint2*>(Kh + t * L::PK + p0) = make_uint2(kz[u].x, kz[u].y);
                        *reinterpret_cast<uint2*>(Kh + t * L::PK + p0 + 8) = make_uint2(kz[u].z, kz[u].w);
                        *reinterpret_cast<uint2*>(Qh + t * L::PK + p0) = make_uint2(qz[u].x, qz[u].y);
                        *reinterpret_cast<uint2*>(Qh + t * L::PK + p0 + 8) = make_uint2(qz[u].z, qz[u].w);
                    }
                    return;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int t = 4 * tg + u;
                    *reinterpret_cast<uint4*>(Kh + t * L::PK + c8) = kz[u];
                    *reinterpret_cast<uint4*>(Qh + t * L::PK + c8) = qz[u];
                    if constexpr (MODE == kPrep && !LITE) {
                        *reinterpret_cast<uint4*>(KhI + t * L::PK + c8) = kz[u];
                        *reinterpret_cast<uint4*>(QhI + t * L::PK + c8) = qz[u];
                    }
                }
                // K^T: channel c8 + e, tokens 4 tg .. 4 tg + 3.  The 16 lanes
                // of a token run hold 16 octets, whose rows lie 8 apart: with
                // the row pitch they would meet on a quarter of the banks.  A
                // lane therefore walks its octet from a lane-dependent start
                // (rot, distinct across the 16 octets modulo 8 together with
                // the octet's parity) after rotating its 8 channels by rot.
                if constexpr (!LITE && !ONEBAR) {
                    const int rot = (oct + (oct >> 3)) & 7;
                    const uint32_t sh = static_cast<uint32_t>(rot & 1) * 16u;
                    uint4 rz[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t d[4] = {kz[u].x, kz[u].y, kz[u].z, kz[u].w};
                        uint32_t t1[4], t2[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) t1[j] = (rot & 2) ? d[(j + 1) & 3] : d[j];
#pragma unroll
                        for (int j = 0; j < 4; ++j) t2[j] = (rot & 4) ? t1[(j + 2) & 3] : t1[j];
                        // halves: rz half e = kz half (e + rot) & 7
                        rz[u] = make_uint4(__builtin_amdgcn_alignbit(t2[1], t2[0], sh),
                                           __builtin_amdgcn_alignbit(t2[2], t2[1], sh),
                                           __builtin_amdgcn_alignbit(t2[3], t2[2], sh),
                                           __builtin_amdgcn_alignbit(t2[0], t2[3], sh));
                    }
                    bf16_t* ktl = Kt + c8 * L::PT + 4 * tg;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t x0 = bf16_half(rz[0], e), x1 = bf16_half(rz[1], e);
                        const uint32_t x2 = bf16_half(rz[2], e), x3 = bf16_half(rz[3], e);
                        *reinterpret_cast<uint2*>(ktl + ((e + rot) & 7) * L::PT) =
                            make_uint2(x0 | (x1 << 16), x2 | (x3 << 16));
                    }
                }
            }
    
        };
        if (n != kC) body(std::false_type{}, std::true_type{});
        else if (!KDA || nrm) body(std::true_type{}, std::true_type{});
        else body(std::true_type{}, std::false_type{});
    };

    // A, P and the diagonal-block inverses of chunk c (buffer c & 1).  The
    // tile products run transposed, C^T = Kr M^T (M = Khat rows for A, Qhat
    // rows for P, Kr the right rows), so a lane ends up with 4 consecutive j
    // of one row t and stores 8 bytes.  Waves 0 and 2 hold the diagonal A
    // tiles of blocks 3, 0 and 2, 1 and invert them; the tile lists per wave
    // are below.
    auto prep_ap = [&](int c) {
        const bf16_t* Kh = prep_lds_b(c, L::oKh, L::pKh);
        const bf16_t* Qh = prep_lds_b(c, L::oQh, L::pQh);
        const bf16_t* Kr = Kh;  // right factor (j side) of the fused GDN products
        const float* sb = reinterpret_cast<const float*>(prep_lds_b(c, L::oBeta, L::pBeta));
        bf16_t* Pt = prep_out_b(c, L::oP);
        // kPrep keeps -A and D_r^{-1} in LDS: the image gets (I + A)^{-1} instead
        bf16_t* At = MODE == kPrep ? reinterpret_cast<bf16_t*>(smem + L::pA) : prep_out_b(c, L::oA);
        bf16_t* Dt = MODE == kPrep ? reinterpret_cast<bf16_t*>(smem + L::pD) : prep_out_b(c, L::oD);
        const bool isP = wave & 1;
        const int rA = wave < 2 ? 3 : 2;  // diagonal blocks inverted by waves 0 and 2
        const int rB = wave < 2 ? 0 : 1;
        if constexpr (ONEBAR) {
            // GDN fused: per-wave tile lists.  Waves 0 and 2 also invert the
            // diagonal blocks (3, 0) and (2, 1), so they form only those A
            // tiles and one more; waves 1 and 3 form the other 14.  Each wave
            // loads every right-hand (Kr) and left-hand (Khat / Qhat rows)
            // fragment it needs once per K step.  Gates: diagonal tiles take
            // 2^(G_t - G_j) per element, the others row x block-pair x column
            // factors.
            const float* sG = sGp(c);
            const float* ops = reinterpret_cast<const float*>(smem + (c % 3) * L::OPS);
            auto run = [&](auto tag) {
                using TL = decltype(tag);
                constexpr int NT = TL::n;
                auto uses_col = [&](int cc, int diag) {  // diag: -1 any, 0 off-diagonal, 1 diagonal
                    bool u = false;
#pragma unroll
                    for (int x = 0; x < NT; ++x) {
                        const int cd = TL::code[x], r = (cd >> 2) & 3, cl = cd & 3;
                        u |= cl == cc && (diag < 0 || (diag == 1) == (cl == r));
                    }
                    return u;
                };
                auto uses_row = [&](int rr, int what) {  // what: 0 any, 1 A tile, 2 diagonal, 3 off-diagonal
                    bool u = false;
#pragma unroll
                    for (int x = 0; x < NT; ++x) {
                        const int cd = TL::code[x], r = (cd >> 2) & 3, cl = cd & 3;
                        u |= r == rr && (what == 0 || (what == 1 && cd < 16) || (what == 2 && cl == r) ||
                                         (what == 3 && cl < r));
                    }
                    return u;
                };
                auto uses_m = [&](int key) {  // key = 4 isP + row
                    bool u = false;
#pragma unroll
                    for (int x = 0; x < NT; ++x) u |= (TL::code[x] >> 2) == key;
                    return u;
                };
                // epilogue scalars, read before the products
                float bt[4], gt[4], ut[4];
                float4 gj[4], wj[4], cr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (uses_row(r, 1)) bt[r] = sb[16 * r + lr];
                    if (uses_row(r, 2)) gt[r] = sG[16 * r + lr];
                    if (uses_row(r, 3)) {
                        ut[r] = ops[L::uU / 4 + 16 * r + lr];
                        cr[r] = *reinterpret_cast<const float4*>(ops + L::uC / 4 + 4 * r);
                    }
                }
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    if (uses_col(cc, 1)) gj[cc] = *reinterpret_cast<const float4*>(sG + 16 * cc + 4 * lg);
                    if (uses_col(cc, 0)) wj[cc] = *reinterpret_cast<const float4*>(ops + L::uW / 4 + 16 * cc + 4 * lg);
                }
                f32x4 acc[NT];
#pragma unroll
                for (int x = 0; x < NT; ++x) acc[x] = zero4();
#pragma unroll
                for (int s = 0; s < NKS; ++s) {
                    bf16x8 kr[4], mf[8];
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc)
                        if (uses_col(cc, -1)) kr[cc] = lds8(Kr + (16 * cc + lr) * L::PK + 32 * s + 8 * lg);
#pragma unroll
                    for (int key = 0; key < 8; ++key)
                        if (uses_m(key))
                            mf[key] = lds8((key >= 4 ? Qh : Kh) + (16 * (key & 3) + lr) * L::PK + 32 * s + 8 * lg);
#pragma unroll
                    for (int x = 0; x < NT; ++x) acc[x] = mfma32(kr[TL::code[x] & 3], mf[TL::code[x] >> 2], acc[x]);
                }
#pragma unroll
                for (int x = 0; x < NT; ++x) {
                    const int cd = TL::code[x], tP_ = cd >> 4, r = (cd >> 2) & 3, cl = cd & 3;
                    const int t = 16 * r + lr;
                    f32x4 val;
                    if (cl < r) {
                        const float4 w = wj[cl];
                        const float cf = cl == 0 ? cr[r].x : cl == 1 ? cr[r].y : cr[r].z;
                        // P tiles carry the output scale
                        const float f = tP_ ? ut[r] * cf * scale : ut[r] * cf;
                        const float wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float xx = acc[x][i] * f * wv[i];
                            val[i] = tP_ ? xx : bt[r] * xx;
                        }
                    } else {
                        const float4 g = gj[cl];
                        const float gv[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int j = 16 * cl + 4 * lg + i;
                            const float xx = acc[x][i] * ex2(fminf(gt[r] - gv[i], 0.f));
                            val[i] = tP_ ? (j <= t ? xx * scale : 0.f) : (j < t ? bt[r] * xx : 0.f);
                        }
                    }
                    if (tP_) {
                        st4(Pt + ptile(r, cl) * 16 * L::PD + lr * L::PD + 4 * lg, val);
                    } else if (cl < r) {
                        st4(At + atile(r, cl) * 16 * L::PD + lr * L::PD + 4 * lg, -val);
                    } else {  // diagonal tile, stored transposed: scr[j][t] = A[t][j]
                        float* scr = scr0 + r * 16 * L::PS;
#pragma unroll
                        for (int i = 0; i < 4; ++i) scr[(4 * lg + i) * L::PS + lr] = val[i];
                    }
                }
            };
            if (wave == 0) run(Tiles<tA(3, 3), tA(0, 0), tA(3, 2)>{});
            else if (wave == 1) run(Tiles<tP(3, 0), tP(3, 1), tP(3, 2), tP(3, 3), tA(3, 0), tA(3, 1), tP(0, 0)>{});
            else if (wave == 2) run(Tiles<tA(2, 2), tA(1, 1), tA(2, 1)>{});
            else run(Tiles<tP(2, 0), tP(2, 1), tP(2, 2), tP(1, 0), tP(1, 1), tA(2, 0), tA(1, 0)>{});
        } else {
            // Per-wave tile lists (code = 16 isP + 4 row + column): waves 0
            // and 2 form only the diagonal A tiles of the blocks they invert
            // (3, 0 and 2, 1), waves 1 and 3 the other 16 tiles, so that the
            // inversions run beside the larger share of the products.  Each
            // wave loads every right-hand fragment (KDA: from the row block's
            // own set of right rows) and left-hand fragment it needs once per
            // K step.
            const float* sG = sGp(c);
            auto run = [&](auto tag) {
                using TL = decltype(tag);
                constexpr int NT = TL::n;
                auto uses_rc = [&](int rr, int cc) {  // right fragment: row block rr's set (KDA), column tile cc
                    bool u = false;
#pragma unroll
                    for (int x = 0; x < NT; ++x) {
                        const int cd = TL::code[x], r = (cd >> 2) & 3, cl = cd & 3;
                        u |= cl == cc && (!KDA || r == rr);
                    }
                    return u;
                };
                auto uses_row = [&](int rr, int what) {  // what: 0 any tile, 1 A tile
                    bool u = false;
#pragma unroll
                    for (int x = 0; x < NT; ++x) {
                        const int cd = TL::code[x], r = (cd >> 2) & 3;
                        u |= r == rr && (what == 0 || cd < 16);
                    }
                    return u;
                };
                auto uses_m = [&](int key) {  // key = 4 isP + row
                    bool u = false;
#pragma unroll
                    for (int x = 0; x < NT; ++x) u |= (TL::code[x] >> 2) == key;
                    return u;
                };
                // epilogue scalars, read before the products
                float bt[4], gt[4];
                float4 gj[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (uses_row(r, 1)) bt[r] = sb[16 * r + lr];
                    if (!KDA && uses_row(r, 0)) gt[r] = sG[16 * r + lr];
                }
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
                    if (!KDA && uses_rc(0, cc)) gj[cc] = *reinterpret_cast<const float4*>(sG + 16 * cc + 4 * lg);
                f32x4 acc[NT];
#pragma unroll
                for (int x = 0; x < NT; ++x) acc[x] = zero4();
                constexpr int NR = KDA ? 4 : 1;  // right-row sets
#pragma unroll
                for (int s = 0; s < NKS; ++s) {
                    bf16x8 kr[NR][4], mf[8];
#pragma unroll
                    for (int rr = 0; rr < NR; ++rr)
#pragma unroll
                        for (int cc = 0; cc < 4; ++cc)
                            if (uses_rc(rr, cc)) {
                                const int row = (KDA ? rr_row0(rr) : 0) + 16 * cc + lr;  // row of Kc (KDA) / Khat
                                kr[rr][cc] = lds8((KDA ? Kc : Kh) + row * L::PK + kpos(row, 32 * s + 8 * lg));
                            }
#pragma unroll
                    for (int key = 0; key < 8; ++key)
                        if (uses_m(key)) {
                            const int row = 16 * (key & 3) + lr;
                            mf[key] = lds8((key >= 4 ? Qh : Kh) + row * L::PK + kpos(row, 32 * s + 8 * lg));
                        }
#pragma unroll
                    for (int x = 0; x < NT; ++x) {
                        const int cd = TL::code[x];
                        acc[x] = mfma32(kr[KDA ? (cd >> 2) & 3 : 0][cd & 3], mf[cd >> 2], acc[x]);
                    }
                }
#pragma unroll
                for (int x = 0; x < NT; ++x) {
                    const int cd = TL::code[x], tP_ = cd >> 4, r = (cd >> 2) & 3, cl = cd & 3;
                    const int t = 16 * r + lr;
                    float gv[4] = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (!KDA) {
                        gv[0] = gj[cl].x; gv[1] = gj[cl].y; gv[2] = gj[cl].z; gv[3] = gj[cl].w;
                    }
                    f32x4 val;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = 16 * cl + 4 * lg + i;
                        float xx = acc[x][i];
                        if constexpr (!KDA) xx *= ex2(fminf(gt[r] - gv[i], 0.f));
                        val[i] = tP_ ? (j <= t ? xx : 0.f) : (j < t ? bt[r] * xx : 0.f);
                    }
                    if (tP_) {
                        st4(Pt + ptile(r, cl) * 16 * L::PD + lr * L::PD + 4 * lg, val);
                    } else if (cl < r) {
                        st4(At + atile(r, cl) * 16 * L::PD + lr * L::PD + 4 * lg, -val);
                    } else {  // diagonal tile, stored transposed: scr[j][t] = A[t][j]
                        float* scr = scr0 + r * 16 * L::PS;
#pragma unroll
                        for (int i = 0; i < 4; ++i) scr[(4 * lg + i) * L::PS + lr] = val[i];
                    }
                }
            };
            if (wave == 0) run(Tiles<tA(3, 3), tA(0, 0)>{});
            else if (wave == 2) run(Tiles<tA(2, 2), tA(1, 1)>{});
            else if (wave == 1)
                run(Tiles<tP(3, 0), tP(3, 1), tP(3, 2), tP(3, 3), tP(0, 0), tA(3, 0), tA(3, 1), tA(3, 2)>{});
            else run(Tiles<tP(2, 0), tP(2, 1), tP(2, 2), tP(1, 0), tP(1, 1), tA(2, 0), tA(2, 1), tA(1, 0)>{});
        }
        // D_r^{-1} = (I + A_rr)^{-1}: lanes 0..15 invert block rA, lanes 16..31
        // block rB; lane c solves column c by right-looking forward
        // substitution (x_i -= A_ij x_j for all i > j at step j).
        if (!isP && lane < 32) {
            const int blk = lane < 16 ? rA : rB;
            const int cl = lane & 15;
            const float* scr = scr0 + blk * 16 * L::PS;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == cl) ? 1.f : 0.f;
            // columns of A_rr are read three steps ahead of their use (only
            // the float4 groups holding rows below the diagonal)
            float4 col[3][4];
            auto load_col = [&](int j, float4 (&dst)[4]) {
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4)
                    if (4 * i4 + 3 > j) dst[i4] = *reinterpret_cast<const float4*>(scr + j * L::PS + 4 * i4);
            };
            load_col(0, col[0]);
            load_col(1, col[1]);
            load_col(2, col[2]);
#pragma unroll
            for (int j = 0; j < 15; ++j) {
                float a[16];
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const float4 r = col[j % 3][i4];
                    a[4 * i4] = r.x; a[4 * i4 + 1] = r.y; a[4 * i4 + 2] = r.z; a[4 * i4 + 3] = r.w;
                }
                if (j + 3 < 15) load_col(j + 3, col[j % 3]);
#pragma unroll
                for (int i = j + 1; i < 16; ++i) x[i] -= a[i] * x[j];
            }
            bf16_t* Dw = Dt + blk * 16 * L::PD;
#pragma unroll
            for (int i = 0; i < 16; ++i) Dw[i * L::PD + cl] = static_cast<bf16_t>(bf_bits(x[i]));
        }
    };

    // kPrep: the 16x16 blocks of T = (I + A)^{-1} from -A and the D_r^{-1}
    // (after the barrier that follows prep_ap):
    //   T_rr = D_r^{-1},  T_rk = D_r^{-1} sum_{k<=m<r} (-A_rm) T_mk.
    // Each column k of blocks depends only on its own blocks above, so the
    // columns are independent chains: part 0 forms column 0 (T_10, T_20,
    // T_30), part 1 columns 1 and 2 (T_21, T_31, T_32) and copies the T_rr.
    // Z = sum_m (-A_rm) T_mk is formed in the accumulator layout, which is
    // the A-operand layout of Z^T, so the second product gives (D_r^{-1} Z)^T,
    // whose accumulator layout is the row-fragment layout the chain reads.
    auto prep_t = [&](int c, int part) {
        const bf16_t* Ab = reinterpret_cast<const bf16_t*>(smem + L::pA);
        const bf16_t* Dl = reinterpret_cast<const bf16_t*>(smem + L::pD);
        bf16_t* Tl = reinterpret_cast<bf16_t*>(smem + L::pT);
        bf16_t* Ti = prep_out_b(c, L::oA);  // T_rk, k < r, in the slots of -A_rk
        bf16_t* Di = prep_out_b(c, L::oD);  // T_rr
        auto row_frag = [&](const bf16_t* t) { return lds4(t + lr * L::PD + 4 * lg); };
        auto col_frag = [&](const bf16_t* t) {  // t[4 lg + i][lr], i = 0..3 (transposing read)
            typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
            const bf16_t* p = t + (4 * lg + (lr >> 2)) * L::PD + 4 * (lr & 3);
            return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
        };
        if (part == 1) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<uint2*>(Di + r * 16 * L::PD + lr * L::PD + 4 * lg) =
                    *reinterpret_cast<const uint2*>(Dl + r * 16 * L::PD + lr * L::PD + 4 * lg);
        }
#pragma unroll
        for (int r = 1; r < 4; ++r) {
            const bf16x4 dr = row_frag(Dl + r * 16 * L::PD);
#pragma unroll
            for (int kk = 0; kk < r; ++kk) {
                if ((kk == 0) != (part == 0)) continue;
                f32x4 z = zero4();
#pragma unroll
                for (int m = kk; m < r; ++m) {
                    const bf16_t* tmk = m == kk ? Dl + kk * 16 * L::PD : Tl + atile(m, kk) * 16 * L::PD;
                    z = mfma16(row_frag(Ab + atile(r, m) * 16 * L::PD), col_frag(tmk), z);
                }
                const f32x4 tt = mfma16(cvt4(z), dr, zero4());  // lane: T_rk[lr][4 lg + i]
                st4(Tl + atile(r, kk) * 16 * L::PD + lr * L::PD + 4 * lg, tt);
                st4(Ti + atile(r, kk) * 16 * L::PD + lr * L::PD + 4 * lg, tt);
            }
        }
    };

    // ================= serial-wave work =================
    const int sw = wave - kLead;
    const int col0 = slice * DVS + 16 * sw;  // first value column of this wave
    f32x4 S[NRT];
    f32x4 Uf[4];
    bf16x4 Ub[4];
    bf16x8 bS[NKS];
    const size_t sbase = static_cast<size_t>(srow) * DK * DV;
    const size_t vrow0 = tseq * H + h;  // token (b, 0, h)
    // v of a chunk, loaded a chunk ahead so the registers carry the prefetch
    // across the barrier.  Staged (VSTAGE): two 16-byte loads per lane (rows
    // 32 x + lane / 2, 8 columns each), later written to the wave's LDS tile
    // and read back transposed into the accumulator layout.  Otherwise: the
    // 32-bit word holding this lane's column for each of its 16 rows (two
    // lanes share a word; the half is picked where it is used).
    constexpr bool VSTAGE = L::vstage(MODE, KDA);
    typedef unsigned int VIn __attribute__((ext_vector_type(VSTAGE ? 8 : 16)));
    auto serial_vload = [&](int c, VIn& V) {
        const int t0 = c * kC, nn = min(kC, T - t0);
        const bf16_t* vb = v + (vrow0 + static_cast<size_t>(t0) * H) * DV + col0;  // uniform
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(vb, static_cast<uint32_t>(nn * H * DV * 2));
        if constexpr (VSTAGE) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int t = 32 * x + (lane >> 1);
                const uint32_t off = t < nn ? static_cast<uint32_t>((t * H * DV + 8 * (lane & 1)) * 2) : kOOB;
                const uint4 w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
                V[4 * x] = w.x; V[4 * x + 1] = w.y; V[4 * x + 2] = w.z; V[4 * x + 3] = w.w;
            }
        } else {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * rt + 4 * lg + i;
                    const uint32_t off = t < nn ? static_cast<uint32_t>((t * H * DV + (lr & ~1)) * 2) : kOOB;
                    V[4 * rt + i] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
                }
        }
    };
    // ---- operands of one chunk, grouped by the phase that consumes them ----
    // kFused loads each group right before its phase; kChain issues the next
    // group's LDS reads before each phase's products (scheduling barriers keep
    // that order), so LDS latency overlaps the matrix-core work.
    typedef bf16x8 KFrag[4][NKS];
    struct OpsA {
        KFrag kf;                     // Khat rows 16 rt + lr, permuted k
        float4 b4[4], e4[4];          // beta_t, GDN 2^G_t, rows t = 16 rt + 4 lg + i
        bf16x4 Df[4], Af[6];          // kFused: D_r^{-1} and -A_rk; kChain: blocks of (I + A)^{-1}
    };
    struct OpsB {
        bf16x8 qf[4][NKS], pf[6];     // Qhat rows 16 rt + lr; P pieces (rt, s) with 2 s <= rt
        float egt[4];                 // GDN 2^G_t of row t = 16 rt + lr
        bf16x8 kt[NRT][2];            // Ktil^T rows 16 r + lr, permuted k (tokens)
        float4 ek[2][2];              // GDN 2^(G_end - G_t), U rows 32 s + 16 h + 4 lg + i
        float4 ge[KDA ? NRT : 1];     // 2^G_end (KDA: of S rows 16 r + 4 lg + i)
    };
    // LITE chain: fragments of the staged raw rows (unit-permuted, see swz)
    auto stg = [&](int c, int region) { return smem + (c & 1) * kStride + region; };
    auto perm_frag = [&](const unsigned char* base, int t, int e) {  // elements e..e+3, e+16..e+19 of row t
        const int sw = swz<L::U>(t);
        const unsigned char* row = base + t * (L::DKP * 2);
        const uint2 lo = *reinterpret_cast<const uint2*>(row + 16 * ((e >> 3) ^ sw) + 2 * (e & 7));
        const uint2 hi = *reinterpret_cast<const uint2*>(row + 16 * (((e + 16) >> 3) ^ sw) + 2 * (e & 7));
        return cat8(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
    };
    // transposing read: the 16 lanes of a group address 4 rows (lr >> 2) at
    // 4 column quads (lr & 3); lane m receives column e0 + m of the 4 rows
    auto tr_frag = [&](const unsigned char* base, int t, int e) {
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const unsigned char* p = base + t * (L::DKP * 2) + 16 * ((e >> 3) ^ swz<L::U>(t)) + 2 * (e & 7);
        return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
    };
    auto load_a1 = [&](int c, OpsA& A) {
        if constexpr (LITE && MODE == kChain) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int s = 0; s < NKS; ++s)
                    A.kf[rt][s] = perm_frag(stg(c, L::lK), 16 * rt + lr, 32 * s + 4 * lg);
            return;
        }
        const bf16_t* Kh = bfp(c, L::oKh);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int s = 0; s < NKS; ++s)
                A.kf[rt][s] = ONEBAR ? lds8(Kh + (16 * rt + lr) * L::PK + 32 * s + 8 * lg)  // permuted rows
                                     : lds_perm(Kh + (16 * rt + lr) * L::PK + 32 * s + 4 * lg);
    };
    auto load_a2 = [&](int c, OpsA& A) {
        const float* sb = f32p(c, L::oBeta);
        const float* eg = f32p(c, L::oEg);
        const bf16_t* At = bfp(c, L::oA);
        const bf16_t* Dt = bfp(c, L::oD);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            A.b4[rt] = *reinterpret_cast<const float4*>(sb + 16 * rt + 4 * lg);
            A.e4[rt] = KDA ? make_float4(1.f, 1.f, 1.f, 1.f)
                           : *reinterpret_cast<const float4*>(eg + 16 * rt + 4 * lg);
            A.Df[rt] = lds4(Dt + rt * 16 * L::PD + lr * L::PD + 4 * lg);
        }
#pragma unroll
        for (int x = 0; x < 6; ++x) A.Af[x] = lds4(At + x * 16 * L::PD + lr * L::PD + 4 * lg);
    };
    auto load_b1 = [&](int c, OpsB& Bo) {
        const bf16_t* Qh = bfp(c, L::oQh);
        const bf16_t* Pt = bfp(c, L::oP);
        const float* eg = f32p(c, L::oEg);
        const float* es = ONEBAR ? reinterpret_cast<const float*>(smem + (c % 3) * L::OPS + L::uEs) : eg;
        const bf16x4 z4 = cvt4(zero4());
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
            for (int s = 0; s < NKS; ++s)
                Bo.qf[rt][s] = (LITE && MODE == kChain)
                    ? perm_frag(stg(c, L::lQ), 16 * rt + lr, 32 * s + 4 * lg)
                    : ONEBAR ? lds8(Qh + (16 * rt + lr) * L::PK + 32 * s + 8 * lg)  // permuted rows
                             : lds_perm(Qh + (16 * rt + lr) * L::PK + 32 * s + 4 * lg);
            // GDN 2^G_t (ONEBAR: scale 2^G_t; P carries the scale too)
            Bo.egt[rt] = KDA ? 1.f : ONEBAR ? es[16 * rt + lr] : eg[16 * rt + lr];
        }
        // P pieces: (rt, s) for 2 s <= rt -> 6 pieces
#pragma unroll
        for (int rt = 0, x = 0; rt < 4; ++rt)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                if (2 * s <= rt) {
                    const bf16x4 plo = lds4(Pt + ptile(rt, 2 * s) * 16 * L::PD + lr * L::PD + 4 * lg);
                    const bf16x4 phi = (2 * s + 1 <= rt)
                        ? lds4(Pt + ptile(rt, 2 * s + 1) * 16 * L::PD + lr * L::PD + 4 * lg) : z4;
                    Bo.pf[x++] = cat8(plo, phi);
                }
    };
    auto load_b2 = [&](int c, OpsB& Bo) {
        const bf16_t* Kt = ONEBAR ? bfp(c, L::oKh) : bfp(c, L::oKt);  // ONEBAR: Khat rows, read transposed
        const float* ek = f32p(c, L::oEk);
        const float* ge = f32p(c, L::oGend);
#pragma unroll
        for (int r = 0; r < NRT; ++r)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if constexpr (LITE && MODE == kChain) {
                    const int t = 32 * s + 4 * lg + (lr >> 2), e = 16 * r + 4 * (lr & 3);
                    Bo.kt[r][s] = cat8(tr_frag(stg(c, L::lK), t, e), tr_frag(stg(c, L::lK), t + 16, e));
                } else if constexpr (ONEBAR) {
                    // lane m of a 16-lane group receives K[t0 + i][16 r + m], i = 0..3,
                    // from 4 rows x 4 channel quads addressed by the group (the
                    // quad of channels 16 r + 4 q .. + 3 sits at perm_pos(16 r + 4 q))
                    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
                    const bf16_t* p = Kt + (32 * s + 4 * lg + (lr >> 2)) * L::PK + 32 * (r >> 1) + 8 * (lr & 3) + 4 * (r & 1);
                    const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
                    const bf16x4 hi = __builtin_bit_cast(
                        bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * L::PK)));
                    Bo.kt[r][s] = cat8(lo, hi);
                } else {
                    Bo.kt[r][s] = lds_perm(Kt + (16 * r + lr) * L::PT + 32 * s + 4 * lg);
                }
            }
        if constexpr (KDA) {
#pragma unroll
            for (int r = 0; r < NRT; ++r) Bo.ge[r] = *reinterpret_cast<const float4*>(ge + 16 * r + 4 * lg);
        } else {
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    Bo.ek[s][hh] = *reinterpret_cast<const float4*>(ek + 32 * s + 16 * hh + 4 * lg);
            Bo.ge[0] = make_float4(ge[0], 0.f, 0.f, 0.f);
        }
    };

    // phase 1: Khat S (the B operands are S rounded to bf16)
    auto phase_ks = [&](const OpsA& A, f32x4 (&acc)[4]) {
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const f32x4 lo = S[2 * s];
            const f32x4 hi = (2 * s + 1 < NRT) ? S[2 * s + 1] : zero4();
            bS[s] = cat8(cvt4(lo), cvt4(hi));
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[rt] = zero4();
#pragma unroll
        for (int s = 0; s < NKS; ++s)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) acc[rt] = mfma32(A.kf[rt][s], bS[s], acc[rt]);
    };
    // v of the chunk in the accumulator layout, vv[rt][i] = v[16 rt + 4 lg + i][col0 + lr]
    // (staged: through the wave's LDS tile)
    auto v_regs = [&](const VIn& V, float (&vv)[4][4]) {
        if constexpr (VSTAGE) {
            typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
            unsigned char* vt = smem + L::vbase(MODE, KDA) + sw * L::VST;
#pragma unroll
            for (int x = 0; x < 2; ++x)
                *reinterpret_cast<uint4*>(vt + 1024 * x + 16 * lane) =
                    make_uint4(V[4 * x], V[4 * x + 1], V[4 * x + 2], V[4 * x + 3]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const unsigned char* p = vt + (16 * rt + 4 * lg + (lr >> 2)) * 32 + 8 * (lr & 3);
                const s16x4 w = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    vv[rt][i] = __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(w[i])) << 16);
            }
        } else {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    vv[rt][i] = (lr & 1) ? bf_hi(V[4 * rt + i]) : bf_lo(V[4 * rt + i]);
        }
    };
    // phase 2: X = diag(beta) (V - Khat S), U = (I + A)^{-1} X
    auto phase_u = [&](const OpsA& A, const f32x4 (&acc)[4], const float (&vv)[4][4]) {
        f32x4 X[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const float bb[4] = {A.b4[rt].x, A.b4[rt].y, A.b4[rt].z, A.b4[rt].w};
            const float ee[4] = {A.e4[rt].x, A.e4[rt].y, A.e4[rt].z, A.e4[rt].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) X[rt][i] = bb[i] * (vv[rt][i] - ee[i] * acc[rt][i]);
        }
        if constexpr (MODE == kChain) {
            // U_r = sum_{k <= r} T_rk X_k: independent products (no chain)
            bf16x4 Xb[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) Xb[rt] = cvt4(X[rt]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 w = mfma16(A.Df[rt], Xb[rt], zero4());
#pragma unroll
                for (int kb = 0; kb < rt; ++kb) w = mfma16(A.Af[atile(rt, kb)], Xb[kb], w);
                Uf[rt] = w;
                Ub[rt] = cvt4(w);
            }
        } else {
            // blocked forward substitution: U_r = D_r^{-1} (X_r - sum_{k<r} A_rk U_k)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 w = X[rt];
#pragma unroll
                for (int kb = 0; kb < rt; ++kb) w = mfma16(A.Af[atile(rt, kb)], Ub[kb], w);
                Uf[rt] = mfma16(A.Df[rt], cvt4(w), zero4());
                Ub[rt] = cvt4(Uf[rt]);
            }
        }
    };
    // phase 3: O = scale (Qhat S + P U), computed transposed (a lane holds 4
    // consecutive columns of one token row)
    auto phase_o = [&](int c, const OpsB& Bo) {
        const int t0 = c * kC, n = min(kC, T - t0);
        const bf16_t* ob = o + (vrow0 + static_cast<size_t>(t0) * H) * DV + col0;  // uniform
        const __amdgpu_buffer_rsrc_t ors = make_rsrc(ob, static_cast<uint32_t>(n * H * DV * 2));
        f32x4 oacc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
        for (int s = 0; s < NKS; ++s)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) oacc[rt] = mfma32(bS[s], Bo.qf[rt][s], oacc[rt]);
        const bf16x8 u01 = cat8(Ub[0], Ub[1]), u23 = cat8(Ub[2], Ub[3]);
#pragma unroll
        for (int rt = 0, x = 0; rt < 4; ++rt) {
            if constexpr (!KDA) oacc[rt] *= Bo.egt[rt];
            oacc[rt] = mfma32(u01, Bo.pf[x++], oacc[rt]);
            if (rt >= 2) oacc[rt] = mfma32(u23, Bo.pf[x++], oacc[rt]);
            const int t = 16 * rt + lr;
            const uint32_t off = t < n ? static_cast<uint32_t>((t * H * DV + 4 * lg) * 2) : kOOB;
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, cvt4(ONEBAR ? oacc[rt] : oacc[rt] * scale)), ors,
                                                  off, 0, 0);
        }
    };
    // phase 4: S <- diag(2^G_end) S + Ktil^T U
    auto phase_s = [&](const OpsB& Bo) {
        bf16x8 bU[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if constexpr (KDA) {
                bU[s] = cat8(Ub[2 * s], Ub[2 * s + 1]);
            } else {
                f32x4 lo = Uf[2 * s], hi = Uf[2 * s + 1];
                const float4 k0 = Bo.ek[s][0], k1 = Bo.ek[s][1];
                lo[0] *= k0.x; lo[1] *= k0.y; lo[2] *= k0.z; lo[3] *= k0.w;
                hi[0] *= k1.x; hi[1] *= k1.y; hi[2] *= k1.z; hi[3] *= k1.w;
                bU[s] = cat8(cvt4(lo), cvt4(hi));
            }
        }
#pragma unroll
        for (int r = 0; r < NRT; ++r) {
            if constexpr (KDA) {
                S[r][0] *= Bo.ge[r].x; S[r][1] *= Bo.ge[r].y; S[r][2] *= Bo.ge[r].z; S[r][3] *= Bo.ge[r].w;
            } else {
                S[r] *= Bo.ge[0].x;
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int r = 0; r < NRT; ++r) S[r] = mfma32(Bo.kt[r][s], bU[s], S[r]);
    };

    // ================= pipeline =================
    auto serial_init = [&]() {
#pragma unroll
        for (int r = 0; r < NRT; ++r) {
            S[r] = zero4();
            if (init) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[r][i] = state_in[sbase + static_cast<size_t>(16 * r + 4 * lg + i) * DV + col0 + lr];
            }
        }
        // Wait for the initial state here, so that no load into S is pending
        // at the loop head (otherwise every iteration would wait for all
        // memory operations, including the previous chunk's output stores).
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    };
    auto serial_fini = [&]() {
#pragma unroll
        for (int r = 0; r < NRT; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                state_out[sbase + static_cast<size_t>(16 * r + 4 * lg + i) * DV + col0 + lr] = S[r][i];
    };
    // Four dropped (out-of-range) stores: the loop head is then reached with
    // the same memory-op order from both sides (v loads, then the four output
    // stores), so the wait for v there does not also wait for output stores.
    auto dummy_stores = [&]() {
        const __amdgpu_buffer_rsrc_t nul = make_rsrc(o, 0);
#pragma unroll
        for (int x = 0; x < 4; ++x) __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, nul, kOOB + 8 * x, 0, 0);
    };

    if constexpr (MODE == kPrep) {
        // A few consecutive chunks of one head per workgroup; the inputs of
        // chunk c+1 are loaded into registers while chunk c is gated and
        // multiplied, and the outputs go straight to the image.  prep_t of
        // chunk c only touches its own LDS tiles, which the next chunk's
        // products overwrite after the next barrier.  It runs on waves 1 and
        // 3 (one column chain each side), which invert nothing.
        PrepIn pin;
        // (a packed sequence may end before this workgroup's chunks begin)
        if (pc < pc_end) prep_load(pc, pin);
        for (int c = pc; c < pc_end; ++c) {
            zero_image_pad(c);
            prep_gate(c, pin);
            if (c + 1 < pc_end) prep_load(c + 1, pin);
            lds_barrier();
            prep_ap(c);
            lds_barrier();
            if (wave & 1) prep_t(c, wave >> 1);
        }
    } else if constexpr (MODE == kChain) {
        if (wave < kLoad) {
            // Loader: image of chunk c -> LDS buffer c & 1, 1 KB per instruction
            // (lane l moves bytes [16 l, 16 l + 16) of each kilobyte).
            auto copy_in = [&](int c) {
                const unsigned char* src = imgp(c) + 16 * lane;
                auto dst = (__attribute__((address_space(3))) unsigned char*)(smem + (c & 1) * L::IMG);
                for (int j = wave; j < L::IMG / 1024; j += kLoad)
                    __builtin_amdgcn_global_load_lds(src + 1024 * j, dst + 1024 * j, 16, 0, 0);
            };
            copy_in(c0);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the copy has landed in LDS
            lds_barrier();
            for (int i = c0; i < nch; ++i) {
                if (i + 1 < nch) copy_in(i + 1);
                __builtin_amdgcn_s_waitcnt(0x0F70);
                lds_barrier();
            }
        } else {
            serial_init();
            // LITE: each serial wave stages its share of the next chunk's raw
            // k and q rows (range-checked buffer loads: rows past a ragged end
            // read as zeros) and of its tile image through registers
            constexpr int NUK = kC * (DK / 8);  // 16-byte units of k (or q) rows
            constexpr int NUI = L::TIMG / 16;
            constexpr int NT = NSW * 64;
            constexpr int XK = LITE ? (NUK + NT - 1) / NT : 1, XI = LITE ? (NUI + NT - 1) / NT : 1;
            const int sl = sw * 64 + lane;
            // (register vectors, not arrays, so the staging stays in registers)
            typedef unsigned int VK __attribute__((ext_vector_type(4 * XK)));
            typedef unsigned int VI __attribute__((ext_vector_type(4 * XI)));
            VK stk, stq;
            VI sti;
            auto stage_load = [&](int c) {
                if constexpr (LITE) {
                    const int t0 = c * kC, nn = min(kC, T - t0);
                    const size_t rb = tok0 + static_cast<size_t>(t0) * H;
                    const uint32_t range = static_cast<uint32_t>(((nn - 1) * H * DK + DK) * 2);
                    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + rb * DK, range);
                    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + rb * DK, range);
#pragma unroll
                    for (int x = 0; x < XK; ++x) {
                        const int g = x * NT + sl, r = g / (DK / 8), u = g % (DK / 8);
                        const uint32_t off = g < NUK ? static_cast<uint32_t>((r * H * DK + 8 * u) * 2) : kOOB;
                        const uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
                        const uint4 bq = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
                        stk[4 * x] = a.x; stk[4 * x + 1] = a.y; stk[4 * x + 2] = a.z; stk[4 * x + 3] = a.w;
                        stq[4 * x] = bq.x; stq[4 * x + 1] = bq.y; stq[4 * x + 2] = bq.z; stq[4 * x + 3] = bq.w;
                    }
                    const uint4* src = reinterpret_cast<const uint4*>(imgp(c));
#pragma unroll
                    for (int x = 0; x < XI; ++x) {
                        const int m = x * NT + sl;
                        const uint4 a = src[m < NUI ? m : 0];
                        sti[4 * x] = a.x; sti[4 * x + 1] = a.y; sti[4 * x + 2] = a.z; sti[4 * x + 3] = a.w;
                    }
                }
            };
            auto stage_store = [&](int c) {
                if constexpr (LITE) {
                    unsigned char* base = smem + (c & 1) * kStride;
#pragma unroll
                    for (int x = 0; x < XK; ++x) {
                        const int g = x * NT + sl, r = g / (DK / 8), u = g % (DK / 8);
                        if (g < NUK) {
                            const int pos = (r * L::DKP + 8 * (u ^ swz<L::U>(r))) * 2;
                            *reinterpret_cast<uint4*>(base + L::lK + pos) =
                                make_uint4(stk[4 * x], stk[4 * x + 1], stk[4 * x + 2], stk[4 * x + 3]);
                            *reinterpret_cast<uint4*>(base + L::lQ + pos) =
                                make_uint4(stq[4 * x], stq[4 * x + 1], stq[4 * x + 2], stq[4 * x + 3]);
                        }
                    }
#pragma unroll
                    for (int x = 0; x < XI; ++x) {
                        const int m = x * NT + sl;
                        if (m < NUI)
                            *reinterpret_cast<uint4*>(base + L::lT + 16 * m) =
                                make_uint4(sti[4 * x], sti[4 * x + 1], sti[4 * x + 2], sti[4 * x + 3]);
                    }
                }
            };
            if constexpr (LITE && L::DKP != DK) {
                // staged rows are DKP wide: zero both buffers once (pad units are never written)
                for (int idx = tid; idx < 2 * L::lT / 16; idx += blockDim.x) {
                    const int bsel = idx / (L::lT / 16), rem16 = idx % (L::lT / 16);
                    *reinterpret_cast<uint4*>(smem + bsel * kStride + 16 * rem16) = make_uint4(0, 0, 0, 0);
                }
                lds_barrier();
            }
            if (c0 < nch) {
                stage_load(c0);
                stage_store(c0);
            }
            VIn vr;  // v of the next chunk, prefetched one step ahead
            if (c0 < nch) serial_vload(c0, vr);
            dummy_stores();
            lds_barrier();  // chunk c0 is in its buffer
            for (int i = c0; i < nch; ++i) {
                if (i + 1 < nch) stage_load(i + 1);
                OpsA A;
                OpsB Bo;
                f32x4 acc[4];
                load_a1(i, A);
                __builtin_amdgcn_sched_barrier(0);
                load_a2(i, A);
                phase_ks(A, acc);
                // v's LDS round trip before the next phase's operand reads:
                // LDS requests complete in order, so X would otherwise wait
                // for all of them
                float vv[4][4];
                v_regs(vr, vv);
                __builtin_amdgcn_sched_barrier(0);
                load_b1(i, Bo);
                phase_u(A, acc, vv);
                if (i + 1 < nch) serial_vload(i + 1, vr);
                __builtin_amdgcn_sched_barrier(0);
                load_b2(i, Bo);
                phase_o(i, Bo);
                __builtin_amdgcn_sched_barrier(0);
                phase_s(Bo);
                if (i + 1 < nch) stage_store(i + 1);
                lds_barrier();  // chunk i + 1 has landed; buffer i & 1 is free
            }
            serial_fini();
        }
    } else if (prep) {
        // Each role runs its own loop: nch + 1 iterations with exactly two
        // workgroup barriers each, so the barriers pair up across roles while
        // the compiler keeps only one role's loop-carried registers live.
        // Inputs of chunk i+2 are loaded into registers while chunk i+1 is
        // gated, so the global loads overlap one whole step.
        PrepIn pin;
        if constexpr (ONEBAR) {
            // one barrier per step: gate chunk i+2 (operand set (i+2) % 3)
            // and form A, P, D_r^{-1} of chunk i+1 (gated a step earlier)
            // while the serial waves run chunk i; nch + 2 barriers in all.
            // The inputs alternate between two register sets (even / odd
            // chunks) and are loaded two steps ahead.
            // Every step issues its loads (past the end: zeros), so the
            // loads come in the same order on every path.
            PrepIn pin2;
            prep_load(0, pin);
            prep_load(1, pin2);
            auto step = [&](int i, PrepIn& cur) {  // cur holds chunk i + 2
                if (i + 2 < nch) prep_gate(i + 2, cur);
                prep_load(i + 4, cur);
                if (i + 1 >= 0 && i + 1 < nch) prep_ap(i + 1);
                lds_barrier();
            };
            for (int i = -2; i < nch; i += 2) {
                step(i, pin);
                if (i + 1 < nch) step(i + 1, pin2);
            }
        } else {
            if (nch > 0) prep_load(0, pin);
            for (int i = -1; i < nch; ++i) {
                if (i + 1 < nch) {
                    prep_gate(i + 1, pin);
                    if (i + 2 < nch) prep_load(i + 2, pin);
                }
                lds_barrier();
                if (i + 1 < nch) prep_ap(i + 1);
                lds_barrier();
            }
        }
    } else if constexpr (ONEBAR) {
        serial_init();
        // a whole chunk between barriers (the prep waves never write the
        // operand set or tile set of the chunk being run); v alternates
        // between two register sets as below
        auto body = [&](int i, VIn& cur, VIn& nxt) {
            if (i + 1 < nch) serial_vload(i + 1, nxt);
            {
                OpsA A;
                f32x4 acc[4];
                float vv[4][4];
                load_a1(i, A);
                load_a2(i, A);
                phase_ks(A, acc);
                v_regs(cur, vv);
                phase_u(A, acc, vv);
            }
            __builtin_amdgcn_sched_barrier(0);
            {
                OpsB Bo;
                load_b1(i, Bo);
                phase_o(i, Bo);
                load_b2(i, Bo);
                phase_s(Bo);
            }
            lds_barrier();
        };
        VIn va, vb;
        if (nch > 0) serial_vload(0, va);
        dummy_stores();
        // prep steps -2 and -1 (gate chunks 0 and 1, form chunk 0) have no
        // serial work
        lds_barrier();
        lds_barrier();
        for (int i = 0; i < nch; i += 2) {
            body(i, va, vb);
            if (i + 1 < nch) body(i + 1, vb, va);
        }
        serial_fini();
    } else {
        serial_init();
        // v alternates between two register sets (even / odd chunks): the
        // loads of chunk i+1 go out at the start of chunk i, independent of
        // the set chunk i consumes
        auto body = [&](int i, VIn& cur, VIn& nxt) {
            if (i + 1 < nch) serial_vload(i + 1, nxt);
            {
                OpsA A;
                f32x4 acc[4];
                float vv[4][4];
                load_a1(i, A);
                load_a2(i, A);
                phase_ks(A, acc);
                v_regs(cur, vv);
                phase_u(A, acc, vv);
            }
            lds_barrier();
            {
                OpsB Bo;
                load_b1(i, Bo);
                phase_o(i, Bo);
                load_b2(i, Bo);
                phase_s(Bo);
            }
            lds_barrier();
        };
        VIn va, vb;
        if (nch > 0) serial_vload(0, va);
        dummy_stores();
        // iteration -1 (prep gates and forms chunk 0) has no serial work; it
        // is peeled so that every loop iteration issues its output stores
        lds_barrier();
        lds_barrier();
        for (int i = 0; i < nch; i += 2) {
            body(i, va, vb);
            if (i + 1 < nch) body(i + 1, vb, va);
        }
        serial_fini();
    }
}

// Chunks per range of the split schedule: the images of one range (all heads)
// stay within 136 MiB, inside the 256 MB last-level cache, so the chain
// kernel reads what the chunk-local kernel has just written from cache (KDA
// workload: 64-chunk ranges; 96 MiB measured 2.4% slower, 160 MiB the same).
constexpr size_t kRangeBytes = size_t(136) << 20;
// Chunk-local workgroups of one range (about two per CU; KDA: one, its LDS
// allows one per CU).
constexpr int prep_groups(bool kda) { return kda ? 256 : 512; }
inline int split_range_chunks(int BH, int nch, size_t img_bytes, bool kda) {
    const size_t per_chunk = static_cast<size_t>(BH) * img_bytes;
    const size_t r = per_chunk ? kRangeBytes / per_chunk : 0;
    int rc = static_cast<int>(std::max<size_t>(1, std::min<size_t>(static_cast<size_t>(nch), r)));
    // A range of a multiple of `unit` chunks gives every chunk-local
    // workgroup the same number of chunks (KDA workload: 40-chunk ranges, 5
    // chunks per workgroup, instead of 45 with 6 for most and 3 for some).
    const int unit = prep_groups(kda) / std::gcd(prep_groups(kda), std::max(BH, 1));
    if (rc < nch && rc > unit) rc = rc / unit * unit;
    return rc;
}

template <int DK, int NSW, bool KDA>
hipError_t launch(int B, int T, int H, int DV, float scale, const bf16_t* q, const bf16_t* k,
                  const bf16_t* v, const float* alpha, const float* beta, const float* s_in,
                  float* s_out, bf16_t* o, unsigned char* img, size_t img_cap, hipStream_t s,
                  const Opts& vl) {
    using L = Layout<DK, NSW, KDA>;
    const int NS = DV / (16 * NSW);
    const int groups = (B * H + 7) / 8;
    const unsigned long long blocks64 = static_cast<unsigned long long>(groups) * 8u * NS;
    if (!grid_fits(blocks64, block_threads<NSW, KDA, kFused>()) ||
        !grid_fits(blocks64, block_threads<NSW, KDA, kChain>()))
        return hipErrorInvalidConfiguration;
    const unsigned blocks = static_cast<unsigned>(blocks64);
    auto set_lds = [](const void* kern, int bytes) {
        return bytes > 64 * 1024 ? hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes)
                                 : hipSuccess;
    };
    hipError_t e;
    if constexpr (KDA) {
        if (!img) return hipErrorInvalidValue;  // KDA runs the split schedule only
    } else if (!img) {
        auto kern = prefill_bf16_kernel<DK, NSW, KDA, kFused>;
        constexpr int fused_lds = L::fBytes(KDA) + (L::vstage(kFused, KDA) ? NSW * L::VST : 0);
        if ((e = set_lds(reinterpret_cast<const void*>(kern), fused_lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(block_threads<NSW, KDA, kFused>()), fused_lds, s, B, T,
                           H, DV, NS, scale, q, k, v, alpha, beta, s_in, s_out, o, nullptr, 0,
                           (T + kC - 1) / kC, vl);
        return hipGetLastError();
    }
    // Per range of chunks: the chunk-local work of every (b, h, chunk), then
    // the recurrence through the range (state carried in state_out).
    using LP = Layout<DK, 1, KDA>;
    auto prep = prefill_bf16_kernel<DK, 1, KDA, kPrep>;
    auto chain = prefill_bf16_kernel<DK, NSW, KDA, kChain>;
    constexpr int chain_lds = (KDA ? L::cBytes : L::lBytes) + (L::vstage(kChain, KDA) ? NSW * L::VST : 0);
    if ((e = set_lds(reinterpret_cast<const void*>(prep), LP::pBytes)) != hipSuccess) return e;
    if ((e = set_lds(reinterpret_cast<const void*>(chain), chain_lds)) != hipSuccess) return e;
    const int nch = (T + kC - 1) / kC;
    const size_t head_chunk = static_cast<size_t>(B) * H * (KDA ? L::IMG : L::TIMG);  // one chunk, all heads
    const int rc = std::max(1, std::min(split_range_chunks(B * H, nch, KDA ? L::IMG : L::TIMG, KDA),
                                        static_cast<int>(std::min<size_t>(nch, img_cap / head_chunk))));
    for (int c0 = 0; c0 < nch; c0 += rc) {
        const int c1 = std::min(nch, c0 + rc);
        // chunks per chunk-local workgroup
        constexpr int kPrepGroups = prep_groups(KDA);
        const int cpw = std::max(1, (B * H * (c1 - c0) + kPrepGroups - 1) / kPrepGroups);
        const int groups_per_head = (c1 - c0 + cpw - 1) / cpw;
        if (!grid_fits(static_cast<unsigned long long>(B) * H * groups_per_head, block_threads<1, KDA, kPrep>()))
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(prep, dim3(static_cast<unsigned>(B * H * groups_per_head)),
                           dim3(block_threads<1, KDA, kPrep>()), LP::pBytes, s, B, T, H, DV, cpw, scale, q, k,
                           v, alpha, beta, s_in, s_out, o, img, c0, c1, vl);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(chain, dim3(blocks), dim3(block_threads<NSW, KDA, kChain>()), chain_lds, s, B, T,
                           H, DV, NS, scale, q, k, v, alpha, beta, c0 == 0 ? s_in : s_out, s_out, o,
                           img, c0, c1, vl);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK, bool KDA>
hipError_t dispatch_dvs(int dvs, int B, int T, int H, int DV, float scale, const bf16_t* q,
                        const bf16_t* k, const bf16_t* v, const float* alpha, const float* beta,
                        const float* s_in, float* s_out, bf16_t* o, unsigned char* img, size_t cap,
                        hipStream_t s, const Opts& vl) {
    switch (dvs) {
        case 16: return launch<DK, 1, KDA>(B, T, H, DV, scale, q, k, v, alpha, beta, s_in, s_out, o, img, cap, s, vl);
        case 32: return launch<DK, 2, KDA>(B, T, H, DV, scale, q, k, v, alpha, beta, s_in, s_out, o, img, cap, s, vl);
        default: return launch<DK, 4, KDA>(B, T, H, DV, scale, q, k, v, alpha, beta, s_in, s_out, o, img, cap, s, vl);
    }
}

template <int DK>
hipError_t dispatch_gate(int kda, int dvs, int B, int T, int H, int DV, float scale,
                         const bf16_t* q, const bf16_t* k, const bf16_t* v, const float* alpha,
                         const float* beta, const float* s_in, float* s_out, bf16_t* o,
                         unsigned char* img, size_t cap, hipStream_t s, const Opts& vl) {
    return kda ? dispatch_dvs<DK, true>(dvs, B, T, H, DV, scale, q, k, v, alpha, beta, s_in, s_out, o, img, cap, s, vl)
               : dispatch_dvs<DK, false>(dvs, B, T, H, DV, scale, q, k, v, alpha, beta, s_in, s_out, o, img, cap, s, vl);
}

template <int DK>
constexpr size_t image_bytes(int kda) {
    return static_cast<size_t>(kda ? Layout<DK, 1, true>::IMG : Layout<DK, 1, false>::TIMG);
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

// Which bf16 prefill schedule runs: the split one (chunk-local kernel + chain
// kernel, needs a workspace) or the fused one.  KDA always runs split (its
// chunk-local work is the expensive part, and a fused kernel would repeat it
// for every value slice); GDN runs fused unless GDR_SCHED_SPLIT asks.
bool prefill_bf16_split(int kda, int flags) {
    return kda != 0 || (flags & GDR_SCHED_SPLIT) != 0;
}

size_t prefill_bf16_image_bytes(int kda, int dk) {
    switch (dk) {
        case 16: return image_bytes<16>(kda);
        case 32: return image_bytes<32>(kda);
        case 64: return image_bytes<64>(kda);
        default: return image_bytes<128>(kda);
    }
}

size_t prefill_bf16_workspace(int kda, int flags, int B, int T, int H, int dk) {
    if (!prefill_bf16_split(kda, flags) || T <= 0 || B <= 0 || H <= 0) return 0;
    const size_t img = prefill_bf16_image_bytes(kda, dk);
    const int nch = (T + kC - 1) / kC;
    return static_cast<size_t>(B) * H * split_range_chunks(B * H, nch, img, kda != 0) * img;
}

hipError_t launch_prefill_bf16(int kda, int B, int T, int H, int dk, int dv, float scale,
                               const bf16_t* q, const bf16_t* k, const bf16_t* v,
                               const float* alpha, const float* beta, const float* state_in,
                               float* state_out, bf16_t* o, void* workspace, size_t workspace_bytes,
                               hipStream_t s, int flags, const Opts& vl) {
    const int dvs = prefill_bf16_slice_width(B, H, dv);
    unsigned char* img = prefill_bf16_split(kda, flags) ? static_cast<unsigned char*>(workspace) : nullptr;
    const size_t cap = workspace_bytes;
    switch (dk) {
        case 16: return dispatch_gate<16>(kda, dvs, B, T, H, dv, scale, q, k, v, alpha, beta, state_in, state_out, o, img, cap, s, vl);
        case 32: return dispatch_gate<32>(kda, dvs, B, T, H, dv, scale, q, k, v, alpha, beta, state_in, state_out, o, img, cap, s, vl);
        case 64: return dispatch_gate<64>(kda, dvs, B, T, H, dv, scale, q, k, v, alpha, beta, state_in, state_out, o, img, cap, s, vl);
        default: return dispatch_gate<128>(kda, dvs, B, T, H, dv, scale, q, k, v, alpha, beta, state_in, state_out, o, img, cap, s, vl);
    }
}

}  // namespace gdr
