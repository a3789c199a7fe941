// Fused chunked KDA prefill for gfx950, bf16 inputs, K = V = 128: one
// workgroup per (batch, head, segment) walks its chunks.  Four producer waves
// do the chunk-local work of chunk c + 1 (gate cumsum, intra-chunk
// similarities, the UT solve) while four consumer waves carry the state
// through chunk c; the chunk operands pass between them through LDS, so the
// path reads its inputs once and writes only o (and the states).
//
// Page: "Kimi K3 — открытая модель, которая обошла закрытых лидеров рынка"
// (aiblin.ru), section "Как распараллелили последовательное обновление": the
// tokens of a chunk are handled together and only the state moves from chunk
// to chunk; long prefills are split into segments whose transitions are
// computed side by side on one card and recombined exactly.  Section "Как
// хранить миллион токенов в памяти": the forget gate is clamped to [e^-5, 1]
// because inside a chunk one divides by the running product of gates; here
// that division only happens inside 16-token blocks (at most e^{80}).
//
// Chunk form (C = 64 tokens in four 16-token blocks, chunk-start state S,
// G = in-chunk inclusive cumsum of the clamped log gates per key channel):
//   A[s][r]   = beta_s sum_c k_s k_r e^{G_s - G_r}   (r < s)
//   Mqk[t][s] = sum_c q_t k_s e^{G_t - G_s}          (s <= t)
//   T = (I + A)^{-1},   K^ = K e^{G},   Q^ = Q e^{G},   K- = K e^{G_C - G}
//   Y = V - K^ S,   U = T diag(beta) Y,   O = Q^ S + Mqk U,
//   S <- Diag(e^{G_C}) S + K-^T U
// (U = T diag(beta) (V - K^ S) is the delta-rule error of the chunk.)
// Exponents: with Gin = the cumsum inside a token's own block and Tot_j the
// total of block j, e^{G_s - G_r} = e^{Gin_s} * prod_{j<k<i} e^{Tot_k} *
// e^{Tot_j - Gin_r} for s in block i > j, all three factors <= 1; inside a
// block e^{Gin_s} e^{-Gin_r} with e^{-Gin_r} <= e^{80}.
// T: D_i = (I + A_ii)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8) for the
// strictly lower N = A_ii (N^16 = 0), on fp16 MFMA; with N' = L D (L the
// strictly block-lower part of A), T = D (I + N')^{-1} and (I + N')^{-1} =
// I - N' + N'^2 - N'^3 (block nilpotent), on 16x16 MFMAs.
//
// MFMA layouts (lane l: r = l % 16, g = l / 16): "acc" = the accumulator
// layout, lane holds X[4g + e][r]; "row" = the A-operand layout of a 16-deep
// product, lane holds X[r][4g + e].  An acc-layout tile used as an A operand
// is the transpose, so mma(row X, acc Y) = XY in acc layout and
// mma(acc Y, row X) = XY in row layout; a product with the identity turns a
// row-layout tile into acc layout (a transpose).  Key channels: a lane of
// lane group g holds channels 32 s + 8 g + j of slab s (j = 0..7, one 16-byte
// load), the slot order of a 32-deep fragment; state tiles are laid out to
// match (chan4 below).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int FC = 64;     // tokens per chunk
constexpr int FK = 128;    // key channels = value columns

// LDS.  Per iteration, phase 1a: the producers do the block-local work of
// chunk c + 1 while the consumers read K^ and Q^ of chunk c and assemble its
// T diag(beta) from D and N'; phase 1b: the consumers read the rest of chunk
// c while the producers write K^, Q^, K-^T, e^{G_C}, the off-diagonal Mqk and
// N' of chunk c + 1.  What the producers write while the consumers may still
// read the previous chunk's copy (K-^T, e^{G_C}, Mqk, D, beta) is
// double-buffered by chunk parity.  Producer scratch: the block-scaled k and
// q fragments and k e^{Tot - Gin}, from phase 1a to 1b.  Each region is an
// array of its own (declared in the kernel), so that the compiler knows a
// store to one does not alias a load from another and can move loads ahead.
// The summary role has no q side: its producers stage V of chunk c + 1 in the
// Q^ and q e^{Gin} arrays instead (one per chunk parity), for consumers that
// hold two states and have no registers to prefetch it.

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// pair index of block pair (i, j), j < i
__host__ __device__ constexpr int pair_ix(int i, int j) { return i * (i - 1) / 2 + j; }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
// the gate clamp [-5, 0] as a [0, 1] clamp of g * kGateScale; kGateToLog2
// turns sums of those back into log2 units
constexpr float kGateScale = -0.2f;
constexpr float kGateToLog2 = 1.4426950408889634f / -0.2f;

// inclusive prefix sums over the 16 lanes of each DPP row (lanes r = 0..15),
// of N independent values: each step over all of them before the next, so
// that no DPP read waits on the add just before it (and no add is fused with
// the multiplication that produced its operand, which would cost a move)
template <int N>
__device__ __forceinline__ void row_scan(float (&x)[N]) {
#pragma clang fp contract(off)
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<0x111>(x[i]);   // row_shr:1
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<0x112>(x[i]);   // row_shr:2
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<0x114>(x[i]);   // row_shr:4
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<0x118>(x[i]);   // row_shr:8
}

__device__ __forceinline__ void unpack4(u32x2 w, float* x) {
    x[0] = __uint_as_float(w[0] << 16);
    x[1] = __uint_as_float(w[0] & 0xffff0000u);
    x[2] = __uint_as_float(w[1] << 16);
    x[3] = __uint_as_float(w[1] & 0xffff0000u);
}
__device__ __forceinline__ bf16x4 bits4(u32x2 w) { return __builtin_bit_cast(bf16x4, w); }
__device__ __forceinline__ bf16x4 to_bf4(f32x4 x) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (bf16)x[i];
    return r;
}
__device__ __forceinline__ f32x4 from_bf4(bf16x4 x) {
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (float)x[i];
    return r;
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[4 + i] = b[i]; }
    return r;
}
// 8 consecutive fp32 values of a lane's channel array as a fragment
__device__ __forceinline__ bf16x8 frag8(const float* x) { return frag_from<bf16>(x); }
// the packed fragment itself from here on: a fragment kept across a barrier
// is then unpacked from its bf16 words (one shift or mask a value) instead of
// its fp32 source being kept and rounded again (twice the registers, two
// operations a value)
__device__ __forceinline__ bf16x8 packed(bf16x8 x) {
    u32x4 w = __builtin_bit_cast(u32x4, x);
    asm volatile("" : "+v"(w));
    return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ f32x4 mm16(bf16x4 a, bf16x4 b) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mm16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f16x4 to_h4(f32x4 x) {
    f16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (_Float16)x[e];
    return r;
}
// 16 x 16 x 16 fp16 product, fp32 accumulation (same operand layouts as mm16)
__device__ __forceinline__ f32x4 mmh(f16x4 a, f16x4 b) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

// (I + N)^{-1} for a strictly lower 16 x 16 N (N^16 = 0), from N in row
// layout: (I - N)(I + N^2)(I + N^4)(I + N^8), the products on fp16 MFMA with
// fp32 accumulation (the operands carry 11 significant bits, the result is
// rounded to bf16 by the caller).  Returns the acc layout.  idt: the identity
// (the same pattern in both layouts).
__device__ __forceinline__ f32x4 inv_unit_lower(f32x4 nr, f16x4 idh, f32x4 idt) {
    const f16x4 nrh = to_h4(nr);
    const f16x4 nah = to_h4(mmh(nrh, idh));                       // acc layout of N (exact)
    const f32x4 n2a = mmh(nrh, nah), n2r = mmh(nah, nrh);
    const f16x4 n2ah = to_h4(n2a), n2rh = to_h4(n2r);
    const f32x4 n4a = mmh(n2rh, n2ah), n4r = mmh(n2ah, n2rh);
    const f32x4 n8a = mmh(to_h4(n4r), to_h4(n4a));
    const f32x4 y1 = mmh(to_h4(n4r + idt), to_h4(n8a + idt));     // (I + N^4)(I + N^8)
    const f32x4 y2 = mmh(to_h4(n2r + idt), to_h4(y1));            // (I + N^2)(...)
    return mmh(to_h4(idt - nr), to_h4(y2));                       // (I - N)(...)
}

__device__ __forceinline__ u32x2 ld_b64(__amdgpu_buffer_rsrc_t r, unsigned voff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, 0);
}
__device__ __forceinline__ u32x4 ld_b128(__amdgpu_buffer_rsrc_t r, unsigned voff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}
// the words of 4 consecutive bf16 values: half h of a 16-byte load
__device__ __forceinline__ u32x2 half_of(u32x4 v, int h) { return h ? u32x2{v[2], v[3]} : u32x2{v[0], v[1]}; }

// Channel order.  A producer lane (g, r) loads 8 consecutive key channels of
// each 32-channel slab s4: 32 s4 + 8 g + j, j = 0..7, which is also slot j of
// the lane's 32-deep MFMA fragment.  The state's accumulator tiles follow:
// tile ct, lane group g, element e holds key channel chan4(ct, g) + e, so that
// two stacked tiles (2 s4, 2 s4 + 1) give the same fragment slots.
__device__ __forceinline__ int chan4(int m, int g) { return 32 * (m >> 1) + 8 * g + 4 * (m & 1); }

}  // namespace



// The LDS regions of a workgroup, each an array of its own so that the
// compiler knows a store to one does not alias a load from another; declared
// in the kernel (NQ, NM: elements of the q-side and Mqk regions, 1 where a
// kernel runs no output pass).
#define KDA_FUSED_LDS(NQ, NM)                                                                     \
    __shared__ bf16x8 hK[4 * 4 * 64];                /* K^ fragments [4 blk][4 slab][64 lanes] */ \
    __shared__ bf16x8 hQ[NQ];                        /* Q^ fragments [4 blk][4 slab][64] */       \
    __shared__ bf16x4 hKb[2 * 4 * 8 * 64];           /* K- tiles, transposed [2][4 blk][8 m][64] */ \
    __shared__ bf16x4 hT[4 * 4 * 64];                /* T diag(beta), row layout [4 ti][4 j][64] */ \
    __shared__ bf16x4 hM[NM];                        /* Mqk, row layout [2][4 ti][4 j][64] */     \
    __shared__ __attribute__((aligned(16))) float hG[2 * FK];        /* e^{G_C} [2][128] */      \
    __shared__ __attribute__((aligned(16))) float sETot[4 * FK];     /* e^{Tot} per block */     \
    __shared__ bf16x8 sKend[3 * 4 * 64];             /* k e^{Tot - Gin} [3 blk][4 slab][64] */    \
    __shared__ float sBeta[2 * 64];                  /* beta [2][64] */                           \
    __shared__ bf16x4 sD[2 * 4 * 64];                /* D_i acc layout [2][4][64] */              \
    __shared__ f32x4 sNa[6 * 64];                    /* N'_ij acc layout [6 pairs][64] */         \
    __shared__ bf16x4 sNr[6 * 64];                   /* N'_ij row layout [6 pairs][64] */         \
    __shared__ __attribute__((aligned(16))) float sFac[4 * 2 * FK];  /* e^{G_b}, e^{G_C - G_b} per wave */ \
    __shared__ bf16x8 sKd[4 * 4 * 64];               /* k e^{Gin} fragments [4 blk][4 slab][64] */ \
    __shared__ bf16x8 sQd[NQ];                       /* q e^{Gin} fragments [4 blk][4 slab][64] */

constexpr int kFusedNQ = 4 * 4 * 64;
constexpr int kFusedNM = 2 * 4 * 4 * 64;

// The output pass: segments from their start states, with output.
template <bool GATE>
__global__ __launch_bounds__(512, 1) void kda_fused_kernel(FusedParams p) {
    KDA_FUSED_LDS(kFusedNQ, kFusedNM)
    constexpr bool SUMMARY = false, FIRST = false;
    const int blk = (int)blockIdx.x;
#include "kda_fused_body.inc"
}

// The first pass of a segmented call: segment 0 with its output (the first
// po.B * po.H workgroups) beside the summaries of segments 1 .. n_seg - 2.
template <bool GATE_OUT>
__global__ __launch_bounds__(512, 1) void kda_fused_first_kernel(FusedParams po, FusedParams ps) {
    KDA_FUSED_LDS(kFusedNQ, kFusedNM)
    const int n_out = po.B * po.H * po.seg_count;
    if ((int)blockIdx.x < n_out) {
        constexpr bool SUMMARY = false, GATE = GATE_OUT, FIRST = true;
        const FusedParams& p = po;
        const int blk = (int)blockIdx.x;
#include "kda_fused_body.inc"
    } else {
        constexpr bool SUMMARY = true, GATE = false, FIRST = true;
        const FusedParams& p = ps;
        const int blk = (int)blockIdx.x - n_out;
#include "kda_fused_body.inc"
    }
}

bool fused_variant_exists(int dtype, int K, int V) { return dtype == 1 && K == 128 && V == 128; }

hipError_t launch_fused_first(const FusedParams& po, const FusedParams& ps, int grid, hipStream_t stream) {
    if (grid <= 0) return hipSuccess;
    if (po.gate) hipLaunchKernelGGL((kda_fused_first_kernel<true>), dim3(grid), dim3(512), 0, stream, po, ps);
    else hipLaunchKernelGGL((kda_fused_first_kernel<false>), dim3(grid), dim3(512), 0, stream, po, ps);
    return hipGetLastError();
}

hipError_t launch_fused(const FusedParams& p, int grid, hipStream_t stream) {
    if (grid <= 0) return hipSuccess;
    if (p.gate) hipLaunchKernelGGL((kda_fused_kernel<true>), dim3(grid), dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((kda_fused_kernel<false>), dim3(grid), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kda
