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

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

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
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
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



template <bool SUMMARY, bool GATE>
__global__ __launch_bounds__(512, 1) void kda_fused_kernel(FusedParams p) {
    constexpr int NQ = SUMMARY ? 1 : 4 * 4 * 64;       // the summary pass has no q: 1-element stand-ins
    constexpr int NM = SUMMARY ? 1 : 2 * 4 * 4 * 64;
    __shared__ bf16x8 hK[4 * 4 * 64];                   // K^ fragments [4 blk][4 slab][64 lanes]
    __shared__ bf16x8 hQ[NQ];                           // Q^ fragments [4 blk][4 slab][64]
    __shared__ bf16x4 hKb[2 * 4 * 8 * 64];              // K- tiles, transposed [2][4 blk][8 m][64]
    __shared__ bf16x4 hT[4 * 4 * 64];                   // T diag(beta), row layout [4 ti][4 j][64]
    __shared__ bf16x4 hM[NM];                           // Mqk, row layout [2][4 ti][4 j][64]
    __shared__ __attribute__((aligned(16))) float hG[2 * FK];        // e^{G_C} [2][128]
    __shared__ __attribute__((aligned(16))) float sETot[4 * FK];     // e^{Tot} of each block [4][128]
    __shared__ bf16x8 sKend[3 * 4 * 64];                // k e^{Tot - Gin} [3 blk][4 slab][64]
    __shared__ float sBeta[2 * 64];                     // beta [2][64]
    __shared__ bf16x4 sD[2 * 4 * 64];                   // D_i acc layout [2][4][64]
    __shared__ f32x4 sNa[6 * 64];                       // N'_ij acc layout [6 pairs][64]
    __shared__ bf16x4 sNr[6 * 64];                      // N'_ij row layout [6 pairs][64]
    __shared__ __attribute__((aligned(16))) float sFac[4 * 2 * FK];  // per producer wave: e^{G_b}, e^{G_C - G_b}
    __shared__ bf16x8 sKd[4 * 4 * 64];                  // k e^{Gin} fragments [4 blk][4 slab][64]
    __shared__ bf16x8 sQd[NQ];                          // q e^{Gin} fragments [4 blk][4 slab][64]

    const int tid = threadIdx.x;
    // the wave index is uniform across the wave: in a scalar register, so
    // that branches on it are scalar branches
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lg = l >> 4, lr = l & 15;
    const bool producer = w < 4;
    const int pw = w;          // producer wave = the 16-token block of the chunk it prepares
    const int cw = w - 4;      // consumer wave: value columns [32 cw, 32 cw + 32)

    const int nseg_here = SUMMARY ? p.n_seg - 1 : p.n_seg;
    const int seg = blockIdx.x % nseg_here;
    const int bh = blockIdx.x / nseg_here;
    const int b = bh / p.H, h = bh % p.H;
    const int BH = p.B * p.H;
    const int n_chunks = (p.T + FC - 1) / FC;
    const int c_begin = seg * p.cps;
    const int c_end = min(c_begin + p.cps, n_chunks);
    const unsigned rowK = (unsigned)p.H * FK * 2u;    // bytes between tokens of q, k, g, v, o
    const unsigned rowB = (unsigned)p.H * 2u;
    if (c_begin >= c_end) return;

    // identity tile: lane (g, r) slot e = [4g + e == r] (as a 16-deep operand,
    // in either layout)
    bf16x4 ident;
    f32x4 identf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        identf[e] = (4 * lg + e == lr) ? 1.f : 0.f;
        ident[e] = (bf16)identf[e];
    }

    // one chunk's token rows of a [B,T,H,128] bf16 tensor; rows past the
    // sequence read as zeros (and stores there are dropped)
    // A chunk past the segment gets an empty resource: its loads return zero
    // and touch no memory, so that every load can be issued unconditionally
    // (the compiler then knows how many loads are in flight at each wait).
    auto chunk_rows = [&](int ci) { return ci < c_end ? min(FC, p.T - ci * FC) : 0; };
    auto chunk_rsrc = [&](const void* base, int ci) {
        const int nt = chunk_rows(ci);
        const size_t row0 = ((size_t)b * p.T + (size_t)ci * FC) * p.H + h;
        return make_rsrc_n(reinterpret_cast<const bf16*>(base) + row0 * FK, nt > 0 ? (unsigned)(nt - 1) * rowK + FK * 2u : 0u);
    };

    if (producer) {
        // ============================================================== producers
        u32x4 kr[4], qr[4], gr[4];             // raw inputs of the chunk being prepared, a slab each
        unsigned short braw = 0;
        bf16x8 kdb[4], kib[4];                  // k e^{Gin}, k e^{-Gin}, 32-deep fragments (1a -> 1b)
        const unsigned voff = (unsigned)(16 * pw + lr) * rowK + (unsigned)(16 * lg);

        // the raw loads of a chunk, per group of channel groups m
        auto load_gkq = [&](int ci, int hv) {
            const __amdgpu_buffer_rsrc_t rg = chunk_rsrc(p.g, ci);
            const __amdgpu_buffer_rsrc_t rk = chunk_rsrc(p.k, ci);
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) gr[2 * hv + sh] = ld_b128(rg, voff + 64u * (2 * hv + sh));
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) kr[2 * hv + sh] = ld_b128(rk, voff + 64u * (2 * hv + sh));
            if (!SUMMARY) {
                const __amdgpu_buffer_rsrc_t rq = chunk_rsrc(p.q, ci);
#pragma unroll
                for (int sh = 0; sh < 2; ++sh) qr[2 * hv + sh] = ld_b128(rq, voff + 64u * (2 * hv + sh));
            }
            if (hv == 0) {
                const int nt = chunk_rows(ci);
                const __amdgpu_buffer_rsrc_t rb = make_rsrc_n(
                    reinterpret_cast<const bf16*>(p.beta) + ((size_t)b * p.T + (size_t)ci * FC) * p.H + h,
                    nt > 0 ? (unsigned)(nt - 1) * rowB + 2u : 0u);
                braw = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)((unsigned)(16 * pw + lr) * rowB), 0, 0);
            }
        };

        // phase 1a of chunk ci: the work local to the wave's block.  The next
        // chunk's loads are issued as this chunk's raw values are used up.
        auto phase_a = [&](int ci) {
            const int buf = ci & 1;
            const float bt = __uint_as_float((unsigned)braw << 16);
            float* etot = sETot + pw * FK;
            if (lg == 0) sBeta[buf * 64 + 16 * pw + lr] = bt;
            f32x4 at = {0.f, 0.f, 0.f, 0.f}, mt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int hv = 0; hv < 2; ++hv) {
                // Gin: the block's inclusive sums of the gate clamped to [-5, 0],
                // scanned as clamp(-g / 5) in [0, 1] (one multiply with the
                // output clamp) and scaled to log2 units before the exponentials
                float gin[16];
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    float x[4];
                    unpack4(half_of(gr[2 * hv + (mm >> 1)], mm & 1), x);
#pragma unroll
                    for (int e = 0; e < 4; ++e) gin[4 * mm + e] = __builtin_amdgcn_fmed3f(x[e] * kGateScale, 0.f, 1.f);
                }
                row_scan(gin);
#pragma unroll
                for (int i = 0; i < 16; ++i) gin[i] *= kGateToLog2;
                float kd[16], ki[16], qd[16], e1[16];
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    float kx[4], qx[4];
                    unpack4(half_of(kr[2 * hv + (mm >> 1)], mm & 1), kx);
                    if (!SUMMARY) unpack4(half_of(qr[2 * hv + (mm >> 1)], mm & 1), qx);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 4 * mm + e;
                        e1[i] = fast_exp2(gin[i]);               // e^{Gin} <= 1
                        const float e2 = fast_exp2(-gin[i]);    // e^{-Gin} <= e^{80}
                        kd[i] = kx[e] * e1[i];
                        ki[i] = kx[e] * e2;
                        if (!SUMMARY) qd[i] = qx[e] * e1[i];
                    }
                }
                load_gkq(ci + 1, hv);
                // the block's last token holds e^{Tot}, the block total
                if (lr == 15) {
#pragma unroll
                    for (int mm = 0; mm < 4; ++mm)
                        *reinterpret_cast<f32x4*>(&etot[chan4(4 * hv + mm, lg)]) =
                            f32x4{e1[4 * mm], e1[4 * mm + 1], e1[4 * mm + 2], e1[4 * mm + 3]};
                }
#pragma unroll
                for (int sh = 0; sh < 2; ++sh) {
                    const int s4 = 2 * hv + sh;
                    kdb[s4] = frag8(&kd[8 * sh]);
                    sKd[(pw * 4 + s4) * 64 + l] = kdb[s4];          // for the off-diagonal blocks
                    kib[s4] = frag8(&ki[8 * sh]);
                    // A_ii transposed (lane (g, s): A[s][4g + e]) and Mqk_ii in
                    // row layout (lane (g, t): Mqk[t][4g + e]), unscaled
                    at = mma(at, kib[s4], kdb[s4]);
                    if (!SUMMARY) {
                        const bf16x8 qf = frag8(&qd[8 * sh]);
                        sQd[(pw * 4 + s4) * 64 + l] = qf;        // q e^{Gin}, for phase 1b
                        mt = mma(mt, kib[s4], qf);
                    }
                }
                // k e^{Tot - Gin} for the off-diagonal blocks of the later
                // blocks: e^{Tot} broadcast from the row's last lane
                if (pw < 3) {
#pragma unroll
                    for (int sh = 0; sh < 2; ++sh) {
                        float ke[8];
#pragma unroll
                        for (int c = 0; c < 8; ++c) ke[c] = ki[8 * sh + c] * dpp_f<0x15F>(e1[8 * sh + c]);   // row_newbcast:15
                        sKend[(pw * 4 + 2 * hv + sh) * 64 + l] = frag8(ke);
                    }
                }
            }
            if (!SUMMARY) {
                // Mqk_ii: s <= t
#pragma unroll
                for (int e = 0; e < 4; ++e) mt[e] = (4 * lg + e <= lr) ? mt[e] : 0.f;
                hM[((buf * 4 + pw) * 4 + pw) * 64 + l] = to_bf4(mt);
            }
            // D_pw = (I + A_ii)^{-1}, A_ii = the r < s part, row s scaled by beta_s
            {
                f32x4 nr;
#pragma unroll
                for (int e = 0; e < 4; ++e) nr[e] = (4 * lg + e < lr) ? bt * at[e] : 0.f;
                const bf16x4 db = to_bf4(inv_unit_lower(nr, to_h4(identf), identf));
                sD[(buf * 4 + pw) * 64 + l] = db;
            }
        };

        // phase 1b of chunk ci: block-prefix factors, K^ / Q^ / K-, the
        // off-diagonal blocks of A and Mqk, N'
        auto phase_b = [&](int ci) {
            const int buf = ci & 1;
            // e^{G_b} (G_b: the gate sum before the block) and e^{G_C - G_b}
            // (the rest of the chunk, the block included), two channels a lane,
            // into the wave's table; wave 0's second factor is e^{G_C}
            float* fac = sFac + pw * 2 * FK;
            {
                float2 t[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) t[j] = *reinterpret_cast<const float2*>(&sETot[j * FK + 2 * l]);
                float2 eg = make_float2(1.f, 1.f), ec = make_float2(1.f, 1.f);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // selects, not branches: the four loads are waited for once
                    const bool pre = j < pw;
                    eg.x *= pre ? t[j].x : 1.f;
                    eg.y *= pre ? t[j].y : 1.f;
                    ec.x *= pre ? 1.f : t[j].x;
                    ec.y *= pre ? 1.f : t[j].y;
                }
                *reinterpret_cast<float2*>(&fac[2 * l]) = eg;
                *reinterpret_cast<float2*>(&fac[FK + 2 * l]) = ec;
                if (pw == 0) *reinterpret_cast<float2*>(&hG[buf * FK + 2 * l]) = ec;
            }
            wave_lds_sync();
            // K^ = k e^{G}, Q^ = q e^{G} and K- = k e^{G_C - G}: the block's
            // stored factors times the block-prefix ones
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                bf16x8 qf;
                if (!SUMMARY) qf = sQd[(pw * 4 + s4) * 64 + l];
                float xk[8], xq[8];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int m = 2 * s4 + hf;
                    const f32x4 egb = *reinterpret_cast<const f32x4*>(&fac[chan4(m, lg)]);
                    const f32x4 ecb = *reinterpret_cast<const f32x4*>(&fac[FK + chan4(m, lg)]);
                    bf16x4 kb4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        xk[4 * hf + e] = (float)kdb[s4][4 * hf + e] * egb[e];
                        if (!SUMMARY) xq[4 * hf + e] = (float)qf[4 * hf + e] * egb[e];
                        kb4[e] = (bf16)((float)kib[s4][4 * hf + e] * ecb[e]);
                    }
                    hKb[((buf * 4 + pw) * 8 + m) * 64 + l] = to_bf4(mm16(kb4, ident));
                }
                hK[(pw * 4 + s4) * 64 + l] = frag8(xk);
                if (!SUMMARY) hQ[(pw * 4 + s4) * 64 + l] = frag8(xq);
            }
            // off-diagonal blocks (i, j), j < i, shared out over the waves:
            // row operands k e^{Gin} and q e^{Gin} of block i, column operand
            // k e^{Tot - Gin} of block j times prod_{j<m<i} e^{Tot_m} (one
            // scaling serves A and Mqk); then N'_ij = A_ij D_j in both layouts
            auto pair = [&](int i, int j) {
                f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    bf16x8 ke = sKend[(j * 4 + s4) * 64 + l];
                    if (i - j > 1) {
                        float kf[8];
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            const int m = 2 * s4 + hf;
                            f32x4 f = *reinterpret_cast<const f32x4*>(&sETot[(j + 1) * FK + chan4(m, lg)]);
                            if (i - j > 2) f = f * *reinterpret_cast<const f32x4*>(&sETot[(j + 2) * FK + chan4(m, lg)]);
#pragma unroll
                            for (int e = 0; e < 4; ++e) kf[4 * hf + e] = (float)ke[4 * hf + e] * f[e];
                        }
                        ke = frag8(kf);
                    }
                    accA = mma(accA, ke, sKd[(i * 4 + s4) * 64 + l]);
                    if (!SUMMARY) accM = mma(accM, ke, sQd[(i * 4 + s4) * 64 + l]);
                }
                if (!SUMMARY) hM[((buf * 4 + i) * 4 + j) * 64 + l] = to_bf4(accM);   // row layout (row t = lane)
                const float bi = sBeta[buf * 64 + 16 * i + lr];
                const bf16x4 ar = to_bf4(accA * bi);            // row layout of A_ij (row s = lane)
                const bf16x4 dj = sD[(buf * 4 + j) * 64 + l];
                sNa[pair_ix(i, j) * 64 + l] = mm16(ar, dj);
                sNr[pair_ix(i, j) * 64 + l] = to_bf4(mm16(dj, ar));
            };
            if (pw == 0) {
                pair(3, 0);
            } else if (pw == 1) {
                pair(2, 0);
            } else if (pw == 2) {
                pair(3, 1);
            } else {
                pair(3, 2);
                pair(2, 1);
                pair(1, 0);
            }
        };

        // prologue: chunk c_begin through phases 1a and 1b; then iteration ci
        // prepares ci + 1 while the consumers run ci
        load_gkq(c_begin, 0);
        load_gkq(c_begin, 1);
        phase_a(c_begin);
        __syncthreads();
        phase_b(c_begin);
        __syncthreads();
        for (int ci = c_begin; ci + 1 < c_end; ++ci) {
            phase_a(ci + 1);
            __syncthreads();
            phase_b(ci + 1);
            __syncthreads();
        }
        __syncthreads();
        __syncthreads();
        return;
    }

    // ================================================================== consumers
    // S[grp][jt][ct]: rows chan4(ct, g) + e, column 32 cw + 16 jt + r of group
    // grp (output pass: the state; summary pass: 0 = local state L, 1 = the
    // transition P, carried as extra columns with identity start and no values)
    constexpr int NG = SUMMARY ? 2 : 1;
    f32x4 S[NG][2][8];
#pragma unroll
    for (int grp = 0; grp < NG; ++grp)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            const int col = 32 * cw + 16 * jt + lr;
            const float* src = nullptr;
            if (!SUMMARY) {
                if (seg == 0) src = p.s0 ? p.s0 + (size_t)bh * FK * FK : nullptr;
                else src = p.seg_init + ((size_t)(seg - 1) * BH + bh) * FK * FK;
            }
#pragma unroll
            for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = chan4(ct, lg) + e;
                    float v0 = 0.f;
                    if (src) v0 = src[(size_t)row * FK + col];
                    else if (SUMMARY && grp == 1) v0 = (row == col) ? 1.f : 0.f;
                    S[grp][jt][ct][e] = v0;
                }
        }
    const bf16x4 z4 = to_bf4(f32x4{0.f, 0.f, 0.f, 0.f});

    // the wave's value columns of a chunk, row layout: lane (g, t) holds
    // V[16 ti + t][32 cw + 16 jt + 4 g + e]; loaded a chunk ahead
    u32x2 vq[4][2];
    // the output gate of the chunk being finished, same layout as o (one token
    // per lane, four consecutive columns), loaded in phase 1a
    u32x2 zq[4][2];
    auto load_zq = [&](int ci) {
        const int nt = chunk_rows(ci);
        const __amdgpu_buffer_rsrc_t rz = make_rsrc_n(
            reinterpret_cast<const bf16*>(p.gate) + (((size_t)b * p.T + (size_t)ci * FC) * p.H + h) * FK,
            nt > 0 ? (unsigned)(nt - 1) * rowK + FK * 2u : 0u);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
                zq[ti][jt] = ld_b64(rz, (unsigned)(16 * ti + lr) * rowK + (unsigned)(2 * (32 * cw + 16 * jt + 4 * lg)));
    };
    auto load_vq = [&](int ci) {
        const __amdgpu_buffer_rsrc_t rv = chunk_rsrc(p.v, ci);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
                vq[ti][jt] = ld_b64(rv, (unsigned)(16 * ti + lr) * rowK + (unsigned)(2 * (32 * cw + 16 * jt + 4 * lg)));
    };

    // T diag(beta), T = D (I + N')^{-1} assembled from D_i = (I + A_ii)^{-1}
    // and N'_ij = A_ij D_j (both from the producers): T_ii = D_i and
    // T_ij = D_i M'_ij with M' = (I + N')^{-1}:
    //   M'_{i,i-1} = -N'_{i,i-1},  M'_20 = N'_21 N'_10 - N'_20,
    //   M'_31 = N'_32 N'_21 - N'_31,  M'_30 = N'_31 N'_10 - N'_30 - N'_32 M'_20,
    // written in row layout.  The ten tiles are shared out so that each wave's
    // chain of dependent products is at most seven long.
    auto t_tiles = [&](int ci) {
        const int buf = ci & 1;
        auto drow = [&](int i) { return to_bf4(mm16(sD[(buf * 4 + i) * 64 + l], ident)); };   // row layout of D_i
        auto na = [&](int i, int j) { return sNa[pair_ix(i, j) * 64 + l]; };
        auto nr = [&](int i, int j) { return sNr[pair_ix(i, j) * 64 + l]; };
        auto diag = [&](int i, bf16x4 dr) {
            const float bt = sBeta[buf * 64 + 16 * i + lr];
            bf16x4 dg;
#pragma unroll
            for (int e = 0; e < 4; ++e) dg[e] = (bf16)((4 * lg + e == lr) ? bt : 0.f);
            hT[(i * 4 + i) * 64 + l] = to_bf4(mm16(dg, dr));             // D_i diag(beta_i)
        };
        auto off = [&](int i, int j, f32x4 mp, bf16x4 dr) {           // mp = M'_ij, acc layout
            const float bj = sBeta[buf * 64 + 16 * j + lr];           // column lr of block j
            hT[(i * 4 + j) * 64 + l] = to_bf4(mm16(to_bf4(mp * bj), dr));
        };
        auto m20 = [&]() { return mm16(nr(2, 1), to_bf4(na(1, 0)), -na(2, 0)); };
        if (cw == 0) {
            diag(0, drow(0));
            const f32x4 m30 = mm16(nr(3, 1), to_bf4(na(1, 0)), -na(3, 0)) - mm16(nr(3, 2), to_bf4(m20()));
            off(3, 0, m30, drow(3));
        } else if (cw == 1) {
            const bf16x4 d1 = drow(1);
            diag(1, d1);
            off(1, 0, -na(1, 0), d1);
            off(2, 0, m20(), drow(2));
        } else if (cw == 2) {
            const bf16x4 d2 = drow(2);
            diag(2, d2);
            off(2, 1, -na(2, 1), d2);
            off(3, 1, mm16(nr(3, 2), to_bf4(na(2, 1)), -na(3, 1)), drow(3));
        } else {
            const bf16x4 d3 = drow(3);
            diag(3, d3);
            off(3, 2, -na(3, 2), d3);
        }
    };

    // Y = V - K^ S, as 32-deep fragments (blocks 2 ks, 2 ks + 1); in the
    // output pass also the inter-chunk part of the output, Q^ S, computed
    // transposed ((Q^ S)^T = S^T Q^^T: the state fragments as the A operand)
    // so that its accumulator holds one token per lane and four consecutive
    // value columns, the layout of the stores
    auto consume_a = [&](int ci, f32x4 (&St)[2][8], bool with_v, bf16x8 (&yb)[2][2], f32x4 (&accO)[4][2]) {
        const int buf = ci & 1;
        f32x4 accY[4][2];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                accY[ti][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (!SUMMARY) accO[ti][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            bf16x8 sb[2];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) sb[jt] = frag_from_tiles<bf16>(St[jt][2 * s4], St[jt][2 * s4 + 1]);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                const bf16x8 a = hK[(ti * 4 + s4) * 64 + l];
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) accY[ti][jt] = mma(accY[ti][jt], a, sb[jt]);
                if (!SUMMARY) {
                    const bf16x8 aq = hQ[(ti * 4 + s4) * 64 + l];
#pragma unroll
                    for (int jt = 0; jt < 2; ++jt) accO[ti][jt] = mma(accO[ti][jt], sb[jt], aq);
                }
            }
        }
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                // V transposed to acc layout (rows = tokens, lane = column)
                if (with_v) accY[ti][jt] = mm16(bits4(vq[ti][jt]), ident) - accY[ti][jt];
                else accY[ti][jt] = -accY[ti][jt];
            }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) yb[ks][jt] = frag_from_tiles<bf16>(accY[2 * ks][jt], accY[2 * ks + 1][jt]);
    };

    // U = T diag(beta) Y, O = Q^ S + Mqk U (stored), then the state update
    auto consume_b = [&](int ci, f32x4 (&St)[2][8], const bf16x8 (&yb)[2][2], bool out, f32x4 (&accO4)[4][2]) {
        const int buf = ci & 1;
        f32x4 U[4][2];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) U[ti][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (2 * ks <= ti) {
                    const bf16x8 a = cat8(hT[(ti * 4 + 2 * ks) * 64 + l],
                                          (2 * ks + 1 <= ti) ? hT[(ti * 4 + 2 * ks + 1) * 64 + l] : z4);
#pragma unroll
                    for (int jt = 0; jt < 2; ++jt) U[ti][jt] = mma(U[ti][jt], a, yb[ks][jt]);
                }
            }
        }
        bf16x8 ub[2][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) ub[ks][jt] = frag_from_tiles<bf16>(U[2 * ks][jt], U[2 * ks + 1][jt]);
        if (out) {
            const int t0 = ci * FC;
            const int nt = min(FC, p.T - t0);
            const size_t row0 = ((size_t)b * p.T + t0) * p.H + h;
            const unsigned span = (unsigned)(nt - 1) * rowK + FK * 2u;
            const __amdgpu_buffer_rsrc_t ro = make_rsrc_n(reinterpret_cast<bf16*>(p.o) + row0 * FK, span);
            // O^T += U^T Mqk^T per 16-token tile (the U fragments as the A
            // operand), rounded to bf16 and stored 8 bytes a lane (4 columns of
            // one token)
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                f32x4 (&accO)[2] = accO4[ti];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (2 * ks <= ti) {
                        const bf16x8 a = cat8(hM[((buf * 4 + ti) * 4 + 2 * ks) * 64 + l],
                                              (2 * ks + 1 <= ti) ? hM[((buf * 4 + ti) * 4 + 2 * ks + 1) * 64 + l] : z4);
#pragma unroll
                        for (int jt = 0; jt < 2; ++jt) accO[jt] = mma(accO[jt], ub[ks][jt], a);
                    }
                }
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    bf16x4 o4 = to_bf4(accO[jt]);
                    const unsigned voff = (unsigned)(16 * ti + lr) * rowK + (unsigned)(2 * (32 * cw + 16 * jt + 4 * lg));
                    if (GATE) {
                        // output gate: o (rounded to bf16) * sigmoid(z), rounded once more
                        float z[4];
                        unpack4(zq[ti][jt], z);
#pragma unroll
                        for (int e = 0; e < 4; ++e) o4[e] = (bf16)((float)o4[e] * sigmoidf_fast(z[e]));
                    }
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o4), ro, (int)voff, 0, 0);
                }
            }
        }
        // S <- Diag(e^{G_C}) S + K-^T U
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const f32x4 gm = *reinterpret_cast<const f32x4*>(&hG[buf * FK + chan4(ct, lg)]);
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) St[jt][ct] = St[jt][ct] * gm;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 a = cat8(hKb[((buf * 4 + 2 * ks) * 8 + ct) * 64 + l],
                                      hKb[((buf * 4 + 2 * ks + 1) * 8 + ct) * 64 + l]);
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) St[jt][ct] = mma(St[jt][ct], a, ub[ks][jt]);
            }
        }
    };

    // the producers' prologue: two phases
    if (!SUMMARY) load_vq(c_begin);
    __syncthreads();
    __syncthreads();
    // Phase 1a may read K^ and V of chunk ci, phase 1b all of its hand-off
    // (the rest is written by the producers in 1a).  The summary pass runs the
    // first half of its local-state columns in 1a, the rest in 1b.
    for (int ci = c_begin; ci < c_end; ++ci) {
        bf16x8 yb[2][2];
        f32x4 accO[4][2];
        if (SUMMARY) {
            // two states to carry: V is loaded in the phase that reads it
            bf16x8 yp[2][2];
            load_vq(ci);
            t_tiles(ci);
            __builtin_amdgcn_sched_barrier(0);
            consume_a(ci, S[0], true, yb, accO);
            __builtin_amdgcn_sched_barrier(0);     // one column group's temporaries at a time
            consume_a(ci, S[NG - 1], false, yp, accO);
            __syncthreads();
            consume_b(ci, S[0], yb, false, accO);
            __builtin_amdgcn_sched_barrier(0);
            consume_b(ci, S[NG - 1], yp, false, accO);
            __syncthreads();
        } else {
            t_tiles(ci);
            consume_a(ci, S[0], true, yb, accO);
            if (GATE) load_zq(ci);
            __syncthreads();
            consume_b(ci, S[0], yb, true, accO);
            load_vq(ci + 1);
            __syncthreads();
        }
    }

    // final state of this segment
#pragma unroll
    for (int grp = 0; grp < NG; ++grp) {
        float* dst = nullptr;
        if (!SUMMARY) {
            if (seg == p.n_seg - 1 && p.sT) dst = p.sT + (size_t)bh * FK * FK;
        } else {
            dst = (grp == 0 ? p.wsL : p.wsP) + ((size_t)seg * BH + bh) * FK * FK;
        }
        if (!dst) continue;
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            const int col = 32 * cw + 16 * jt + lr;
#pragma unroll
            for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(size_t)(chan4(ct, lg) + e) * FK + col] = S[grp][jt][ct][e];
        }
    }
}

bool fused_variant_exists(int dtype, int K, int V) { return dtype == 1 && K == 128 && V == 128; }

hipError_t launch_fused(const FusedParams& p, bool summary, int grid, hipStream_t stream) {
    if (grid <= 0) return hipSuccess;
    if (summary) hipLaunchKernelGGL((kda_fused_kernel<true, false>), dim3(grid), dim3(512), 0, stream, p);
    else if (p.gate) hipLaunchKernelGGL((kda_fused_kernel<false, true>), dim3(grid), dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((kda_fused_kernel<false, false>), dim3(grid), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kda
