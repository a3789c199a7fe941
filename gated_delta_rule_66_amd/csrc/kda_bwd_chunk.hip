// Chunk-form backward of the KDA prefill for gfx950: the gradients of one
// 64-token chunk with respect to q, k, v, g and beta, all chunks at once.
//
// The pages give no backward.  This is the chain rule applied to the chunk
// form of the forward (page "Kimi K3 — открытая модель, которая обошла
// закрытых лидеров рынка" (aiblin.ru), section "Как распараллелили
// последовательное обновление": the tokens of a chunk are handled together
// and only the state passes from chunk to chunk).  Per chunk, with S the
// state before it, G the in-chunk inclusive cumsum of the clamped log-gates
// and e^{G_C} the chunk total, the forward computes
//   Ak[s,r] = sum_c k_s k_r e^{G_s - G_r}  (r < s),  A = diag(beta) Ak
//   M[t,s]  = sum_c q_t k_s e^{G_t - G_s}  (s <= t)
//   W = (I + A)^{-1} diag(beta) (K e^{G}),  U~ = (I + A)^{-1} diag(beta) V
//   U = U~ - W S,  O = (Q e^{G}) S + M U,  S' = Diag(e^{G_C}) S + (K e^{G_C - G})^T U.
// Given dO, dL/dS' (from the reverse state pass, which also hands over
// dU = M^T dO + (K e^{G_C - G}) dL/dS'):
//   D    = tril(dO U^T)                    dQh = dO S^T
//   dKb  = U dS'^T                         dW  = -dU S^T
//   (I + A)^T [dBv | dBk] = [dU | dW]      (back substitution)
//   dv   = diag(beta) dBv                  dKh = diag(beta) dBk
//   E    = -tril_strict(dBv U~^T + dBk W^T),  Et = diag(beta) E
//   dbeta_s = dBv_s . v_s + dBk_s . (k_s e^{G_s}) + sum_r E[s,r] Ak[s,r]
//   X1[s] = sum_{r<s} Et[s,r] k_r e^{G_s - G_r}    X2[r] = sum_{s>r} Et[s,r] k_s e^{G_s - G_r}
//   Y1[t] = sum_{s<=t} D[t,s] k_s e^{G_t - G_s}    Y2[s] = sum_{t>=s} D[t,s] q_t e^{G_t - G_s}
//   dq   = dQh e^{G} + Y1
//   dk   = dKh e^{G} + X1 + X2 + Y2 + dKb e^{G_C - G}
//   dG   = dQh q e^{G} + dKh k e^{G} - dKb k e^{G_C - G} + k (X1 - X2 - Y2) + q Y1
//   dG_C += e^{G_C} rowsum(S * dS') + sum_s dKb_s k_s e^{G_C - G_s}
//   dg_t = [-5 <= g_t <= 0] sum_{t' >= t} dG_{t'}
// Every gated product runs per 16-token sub-chunk pair with sub-chunk
// reference gates R_j (the cumsum before sub-chunk j), so that every
// exponent is either <= 0 or within a sub-chunk (at most 80 at the clamp
// floor), as in the forward.
//
// Three kernels, one workgroup (8 waves) per (b, h, chunk):
//   vside  : U, D, dQh, dKb, dW and the e^{G_C} rowsum term (value-side products)
//   ksolve : Ak, the back substitution (blocked, fp32 MFMA), dv, dKh, Et, dbeta
//   kgrad  : the gated products and dq, dk, dg (fp32 throughout)
// Each issues all of a phase's global loads before it waits on any of them.
// Intermediates live in an fp32 workspace, one slot per chunk.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = kChunk;

constexpr int cmax2(int a, int b) { return a > b ? a : b; }

// 4 fp32 values stored as 4 elements of T
template <typename T>
__device__ __forceinline__ void st4(T* dst, f32x4 x) {
    typename Frag4Of<T>::type f = frag4_from<T>(x);
    *reinterpret_cast<typename Frag4Of<T>::type*>(dst) = f;
}

// 16-byte pieces: every global load of a staging phase is issued before any
// of them is waited on, then the pieces go to LDS
// pieces of the [C][N] token tile (head h, tokens t0 ..) of a [B, T, H, N]
// tensor; rows from nt on (and a null source) are zero
// (buffer loads over exactly the valid rows: rows past nt read as zeros)
template <typename T, int N, int NP, int NT = 256>
__device__ __forceinline__ void load_tok_pieces(const void* src, const BwdParams& p, int b, int h, int t0, int nt,
                                                uint4 (&r)[NP], int tid) {
    constexpr int PR = N * (int)sizeof(T) / 16;
    const unsigned rowb = (unsigned)p.H * N * sizeof(T);
    const T* base = src ? reinterpret_cast<const T*>(src) + (((size_t)b * p.T + t0) * p.H + h) * N : nullptr;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc_n(base, base && nt > 0 ? (unsigned)(nt - 1) * rowb + N * sizeof(T) : 0u);
#pragma unroll
    for (int m = 0; m < NP; ++m) {
        const int i = tid + NT * m, t = i / PR, sg = i % PR;
        const unsigned off = i < C * PR ? (unsigned)t * rowb + (unsigned)sg * 16u : 0xffffffffu - 15u;
        r[m] = buf_load16(rs, off);
    }
}
// one bf16 element at byte offset off of a buffer (zero past its end)
__device__ __forceinline__ float buf_bf16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    const unsigned short x = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    return __uint_as_float((unsigned)x << 16);
}
// a buffer over the rows [0, nt) of the token tile (tokens t0.., head h) of a
// [B, T, H, N] bf16 tensor; row t starts at byte t * H * N * 2
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tok_rsrc(const void* src, const BwdParams& p, int b, int h, int t0,
                                                          int nt, int N) {
    const bf16* base = reinterpret_cast<const bf16*>(src) + (((size_t)b * p.T + t0) * p.H + h) * N;
    return make_rsrc_n(base, nt > 0 ? (unsigned)(nt - 1) * (unsigned)(p.H * N * 2) + (unsigned)(N * 2) : 0u);
}
// fp32 products on bf16 MFMA: x = hi + lo with hi = bf16(x), lo = bf16(x - hi),
// and a b = a.hi b.hi + a.hi b.lo + a.lo b.hi (the dropped a.lo b.lo and the
// rounding of lo are below 2^-16 of |a b|)
struct Split4 {
    bf16x4 hi, lo;
};
__device__ __forceinline__ Split4 split4(f32x4 x) {
    Split4 s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s.hi[i] = (bf16)x[i];
        s.lo[i] = (bf16)(x[i] - (float)s.hi[i]);
    }
    return s;
}
// x as one word: bf16 hi in the upper half, bf16 lo in the lower
__device__ __forceinline__ unsigned pack_hl(float x) {
    const bf16 hi = (bf16)x;
    const bf16 lo = (bf16)(x - (float)hi);
    return ((unsigned)__builtin_bit_cast(unsigned short, hi) << 16) | (unsigned)__builtin_bit_cast(unsigned short, lo);
}
// four packed words (elements 0..3) as the hi and lo fragments
__device__ __forceinline__ Split4 unpack_hl(unsigned w0, unsigned w1, unsigned w2, unsigned w3) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 h = {__builtin_amdgcn_perm(w1, w0, 0x07060302u), __builtin_amdgcn_perm(w3, w2, 0x07060302u)};
    const u32x2 lo = {__builtin_amdgcn_perm(w1, w0, 0x05040100u), __builtin_amdgcn_perm(w3, w2, 0x05040100u)};
    Split4 s;
    s.hi = __builtin_bit_cast(bf16x4, h);
    s.lo = __builtin_bit_cast(bf16x4, lo);
    return s;
}
__device__ __forceinline__ f32x4 mma16x3(f32x4 acc, const Split4& a, const Split4& b) {
    acc = mma16(acc, a.lo, b.hi);
    acc = mma16(acc, a.hi, b.lo);
    return mma16(acc, a.hi, b.hi);
}
// x of the lane N places further round its row of 16 lanes (DPP row_ror)
template <int N>
__device__ __forceinline__ float row_ror_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}
// one bf16 element to byte offset off of a buffer (dropped past its end)
__device__ __forceinline__ void buf_st_bf16(__amdgpu_buffer_rsrc_t r, unsigned off, float v) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)v), r, (int)off, 0, 0);
}
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// pieces [0, n) of a contiguous array
template <int NP, int NT = 256>
__device__ __forceinline__ void load_flat_pieces(const void* src, int n, uint4 (&r)[NP], int tid) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc_n(src, (unsigned)n * 16u);
#pragma unroll
    for (int m = 0; m < NP; ++m) r[m] = buf_load16(rs, (unsigned)(tid + NT * m) * 16u);
}
// piece i to row i / PR, byte (i % PR) 16 of an LDS array with row stride ld_bytes
template <int NP, int NT = 256>
__device__ __forceinline__ void store_pieces(void* dst, int ld_bytes, int PR, int n, const uint4 (&r)[NP], int tid) {
#pragma unroll
    for (int m = 0; m < NP; ++m) {
        const int i = tid + NT * m;
        if (i < n) *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(dst) + (i / PR) * ld_bytes + (i % PR) * 16) = r[m];
    }
}

// the in-chunk cumsum of the clamped log-gates (log2 units) from the raw gates
// in LDS ([C][K], zero rows past nt), and the sub-chunk references R_j
// (j = 0..4; R_4 = G_C).  All NT threads take part: the P = NT / K
// consecutive lanes of a channel each scan C / P tokens in registers, and
// their totals are combined by shuffles (no barrier, no LDS scratch).
template <typename T, int LDG, int K, int NT>
__device__ __forceinline__ void gate_cumsum_par(const T* sgraw, int tid, float* sG, float* sR) {
    constexpr int P = NT / K, L = C / P;
    static_assert(P * K == NT && L * P == C && 16 % L == 0 && (P & (P - 1)) == 0, "cumsum split");
    const int c = tid / P, part = tid % P;
    float x[L];
#pragma unroll
    for (int i = 0; i < L; ++i) x[i] = to_f32(sgraw[(part * L + i) * K + c]);
#pragma unroll
    for (int i = 0; i < L; ++i) x[i] = fminf(fmaxf(x[i], -5.f), 0.f) * kLog2e + (i ? x[i - 1] : 0.f);
    const float tot = x[L - 1];
    float incl = tot;
#pragma unroll
    for (int d = 1; d < P; d <<= 1) {
        const float y = __shfl_up(incl, d, P);
        if (part >= d) incl += y;
    }
    const float off = incl - tot;
#pragma unroll
    for (int i = 0; i < L; ++i) sG[(part * L + i) * LDG + c] = off + x[i];
    if (part == 0) sR[c] = 0.f;
    if (((part + 1) * L) % 16 == 0) sR[((part + 1) * L / 16) * K + c] = incl;
}

}  // namespace

// ============================================================================
// vside: U = U~ - W S;  D = tril(dO U^T);  dQh = dO S^T;  dKb = U dS'^T;
//        dW = -dU S^T;  rs = e^{G_C} rowsum(S * dS')
// ============================================================================
template <typename T, int K, int V>
struct VsideLayout {
    static constexpr int SZ = (int)sizeof(T), PAD = 16 / SZ;
    static constexpr int LDK = K + PAD, LDV = V + PAD;
    static constexpr int oR1 = 0;                                        // S^T [V][LDK], then S [K][LDV]
    static constexpr int oR2 = oR1 + cmax2(V * LDK, K * LDV) * SZ;       // W [C][LDK], then dO [C][LDV]
    static constexpr int oU = oR2 + cmax2(C * LDK, C * LDV) * SZ;        // U [C][LDV]
    static constexpr int oDS = oU + C * LDV * SZ;                        // dS' [K][LDV]
    static constexpr int oDU = oDS + K * LDV * SZ;                       // dU [C][LDV]
    static constexpr int TOTAL = oDU + C * LDV * SZ;
    static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
};

template <typename T, int K, int V>
__global__ __launch_bounds__(512) void kda_bwd_vside_kernel(BwdParams p) {
    using L = VsideLayout<T, K, V>;
    using Frag = typename FragOf<T>::type;
    constexpr int LDK = L::LDK, LDV = L::LDV, SZ = L::SZ;
    constexpr int NT = 512, NW = 8;
    constexpr int KS = K / 32, VS = V / 32, NVT = V / 16, NKT = K / 16;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
    T* sR1 = reinterpret_cast<T*>(smem + L::oR1);
    T* sR2 = reinterpret_cast<T*>(smem + L::oR2);
    T* sU = reinterpret_cast<T*>(smem + L::oU);
    T* sDS = reinterpret_cast<T*>(smem + L::oDS);
    T* sDU = reinterpret_cast<T*>(smem + L::oDU);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lg = l >> 4, lr = l & 15;
    // persistent: workgroup x takes items x, x + G, ... (item = bh * NC + ci);
    // the next item's S and dS' are loaded while this item's products run
    const int NC = p.NC;
    const long n_items = (long)p.B * p.H * NC;
    const size_t KV = (size_t)K * V;
    const RecLayout RL = rec_layout(K, V, SZ);
    constexpr int NS = K * V / 4 / NT;               // S / dS' pieces per thread
    constexpr int RQ = V / 4;                        // pieces per state row
    static_assert(NS * NT * 4 == K * V && 64 % RQ == 0, "state tiling");
    constexpr int PRK = K * SZ / 16, PRV = V * SZ / 16;
    constexpr int NPW = (C * PRK + NT - 1) / NT, NPO = (C * PRV + NT - 1) / NT;
    constexpr int NDU = (C * V / 4 + NT - 1) / NT;
    constexpr int NUT = 4 * NVT / NW;                // U tiles per wave
    static_assert(NUT * NW == 4 * NVT, "U tiles per wave");
    f32x4 rS[NS], rD[NS], rU[NDU];
    uint4 rw[NPW], ro[NPO];
    float egr[NS];
    typename Frag4Of<T>::type utr[NUT];
    // S (chunk start) and dS' (chunk end) of an item, fp32, 4 columns per
    // piece; a missing S0 or dL/dS_T reads as zeros
    auto load_states = [&](long it_) {
        const int ci_ = (int)(it_ % NC);
        const long bh_ = it_ / NC;
        const int b_ = (int)(bh_ / p.H), h_ = (int)(bh_ % p.H);
        const float* S0 = ci_ == 0 ? (p.s0 ? p.s0 + (size_t)bh_ * KV : nullptr)
                                   : p.snaps + (((size_t)b_ * NC + ci_ - 1) * p.H + h_) * KV;
        const float* dSp = ci_ == NC - 1 ? (p.dsT ? p.dsT + (size_t)bh_ * KV : nullptr) : p.adj + (size_t)it_ * KV;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc_n(S0, S0 ? (unsigned)(KV * 4) : 0u);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc_n(dSp, dSp ? (unsigned)(KV * 4) : 0u);
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const unsigned off = (unsigned)(tid + NT * m) * 16u;
            const uint4 a = buf_load16(rs, off), d = buf_load16(rd, off);
            rS[m] = f32x4{__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w)};
            rD[m] = f32x4{__uint_as_float(d.x), __uint_as_float(d.y), __uint_as_float(d.z), __uint_as_float(d.w)};
        }
    };
    const long G = gridDim.x;
    if ((long)blockIdx.x < n_items) load_states(blockIdx.x);
    for (long item = blockIdx.x; item < n_items; item += G) {
    const int ci = (int)(item % NC), bh = (int)(item / NC);
    const int b = bh / p.H, h = bh % p.H;
    const int t0 = ci * C, nt = min(C, p.T - t0);
    const size_t cs = (size_t)item;
    const unsigned char* rec = p.rec + cs * RL.bytes;

    // e^{G_C} of the state rows this thread sums for rs, and the U~ values of
    // this wave's U tiles: loaded first, so that no phase below waits on a
    // global load of its own
    {
        const float* egc = reinterpret_cast<const float*>(rec + RL.oEgc);
#pragma unroll
        for (int m = 0; m < NS; ++m) egr[m] = egc[(tid + NT * m) / RQ];
#pragma unroll
        for (int it = 0; it < NUT; ++it) {
            const int u = w + NW * it, vt = u >> 2, ti = u & 3;
            utr[it] = ld_frag4<T>(reinterpret_cast<const T*>(rec + RL.oUtT) + (size_t)(16 * vt + lr) * C + 16 * ti + 4 * lg);
        }
    }
    load_flat_pieces<NPW, NT>(rec + RL.oW, C * PRK, rw, tid);
    load_tok_pieces<T, V, NPO, NT>(p.d_o, p, b, h, t0, nt, ro, tid);
    {
        const __amdgpu_buffer_rsrc_t ru = make_rsrc_n(p.cdU + cs * C * V, (unsigned)(C * V * 4));
#pragma unroll
        for (int m = 0; m < NDU; ++m) {
            const uint4 a = buf_load16(ru, (unsigned)(tid + NT * m) * 16u);
            rU[m] = f32x4{__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w)};
        }
    }

    // ---- phase 1: S^T and W; U = U~ - W S ----------------------------------------
#pragma unroll
    for (int m = 0; m < NS; ++m) {
        const int i = tid + NT * m, r = i / RQ, c4 = 4 * (i % RQ);
#pragma unroll
        for (int e = 0; e < 4; ++e) sR1[(c4 + e) * LDK + r] = from_f32<T>(rS[m][e]);
    }
    store_pieces<NPW, NT>(sR2, LDK * SZ, PRK, C * PRK, rw, tid);
    // rs[r] = e^{G_C}[r] sum_v S[r][v] dS'[r][v] (fp32): the RQ consecutive
    // threads of a row add their pieces
#pragma unroll
    for (int m = 0; m < NS; ++m) {
        const int i = tid + NT * m, r = i / RQ;
        float d = rS[m][0] * rD[m][0] + rS[m][1] * rD[m][1] + rS[m][2] * rD[m][2] + rS[m][3] * rD[m][3];
#pragma unroll
        for (int x = 1; x < RQ; x <<= 1) d += __shfl_xor(d, x);
        if (i % RQ == 0) p.crs[cs * K + r] = egr[m] * d;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < NUT; ++it) {
        const int u = w + NW * it, vt = u >> 2, ti = u & 3;
        // U~[t][v] for t = 16 ti + 4 lg + e (the record holds U~^T [V][C])
        f32x4 acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = to_f32(utr[it][e]);
        f32x4 m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            m = mma(m, ld_frag_perm<T>(&sR2[(16 * ti + lr) * LDK + 32 * ks + 4 * lg]),
                    ld_frag_perm<T>(&sR1[(16 * vt + lr) * LDK + 32 * ks + 4 * lg]));
        acc = acc - m;
#pragma unroll
        for (int e = 0; e < 4; ++e) sU[(16 * ti + 4 * lg + e) * LDV + 16 * vt + lr] = from_f32<T>(acc[e]);
    }
    __syncthreads();

    // ---- phase 2: S, dS', dO, dU from the registers ---------------------------------
#pragma unroll
    for (int m = 0; m < NS; ++m) {
        const int i = tid + NT * m, r = i / RQ, c4 = 4 * (i % RQ);
        st4<T>(&sR1[r * LDV + c4], rS[m]);
        st4<T>(&sDS[r * LDV + c4], rD[m]);
    }
    store_pieces<NPO, NT>(sR2, LDV * SZ, PRV, C * PRV, ro, tid);
#pragma unroll
    for (int m = 0; m < NDU; ++m) {
        const int i = tid + NT * m, t = i / RQ, c4 = 4 * (i % RQ);
        if (i < C * V / 4) st4<T>(&sDU[t * LDV + c4], rU[m]);
    }
    // the registers of S and dS' are free: the next item's are loaded behind
    // this item's products
    if (item + G < n_items) load_states(item + G);
    __syncthreads();

    // D = tril(dO U^T): 16 tiles (zeros above the diagonal blocks)
    float* Dg = p.cD + cs * C * C;
    for (int d = w; d < 16; d += NW) {
        const int i = d >> 2, j = d & 3;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (j <= i) {
#pragma unroll
            for (int ks = 0; ks < VS; ++ks)
                acc = mma(acc, ld_frag_perm<T>(&sR2[(16 * i + lr) * LDV + 32 * ks + 4 * lg]),
                          ld_frag_perm<T>(&sU[(16 * j + lr) * LDV + 32 * ks + 4 * lg]));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * i + 4 * lg + e, s = 16 * j + lr;
            Dg[t * C + s] = (s <= t) ? acc[e] : 0.f;
        }
    }
    // dQh = dO S^T, dW = -dU S^T, dKb = U dS'^T: 4 x NKT tiles each
    float* dQh = p.cdQh + cs * C * K;
    float* dKb = p.cdKb + cs * C * K;
    float* dW = p.cdW + cs * C * K;
    for (int q = w; q < 4 * NKT; q += NW) {
        const int i = q / NKT, ct = q % NKT;
        f32x4 aq = {0.f, 0.f, 0.f, 0.f}, aw = aq, ak = aq;
#pragma unroll
        for (int ks = 0; ks < VS; ++ks) {
            const Frag bS = ld_frag_perm<T>(&sR1[(16 * ct + lr) * LDV + 32 * ks + 4 * lg]);
            const Frag bD = ld_frag_perm<T>(&sDS[(16 * ct + lr) * LDV + 32 * ks + 4 * lg]);
            aq = mma(aq, ld_frag_perm<T>(&sR2[(16 * i + lr) * LDV + 32 * ks + 4 * lg]), bS);
            aw = mma(aw, ld_frag_perm<T>(&sDU[(16 * i + lr) * LDV + 32 * ks + 4 * lg]), bS);
            ak = mma(ak, ld_frag_perm<T>(&sU[(16 * i + lr) * LDV + 32 * ks + 4 * lg]), bD);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t o = (size_t)(16 * i + 4 * lg + e) * K + 16 * ct + lr;
            dQh[o] = aq[e];
            dW[o] = -aw[e];
            dKb[o] = ak[e];
        }
    }
    __syncthreads();                                 // the next item overwrites the LDS operands
    }
}

// ============================================================================
// ksolve: Ak; (I + A)^T [dBv | dBk] = [dU | dW]; dv, dKh, Et, dbeta
// ============================================================================
template <typename T, int K, int V>
struct KsolveLayout {
    static constexpr int SZ = (int)sizeof(T), PAD = 16 / SZ;
    static constexpr int LDK = K + PAD, LDV = V + PAD, LDC = C + PAD;
    static constexpr int LDG = K + 4, LDA = C + 4;
    static constexpr int oG = 0;                                // fp32 [C][LDG] cumsum (log2 units)
    static constexpr int oR = oG + C * LDG * 4;                 // fp32 [5][K] sub-chunk references
    static constexpr int oB = oR + 5 * K * 4;                   // fp32 [C] beta
    static constexpr int oK = oB + C * 4;                       // T [C][LDK] k
    static constexpr int oAkT = oK + C * LDK * SZ;              // fp32 [C][LDA] Ak^T
    static constexpr int oBV = oAkT + C * LDA * 4;              // T [C][LDV] dBv
    static constexpr int oBK = oBV + C * LDV * SZ;              // T [C][LDK] dBk
    static constexpr int oW = oBK + C * LDK * SZ;               // T [C][LDK] W      } then E fp32 [C][LDA]
    static constexpr int oUt = oW + C * LDK * SZ;               // T [V][LDC] U~^T   } and v T [C][V]
    static constexpr int TOTAL = oW + cmax2(C * LDK * SZ + V * LDC * SZ, C * LDA * 4 + C * V * SZ);
    static_assert(C * K * SZ <= C * LDA * 4, "the raw gates must fit over Ak^T");
    static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
};

template <typename T, int K, int V>
__global__ __launch_bounds__(512) void kda_bwd_ksolve_kernel(BwdParams p) {
    using L = KsolveLayout<T, K, V>;
    using Frag = typename FragOf<T>::type;
    constexpr int LDK = L::LDK, LDV = L::LDV, LDC = L::LDC, LDG = L::LDG, LDA = L::LDA, SZ = L::SZ;
    constexpr int NT = 512, NW = 8;
    constexpr int KS = K / 32, VS = V / 32;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
    float* sG = reinterpret_cast<float*>(smem + L::oG);
    float* sR = reinterpret_cast<float*>(smem + L::oR);
    float* sB = reinterpret_cast<float*>(smem + L::oB);
    T* sK = reinterpret_cast<T*>(smem + L::oK);
    float* sAkT = reinterpret_cast<float*>(smem + L::oAkT);
    T* sBV = reinterpret_cast<T*>(smem + L::oBV);
    T* sBK = reinterpret_cast<T*>(smem + L::oBK);
    T* sW = reinterpret_cast<T*>(smem + L::oW);
    T* sUt = reinterpret_cast<T*>(smem + L::oUt);
    float* sE = reinterpret_cast<float*>(smem + L::oW);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lg = l >> 4, lr = l & 15;
    const int NC = p.NC;
    const int ci = blockIdx.x % NC, bh = blockIdx.x / NC;
    const int b = bh / p.H, h = bh % p.H;
    const int t0 = ci * C, nt = min(C, p.T - t0);
    const size_t cs = (size_t)bh * NC + ci;
    const RecLayout RL = rec_layout(K, V, SZ);
    const unsigned char* rec = p.rec + cs * RL.bytes;

    // right-hand sides [dU | dW] of this wave's 16-column tiles, accumulator layout
    constexpr int NCT = (V + K) / 16, CPW = (NCT + NW - 1) / NW;
    f32x4 R[CPW][4];
    auto load_rhs = [&]() {
#pragma unroll
        for (int q = 0; q < CPW; ++q) {
            const int ct = w + NW * q;
            const bool vcol = ct < V / 16;
            const int c = (vcol ? 16 * ct : 16 * ct - V) + lr;
            const float* rhs = vcol ? p.cdU + cs * C * V : p.cdW + cs * C * K;
            const int ld = vcol ? V : K;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    R[q][j][e] = ct < NCT ? rhs[(size_t)(16 * j + 4 * lg + e) * ld + c] : 0.f;
        }
    };
    constexpr int NPV = (C * V * SZ / 16 + NT - 1) / NT;
    uint4 rv[NPV];                                  // v rows, for dbeta
    T* sV = reinterpret_cast<T*>(smem + L::oW + C * LDA * 4);   // after E, over U~^T

    // ---- staging (the raw gates pass through the Ak^T area) -------------------------
    {
        constexpr int PRK = K * SZ / 16, PRC = C * SZ / 16;
        constexpr int NPK = (C * PRK + NT - 1) / NT, NPU = (V * PRC + NT - 1) / NT;
        uint4 rk[NPK], rg[NPK], rw[NPK], ru[NPU];
        load_tok_pieces<T, K, NPK, NT>(p.k, p, b, h, t0, nt, rk, tid);
        load_tok_pieces<T, K, NPK, NT>(p.g, p, b, h, t0, nt, rg, tid);
        load_flat_pieces<NPK, NT>(rec + RL.oW, C * PRK, rw, tid);
        load_flat_pieces<NPU, NT>(rec + RL.oUtT, V * PRC, ru, tid);
        const float bt = tid < nt ? to_f32(reinterpret_cast<const T*>(p.beta)[((size_t)b * p.T + t0 + tid) * p.H + h])
                                  : 0.f;
        // this wave's right-hand sides and v: loaded now, used after the Gram
        load_rhs();
        load_tok_pieces<T, V, NPV, NT>(p.v, p, b, h, t0, nt, rv, tid);
        if (tid < C) sB[tid] = bt;
        store_pieces<NPK, NT>(sK, LDK * SZ, PRK, C * PRK, rk, tid);
        store_pieces<NPK, NT>(sAkT, K * SZ, PRK, C * PRK, rg, tid);
        store_pieces<NPK, NT>(sW, LDK * SZ, PRK, C * PRK, rw, tid);
        store_pieces<NPU, NT>(sUt, LDC * SZ, PRC, V * PRC, ru, tid);
    }
    __syncthreads();
    gate_cumsum_par<T, LDG, K, NT>(reinterpret_cast<const T*>(sAkT), tid, sG, sR);
    __syncthreads();
    // (Ak^T needs no clearing: every entry read below is written by the Gram)

    // ---- Ak = sum_c k_s k_r e^{G_s - G_r} (r < s), per sub-chunk block pair (i >= j) ----
    // operands: k_s e^{G_s - R_i} (<= 1) and k_r e^{R_i - G_r} (<= 1 off the diagonal,
    // <= e^80 on it)
    for (int pr = w; pr < 10; pr += NW) {
        int i = 0, j = pr;
        while (j > i) { j -= i + 1; ++i; }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            Frag fa, fb;
            const int s = 16 * i + lr, r = 16 * j + lr;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int c = 32 * ks + 4 * lg + (u & 3) + (u >> 2) * 16;
                const float ri = sR[i * K + c];
                fa[u] = from_f32<T>(to_f32(sK[s * LDK + c]) * fast_exp2(sG[s * LDG + c] - ri));
                fb[u] = from_f32<T>(to_f32(sK[r * LDK + c]) * fast_exp2(ri - sG[r * LDG + c]));
            }
            acc = mma(acc, fa, fb);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = 16 * i + 4 * lg + e, r = 16 * j + lr;
            if (r < s) sAkT[r * LDA + s] = acc[e];
        }
    }
    __syncthreads();

    // ---- back substitution (I + A)^T [dBv | dBk] = [dU | dW], A[r][s] = beta_r Ak[r][s] ----
    // By 16-token blocks from the last: X_j = T_j^T (R_j - sum_{i > j} A_ij^T X_i), with
    // T_j = (I + A_jj)^{-1}, on fp32 MFMA.  T_j^T lives in a block of Ak^T below the
    // diagonal (entries never written or read there otherwise).
    auto tblock = [&](int j) {
        const int I = j < 3 ? j + 1 : 2, J = j < 3 ? 0 : 1;
        return sAkT + 16 * I * LDA + 16 * J;
    };
    if (tid < 64) {
        // column c of T_j by forward substitution; written as row c of T_j^T
        const int j = tid >> 4, c = tid & 15;
        float tc[16];
        // branch-free: T[m][c] = 0 for m < c, so the sums need no mask; rows
        // r <= c keep their start value
#pragma unroll
        for (int r = 0; r < 16; ++r) tc[r] = (float)(r == c);
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            float a = 0.f;
#pragma unroll
            for (int m = 0; m < r; ++m) a += sAkT[(16 * j + m) * LDA + 16 * j + r] * tc[m];
            const float v = -sB[16 * j + r] * a;
            tc[r] = r > c ? v : tc[r];
        }
        float* tt = tblock(j) + c * LDA;
#pragma unroll
        for (int r = 0; r < 16; ++r) tt[r] = tc[r];
    }
    __syncthreads();
    {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < CPW; ++q) {
            const int ct = w + NW * q;
            if (ct >= NCT) break;
            const bool vcol = ct < V / 16;
            const int c = (vcol ? 16 * ct : 16 * ct - V) + lr;      // column within dU or dW
            f32x4 X[4];
#pragma unroll
            for (int j = 3; j >= 0; --j) {
                f32x4 acc = R[q][j];
#pragma unroll
                for (int i = j + 1; i < 4; ++i) {
                    // -A_ij^T: row s = 16 j + lr, reduction r = 16 i + 4 lg + u
                    const f32x4 ak = *reinterpret_cast<const f32x4*>(&sAkT[(16 * j + lr) * LDA + 16 * i + 4 * lg]);
                    const f32x4 bt = *reinterpret_cast<const f32x4*>(&sB[16 * i + 4 * lg]);
                    acc = mma16(acc, -(ak * bt), X[i]);
                }
                X[j] = mma16(z, *reinterpret_cast<const f32x4*>(tblock(j) + lr * LDA + 4 * lg), acc);
            }
            T* dvp = reinterpret_cast<T*>(p.dv) + (((size_t)b * p.T + t0) * p.H + h) * V + c;
            float* dkh = p.cdKh + cs * C * K + c;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 16 * j + 4 * lg + e;
                    const float x = X[j][e], y = sB[s] * x;
                    if (vcol) {
                        sBV[s * LDV + c] = from_f32<T>(x);
                        if (s < nt) dvp[(size_t)s * p.H * V] = from_f32<T>(y);
                    } else {
                        sBK[s * LDK + c] = from_f32<T>(x);
                        dkh[(size_t)s * K] = y;
                    }
                }
        }
    }
    __syncthreads();

    // ---- E = -(dBv U~^T + dBk W^T), strictly lower; Et = diag(beta) E ---------------
    f32x4 eacc[(10 + NW - 1) / NW];
    int npr = 0;
    for (int pr = w; pr < 10; pr += NW, ++npr) {
        int i = 0, j = pr;
        while (j > i) { j -= i + 1; ++i; }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < VS; ++ks) {
            // B operand (column r, reduction v) gathered from U~^T [v][r]
            Frag fb;
            const T* u0 = sUt + (32 * ks + 4 * lg) * LDC + 16 * j + lr;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                fb[u] = u0[u * LDC];
                fb[4 + u] = u0[(16 + u) * LDC];
            }
            acc = mma(acc, ld_frag_perm<T>(&sBV[(16 * i + lr) * LDV + 32 * ks + 4 * lg]), fb);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            acc = mma(acc, ld_frag_perm<T>(&sBK[(16 * i + lr) * LDK + 32 * ks + 4 * lg]),
                      ld_frag_perm<T>(&sW[(16 * j + lr) * LDK + 32 * ks + 4 * lg]));
        eacc[npr] = -acc;
    }
    __syncthreads();                                // W, U~^T no longer read: E goes over them
    float* Et = p.cEt + cs * C * C;
    npr = 0;
    for (int pr = w; pr < 10; pr += NW, ++npr) {
        int i = 0, j = pr;
        while (j > i) { j -= i + 1; ++i; }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = 16 * i + 4 * lg + e, r = 16 * j + lr;
            const float ev = r < s ? eacc[npr][e] : 0.f;
            sE[s * LDA + r] = ev;
            Et[s * C + r] = sB[s] * ev;
        }
    }
    // the six blocks above the diagonal of Et are zero
    for (int pr = w; pr < 6; pr += NW) {
        const int i = pr < 3 ? 0 : (pr < 5 ? 1 : 2);
        const int j = pr < 3 ? pr + 1 : (pr < 5 ? pr - 1 : 3);
#pragma unroll
        for (int e = 0; e < 4; ++e) Et[(16 * i + 4 * lg + e) * C + 16 * j + lr] = 0.f;
    }
    store_pieces<NPV, NT>(sV, V * SZ, V * SZ / 16, C * V * SZ / 16, rv, tid);
    __syncthreads();

    // ---- dbeta: eight threads per token, each on a contiguous eighth of the
    // value and key columns (16-byte LDS reads) -------------------------------------
    {
        const int s = tid >> 3, part = tid & 7;
        constexpr int VP = V / 8, KP = K / 8;
        static_assert(VP % 8 == 0 && KP % 8 == 0, "whole 8-element pieces per thread");
        float acc = 0.f;
        if (s < nt) {
#pragma unroll
            for (int u = 0; u < VP / 8; ++u) {
                const int v = VP * part + 8 * u;
                const Frag a = ld_frag<T>(&sBV[s * LDV + v]), b = ld_frag<T>(&sV[s * V + v]);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc += to_f32(a[e]) * to_f32(b[e]);
            }
#pragma unroll
            for (int u = 0; u < KP / 8; ++u) {
                const int c = KP * part + 8 * u;
                const Frag a = ld_frag<T>(&sBK[s * LDK + c]), b = ld_frag<T>(&sK[s * LDK + c]);
                float gv[8];
                ld8f(&sG[s * LDG + c], gv);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc += to_f32(a[e]) * to_f32(b[e]) * fast_exp2(gv[e]);
            }
            for (int r = part; r < s; r += 8) acc += sE[s * LDA + r] * sAkT[r * LDA + s];
        }
        acc += __shfl_xor(acc, 1);
        acc += __shfl_xor(acc, 2);
        acc += __shfl_xor(acc, 4);
        if (part == 0 && s < nt)
            reinterpret_cast<T*>(p.dbeta)[((size_t)b * p.T + t0 + s) * p.H + h] = from_f32<T>(acc);
    }
}

// ============================================================================
// kgrad: X1, X2, Y1, Y2 and dq, dk, dg
// ============================================================================
// All in fp32 (operands and MFMA), whatever the input dtype: the terms of dG
// are each far larger than their sum (they cancel), so bf16 operands here
// would cost dg most of its precision.
// The products are independent per channel: a workgroup takes KH of the K
// channels (two workgroups per chunk at K = 128), so that two fit on a CU.
template <typename T, int KH>
struct KgradLayout {
    static constexpr int SZ = (int)sizeof(T), PAD = 16 / SZ;
    static constexpr int LDK = KH + PAD, LDC = C + 4, LDG = KH + 4;
    static constexpr int oG = 0;                                // fp32 [C][LDG] cumsum (log2 units)
    static constexpr int oR = oG + C * LDG * 4;                 // fp32 [5][KH]
    static constexpr int oK = oR + 5 * KH * 4;                  // T [C][LDK] k (exact in fp32)
    static constexpr int oQ = oK + C * LDK * SZ;                // T [C][LDK] q
    static constexpr int oD = oQ + C * LDK * SZ;                // fp32 [C][LDC] D      } then dG [C][LDG]
    static constexpr int oE = oD + C * LDC * 4;                 // fp32 [C][LDC] Et     }
    static constexpr int oCS = oE + C * LDC * 4;                // fp32 [4][KH] column sums
    static constexpr int oGR = oCS + 4 * KH * 4;                // T [C][KH] raw gates
    static constexpr int TOTAL = oGR + C * KH * SZ;
    static_assert(C * LDG <= 2 * C * LDC, "dG must fit over D and Et");
    static_assert(TOTAL <= (SZ == 2 ? 80 : 160) * 1024, "two bf16 workgroups per CU");
};

// pieces of columns [c0, c0 + KH) of the [C][N] token tile of a [B, T, H, N]
// tensor (head h, tokens t0 ..); rows from nt on are zero
template <typename T, int N, int KH, int NP, int NT>
__device__ __forceinline__ void load_tok_cols(const void* src, const BwdParams& p, int b, int h, int t0, int nt,
                                              int c0, uint4 (&r)[NP], int tid) {
    constexpr int PR = KH * (int)sizeof(T) / 16;
    const unsigned rowb = (unsigned)p.H * N * sizeof(T);
    const T* base = reinterpret_cast<const T*>(src) + (((size_t)b * p.T + t0) * p.H + h) * N + c0;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc_n(base, nt > 0 ? (unsigned)(nt - 1) * rowb + KH * sizeof(T) : 0u);
#pragma unroll
    for (int m = 0; m < NP; ++m) {
        const int i = tid + NT * m, t = i / PR, sg = i % PR;
        const unsigned off = i < C * PR ? (unsigned)t * rowb + (unsigned)sg * 16u : 0xffffffffu - 15u;
        r[m] = buf_load16(rs, off);
    }
}

template <typename T, int K, int KH>
__global__ __launch_bounds__(512) void kda_bwd_kgrad_kernel(BwdParams p) {
    using L = KgradLayout<T, KH>;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDG = L::LDG, SZ = L::SZ;
    constexpr int NT = 512, NW = 8, NH = K / KH;
    constexpr int NKT = KH / 16;                 // channel tiles (4 NKT tiles in all)
    constexpr int TPW = 4 * NKT / NW;            // tiles per wave
    static_assert(TPW * NW == 4 * NKT, "tiles per wave");
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
    float* sG = reinterpret_cast<float*>(smem + L::oG);
    float* sR = reinterpret_cast<float*>(smem + L::oR);
    T* sK = reinterpret_cast<T*>(smem + L::oK);
    T* sQ = reinterpret_cast<T*>(smem + L::oQ);
    float* sD = reinterpret_cast<float*>(smem + L::oD);
    float* sE = reinterpret_cast<float*>(smem + L::oE);
    float* sDG = reinterpret_cast<float*>(smem + L::oD);
    float* sCS = reinterpret_cast<float*>(smem + L::oCS);
    T* sGR = reinterpret_cast<T*>(smem + L::oGR);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lg = l >> 4, lr = l & 15;
    const int NC = p.NC;
    // workgroup (b, h, chunk, channel block); the blocks of a chunk are adjacent
    const int c0 = (blockIdx.x % NH) * KH;
    const int item = blockIdx.x / NH;
    const int ci = item % NC, bh = item / NC;
    const int b = bh / p.H, h = bh % p.H;
    const int t0 = ci * C, nt = min(C, p.T - t0);
    const size_t cs = (size_t)bh * NC + ci;
    const size_t rowK = (size_t)p.H * K;

    {
        constexpr int PRK = KH * SZ / 16, PRC = C * 4 / 16;
        constexpr int NPK = (C * PRK + NT - 1) / NT, NPC = (C * PRC + NT - 1) / NT;
        uint4 rk[NPK], rq[NPK], rg[NPK], rd[NPC], re[NPC];
        load_tok_cols<T, K, KH, NPK, NT>(p.k, p, b, h, t0, nt, c0, rk, tid);
        load_tok_cols<T, K, KH, NPK, NT>(p.q, p, b, h, t0, nt, c0, rq, tid);
        load_tok_cols<T, K, KH, NPK, NT>(p.g, p, b, h, t0, nt, c0, rg, tid);
        load_flat_pieces<NPC, NT>(p.cD + cs * C * C, C * PRC, rd, tid);
        load_flat_pieces<NPC, NT>(p.cEt + cs * C * C, C * PRC, re, tid);
        store_pieces<NPK, NT>(sK, LDK * SZ, PRK, C * PRK, rk, tid);
        store_pieces<NPK, NT>(sQ, LDK * SZ, PRK, C * PRK, rq, tid);
        store_pieces<NPK, NT>(sGR, KH * SZ, PRK, C * PRK, rg, tid);
        store_pieces<NPC, NT>(sD, LDC * 4, PRC, C * PRC, rd, tid);
        store_pieces<NPC, NT>(sE, LDC * 4, PRC, C * PRC, re, tid);
    }
    __syncthreads();
    gate_cumsum_par<T, LDG, KH, NT>(sGR, tid, sG, sR);
    __syncthreads();

    const float* dQhg = p.cdQh + cs * C * K + c0;
    const float* dKbg = p.cdKb + cs * C * K + c0;
    const float* dKhg = p.cdKh + cs * C * K + c0;
    T* dqo = reinterpret_cast<T*>(p.dq) + (((size_t)b * p.T + t0) * p.H + h) * K + c0;
    T* dko = reinterpret_cast<T*>(p.dk) + (((size_t)b * p.T + t0) * p.H + h) * K + c0;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 dgr[TPW];                              // dG of this wave's tiles until D, Et are done
#pragma unroll
    for (int it = 0; it < TPW; ++it) {
        const int q = w + NW * it;
        const int i = q / NKT, ct = q % NKT;
        const int c = 16 * ct + lr;              // channel within the block
        const float Ri = sR[i * KH + c];
        // the epilogue's fp32 operands, loaded ahead of the tile's products
        float eQh[4], eKb[4], eKh[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t o = (size_t)(16 * i + 4 * lg + e) * K + c;
            eQh[e] = dQhg[o];
            eKb[e] = dKbg[o];
            eKh[e] = dKhg[o];
        }
        // forward type on token block i: Y1 = D (k gated), X1 = Et (k gated)
        f32x4 y1 = z, x1 = z;
        for (int j = 0; j <= i; ++j) {
            const float ref = j == i ? Ri : sR[(j + 1) * KH + c];
            f32x4 bk;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int s = 16 * j + 4 * lg + u;
                bk[u] = to_f32(sK[s * LDK + c]) * fast_exp2(ref - sG[s * LDG + c]);
            }
            const f32x4 tD = mma16(z, *reinterpret_cast<const f32x4*>(&sD[(16 * i + lr) * LDC + 16 * j + 4 * lg]), bk);
            const f32x4 tE = mma16(z, *reinterpret_cast<const f32x4*>(&sE[(16 * i + lr) * LDC + 16 * j + 4 * lg]), bk);
            const float f = j == i ? 1.f : fast_exp2(Ri - ref);
            y1 += f * tD;
            x1 += f * tE;
        }
        // transposed type on token block i: Y2 = D^T (q gated), X2 = Et^T (k gated)
        f32x4 y2d = z, x2d = z, y2o = z, x2o = z;
        const float Rn = sR[(i + 1) * KH + c];
        for (int i2 = i; i2 < 4; ++i2) {
            const float R2 = sR[i2 * KH + c];
            f32x4 bq, bk, aD, aE;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = 16 * i2 + 4 * lg + u;
                const float gf = fast_exp2(sG[t * LDG + c] - R2);
                bq[u] = to_f32(sQ[t * LDK + c]) * gf;
                bk[u] = to_f32(sK[t * LDK + c]) * gf;
                aD[u] = sD[t * LDC + 16 * i + lr];
                aE[u] = sE[t * LDC + 16 * i + lr];
            }
            const f32x4 tY = mma16(z, aD, bq);
            const f32x4 tX = mma16(z, aE, bk);
            if (i2 == i) {
                y2d = tY;
                x2d = tX;
            } else {
                const float f = fast_exp2(R2 - Rn);
                y2o += f * tY;
                x2o += f * tX;
            }
        }
        // epilogue on rows t = 16 i + 4 lg + e, channel c
        const float RC = sR[4 * KH + c];
        float colpart = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * i + 4 * lg + e;
            const float gl = sG[t * LDG + c];
            const float eg = fast_exp2(gl), egc = fast_exp2(RC - gl);
            const float fwd = fast_exp2(gl - Ri);
            const float Y1 = fwd * y1[e], X1 = fwd * x1[e];
            const float Y2 = fast_exp2(Ri - gl) * y2d[e] + fast_exp2(Rn - gl) * y2o[e];
            const float X2 = fast_exp2(Ri - gl) * x2d[e] + fast_exp2(Rn - gl) * x2o[e];
            const float kk = to_f32(sK[t * LDK + c]), qq = to_f32(sQ[t * LDK + c]);
            const float dQh = eQh[e], dKb = eKb[e], dKh = eKh[e];
            const float kb = kk * egc;
            dgr[it][e] = dQh * qq * eg + dKh * kk * eg - dKb * kb + kk * (X1 - X2 - Y2) + qq * Y1;
            colpart += dKb * kb;
            if (t < nt) {
                dqo[(size_t)t * rowK + c] = from_f32<T>(dQh * eg + Y1);
                dko[(size_t)t * rowK + c] = from_f32<T>(dKh * eg + X1 + X2 + Y2 + dKb * egc);
            }
        }
        colpart += __shfl_xor(colpart, 16);
        colpart += __shfl_xor(colpart, 32);
        if (lg == 0) sCS[i * KH + c] = colpart;
    }
    __syncthreads();                             // D and Et are no longer read: dG goes over them
#pragma unroll
    for (int it = 0; it < TPW; ++it) {
        const int q = w + NW * it;
        const int i = q / NKT, ct = q % NKT;
#pragma unroll
        for (int e = 0; e < 4; ++e) sDG[(16 * i + 4 * lg + e) * LDG + 16 * ct + lr] = dgr[it][e];
    }
    __syncthreads();

    // dg: reverse cumsum over the chunk plus the G_C terms, gate-derivative mask
    if (tid < KH) {
        const int c = tid;
        float tot = p.crs[cs * K + c0 + c] + sCS[c] + sCS[KH + c] + sCS[2 * KH + c] + sCS[3 * KH + c];
        T* dgo = reinterpret_cast<T*>(p.dg) + (((size_t)b * p.T + t0) * p.H + h) * K + c0 + c;
        for (int t = C - 1; t >= 0; --t) {
            tot += sDG[t * LDG + c];
            // the clamp passes the gradient where the raw gate lies in [-5, 0]
            const float gv = to_f32(sGR[t * KH + c]);
            if (t < nt) dgo[(size_t)t * rowK] = from_f32<T>(gv >= -5.f && gv <= 0.f ? tot : 0.f);
        }
    }
}

// ============================================================================
// fused: the three stages above in one workgroup per chunk (bf16, K = V = 128)
// ============================================================================
// Nothing between the stages leaves the workgroup: D, E and the Gram stay in
// LDS, and dQh, dKb, dKh stay in the registers of the wave that uses them.
// Wave w owns channel (and value) columns 16 w .. 16 w + 15 throughout:
//   dQh = dO S^T, dKb = U dS'^T and dBk = -dBv S^T take their B operands
//   from rows 16 w .. of S and dS', loaded straight into this wave's
//   registers; the back substitution solves value column tile w; the gated
//   products and the epilogue run on channel tile w.
// dBk needs no solve of its own: W = (I + A)^{-1} diag(beta) K e^G enters
// only through U = U~ - W S, so dW = -dU S^T and, the solve being linear,
// (I + A)^{-T} dW = -((I + A)^{-T} dU) S^T = -dBv S^T.
struct FusedBwdLayout {
    static constexpr int K = 128, V = 128;
    static constexpr int LDK = K + 8, LDV = V + 8, LDC = C + 8;     // bf16 row strides
    static constexpr int LDA = C + 4, LDG = K + 4, LDDG = K + 1;     // fp32 row strides
    static constexpr int oA = 0;                  // S^T [V][LDK] | Ak^T, D (hi|lo words) [C][LDA] | dG [C][LDDG]
    static constexpr int oAkT = oA, oD = oA + C * LDA * 4;
    static constexpr int oW = oA + V * LDK * 2;   // W [C][LDK] | diag(beta) E (hi|lo words) [C][LDA]
    static constexpr int oUt = oW + C * LDK * 2;  // U~^T [V][LDC] | column sums fp32 [4][K], E.Ak partial sums [C][4]
    static constexpr int oDO = oUt + V * LDC * 2; // dO [C][LDV] | dBv [C][LDV]
    static constexpr int oK = oDO + C * LDV * 2;  // k [C][LDK]
    static constexpr int oG = oK + C * LDK * 2;   // G fp32 [C][LDG] (log2 units)
    static constexpr int oU = oG + C * LDG * 4;   // U [C][LDV] | dBk [C][LDK]
    static constexpr int oR = oU + C * LDV * 2;   // R fp32 [5][K]
    static constexpr int oM = oR + 5 * K * 4;     // clamp pass mask: [K][4] x 16 bits (channel, token block)
    static constexpr int oB = oM + K * 4 * 2;     // beta fp32 [C]
    static constexpr int oTot = oB + C * 4;       // gate totals of the four token blocks fp32 [4][K] | rs at [3][K]
    static constexpr int TOTAL = oTot + 4 * K * 4;
    static_assert(2 * C * LDA * 4 <= V * LDK * 2 && C * LDDG * 4 <= V * LDK * 2, "region A");
    static_assert(C * LDA * 4 <= C * LDK * 2, "E over W");
    static_assert(4 * K * 4 + C * 4 * 4 <= V * LDC * 2, "column sums and E.Ak sums over U~^T");
    static_assert(C * LDK <= C * LDV, "dBk over U");
    static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
};

__global__ __launch_bounds__(512, 1) void kda_bwd_fused_kernel(BwdParams p) {
    using L = FusedBwdLayout;
    using T = bf16;
    constexpr int K = L::K, V = L::V;
    constexpr int LDK = L::LDK, LDV = L::LDV, LDC = L::LDC, LDA = L::LDA, LDG = L::LDG, LDDG = L::LDDG;
    constexpr int NT = 512;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
    T* sST = reinterpret_cast<T*>(smem + L::oA);
    float* sAkT = reinterpret_cast<float*>(smem + L::oAkT);
    unsigned* sD = reinterpret_cast<unsigned*>(smem + L::oD);
    float* sDG = reinterpret_cast<float*>(smem + L::oA);
    T* sW = reinterpret_cast<T*>(smem + L::oW);
    unsigned* sE = reinterpret_cast<unsigned*>(smem + L::oW);
    T* sUt = reinterpret_cast<T*>(smem + L::oUt);
    float* sCS = reinterpret_cast<float*>(smem + L::oUt);
    float* sPE = sCS + 4 * K;                      // [C][4]: sum_r E[s][r] Ak[s][r] over key block j
    T* sDO = reinterpret_cast<T*>(smem + L::oDO);
    T* sBV = reinterpret_cast<T*>(smem + L::oDO);
    T* sK = reinterpret_cast<T*>(smem + L::oK);
    float* sG = reinterpret_cast<float*>(smem + L::oG);
    T* sU = reinterpret_cast<T*>(smem + L::oU);
    T* sBK = reinterpret_cast<T*>(smem + L::oU);
    float* sR = reinterpret_cast<float*>(smem + L::oR);
    unsigned short* sM = reinterpret_cast<unsigned short*>(smem + L::oM);
    float* sB = reinterpret_cast<float*>(smem + L::oB);
    float* sTot = reinterpret_cast<float*>(smem + L::oTot);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lg = l >> 4, lr = l & 15;
    const int cw = 16 * w + lr;                   // this lane's channel / value column
    const int NC = p.NC;
    const int item = blockIdx.x;                  // (b * H + h) * NC + chunk
    const int ci = item % NC, bh = item / NC;
    const int b = bh / p.H, h = bh % p.H;
    const int t0 = ci * C, nt = min(C, p.T - t0);
    const size_t KV = (size_t)K * V;
    const size_t rowK = (size_t)p.H * K;          // token stride of [B, T, H, K] (and V = K)
    const RecLayout RL = rec_layout(K, V, 2);
    const unsigned char* rec = p.rec + (size_t)item * RL.bytes;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};

    // ---- global loads, all issued before any is waited on ---------------------------
    // first what stages 0 and 1 use (S, W, U~^T, the gates), then dS', dO and k,
    // which arrive while they run.  Rows cw of S (chunk start) and dS' (chunk
    // end), bf16: lane group lg holds columns 32 ks + 4 lg + {0..3} and
    // 32 ks + 16 + 4 lg + {0..3} (permuted slots)
    const bf16* S0 = ci == 0 ? (p.s0h ? reinterpret_cast<const bf16*>(p.s0h) + (size_t)bh * KV : nullptr)
                             : reinterpret_cast<const bf16*>(p.snaps16) + (((size_t)b * NC + ci - 1) * p.H + h) * KV;
    const bf16* dSp = ci == NC - 1 ? (p.dsTh ? reinterpret_cast<const bf16*>(p.dsTh) + (size_t)bh * KV : nullptr)
                                   : reinterpret_cast<const bf16*>(p.adj16) + (size_t)item * KV;
    u32x2 rS[8], rDS[8];
    {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc_n(S0, S0 ? (unsigned)(KV * 2) : 0u);
#pragma unroll
        for (int m = 0; m < 8; ++m)
            rS[m] = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)((cw * V + 32 * (m >> 1) + 16 * (m & 1) + 4 * lg) * 2), 0, 0);
    }
    uint4 rw[2], ru[2], ro[2], rk[2];
    load_flat_pieces<2, NT>(rec + RL.oW, C * K * 2 / 16, rw, tid);
    load_flat_pieces<2, NT>(rec + RL.oUtT, V * C * 2 / 16, ru, tid);
    // raw gates of channel gc, tokens 16 gp .. 16 gp + 15 (zeros past the end)
    const int gc = tid & (K - 1), gp = tid >> 7;
    float graw[16];
    {
        const __amdgpu_buffer_rsrc_t rg = tok_rsrc(p.g, p, b, h, t0, nt, K);
#pragma unroll
        for (int i = 0; i < 16; ++i) graw[i] = buf_bf16(rg, (unsigned)((16 * gp + i) * rowK + gc) * 2u);
    }
    float beta_t;
    {
        const T* bb = reinterpret_cast<const T*>(p.beta) + ((size_t)b * p.T + t0) * p.H + h;
        const __amdgpu_buffer_rsrc_t rb = make_rsrc_n(bb, nt > 0 ? (unsigned)((nt - 1) * p.H + 1) * 2u : 0u);
        beta_t = buf_bf16(rb, (unsigned)(tid * p.H) * 2u);   // zero from token nt on
    }
    {
        const __amdgpu_buffer_rsrc_t rd = make_rsrc_n(dSp, dSp ? (unsigned)(KV * 2) : 0u);
#pragma unroll
        for (int m = 0; m < 8; ++m)
            rDS[m] = __builtin_amdgcn_raw_buffer_load_b64(rd, (int)((cw * V + 32 * (m >> 1) + 16 * (m & 1) + 4 * lg) * 2), 0, 0);
    }
    load_tok_pieces<T, V, 2, NT>(p.d_o, p, b, h, t0, nt, ro, tid);
    load_tok_pieces<T, K, 2, NT>(p.k, p, b, h, t0, nt, rk, tid);
    const float egc_c = reinterpret_cast<const float*>(rec + RL.oEgc)[cw];

    // ---- stage 0: S^T, W, U~^T to LDS; S fragments; gate scan within blocks ----------
    typename FragOf<T>::type fS[4], fD[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const u32x4 w4 = {rS[2 * ks][0], rS[2 * ks][1], rS[2 * ks + 1][0], rS[2 * ks + 1][1]};
        fS[ks] = __builtin_bit_cast(bf16x8, w4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sST[(32 * ks + 4 * lg + e) * LDK + cw] = fS[ks][e];
            sST[(32 * ks + 16 + 4 * lg + e) * LDK + cw] = fS[ks][4 + e];
        }
    }
    store_pieces<2, NT>(sW, LDK * 2, K * 2 / 16, C * K * 2 / 16, rw, tid);
    store_pieces<2, NT>(sUt, LDC * 2, C * 2 / 16, V * C * 2 / 16, ru, tid);
    if (tid < C) sB[tid] = beta_t;
    float gx[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        gx[i] = fminf(fmaxf(graw[i], -5.f), 0.f) * kLog2e + (i ? gx[i - 1] : 0.f);
    }
    {
        // the clamp passes the gradient where the raw gate lies in [-5, 0]
        unsigned pass = 0u;
#pragma unroll
        for (int i = 0; i < 16; ++i) pass |= (graw[i] >= -5.f && graw[i] <= 0.f) ? (1u << i) : 0u;
        sM[gc * 4 + gp] = (unsigned short)pass;
    }
    sTot[gp * K + gc] = gx[15];
    __syncthreads();

    // ---- stage 1: G and the references R_j; U = U~ - W S; dS' fragments and rs;
    // dO and k to LDS ------------------------------------------------------------------
    {
        float off = 0.f;
#pragma unroll
        for (int q = 0; q < 3; ++q)
            if (q < gp) off += sTot[q * K + gc];
#pragma unroll
        for (int i = 0; i < 16; ++i) sG[(16 * gp + i) * LDG + gc] = off + gx[i];
        sR[gp * K + gc] = off;
        if (gp == 3) sR[4 * K + gc] = off + gx[15];
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
        f32x4 acc = ld4_as_f32<T>(&sUt[cw * LDC + 16 * ti + 4 * lg]);      // U~[16 ti + 4 lg + e][cw]
        f32x4 m = z;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            m = mma(m, ld_frag_perm<T>(&sW[(16 * ti + lr) * LDK + 32 * ks + 4 * lg]),
                    ld_frag_perm<T>(&sST[cw * LDK + 32 * ks + 4 * lg]));
        acc = acc - m;
#pragma unroll
        for (int e = 0; e < 4; ++e) sU[(16 * ti + 4 * lg + e) * LDV + cw] = from_f32<T>(acc[e]);
    }
    float rsp = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const u32x4 w4 = {rDS[2 * ks][0], rDS[2 * ks][1], rDS[2 * ks + 1][0], rDS[2 * ks + 1][1]};
        fD[ks] = __builtin_bit_cast(bf16x8, w4);
#pragma unroll
        for (int e = 0; e < 8; ++e) rsp += to_f32(fS[ks][e]) * to_f32(fD[ks][e]);
    }
    rsp += __shfl_xor(rsp, 16);
    rsp += __shfl_xor(rsp, 32);
    // e^{G_C} sum_v S[cw][v] dS'[cw][v], kept in the fourth block total's slot
    // (the offsets above read only the first three)
    if (lg == 0) sTot[3 * K + cw] = egc_c * rsp;
    store_pieces<2, NT>(sDO, LDV * 2, V * 2 / 16, C * V * 2 / 16, ro, tid);
    store_pieces<2, NT>(sK, LDK * 2, K * 2 / 16, C * K * 2 / 16, rk, tid);
    __syncthreads();

    // ---- stage 2: the gated Gram Ak; D = tril(dO U^T); dQh = dO S^T; dKb = U dS'^T ----
    // loads for the later stages, issued here so that they are not held
    // through the first ones
    // right-hand side of the solve: dU (fp32) of value column cw, accumulator layout
    f32x4 R[4];
    {
        const float* dUg = p.cdU + (size_t)item * C * V + cw;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) R[j][e] = dUg[(size_t)(16 * j + 4 * lg + e) * V];
    }
    auto pair_ij = [](int pr, int& i, int& j) {
        i = 0;
        j = pr;
        while (j > i) { j -= i + 1; ++i; }
    };
    for (int pr = w; pr < 10; pr += 8) {
        int i, j;
        pair_ij(pr, i, j);
        f32x4 acc = z;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            typename FragOf<T>::type fa, fb;
            const int s = 16 * i + lr, r = 16 * j + lr;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int c = 32 * ks + 4 * lg + (u & 3) + (u >> 2) * 16;
                const float ri = sR[i * K + c];
                fa[u] = from_f32<T>(to_f32(sK[s * LDK + c]) * fast_exp2(sG[s * LDG + c] - ri));
                fb[u] = from_f32<T>(to_f32(sK[r * LDK + c]) * fast_exp2(ri - sG[r * LDG + c]));
            }
            acc = mma(acc, fa, fb);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = 16 * i + 4 * lg + e, r = 16 * j + lr;
            if (r < s) sAkT[r * LDA + s] = acc[e];
        }
    }
    auto d_block = [&](int dd) {
        int i, j;
        pair_ij(dd, i, j);
        f32x4 acc = z;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            acc = mma(acc, ld_frag_perm<T>(&sDO[(16 * i + lr) * LDV + 32 * ks + 4 * lg]),
                      ld_frag_perm<T>(&sU[(16 * j + lr) * LDV + 32 * ks + 4 * lg]));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * i + 4 * lg + e, s = 16 * j + lr;
            sD[t * LDA + s] = s <= t ? pack_hl(acc[e]) : 0u;
        }
    };
    d_block(w);
    if (w >= 6) d_block(15 - w);
    f32x4 qh[4], kb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        qh[i] = z;
        kb[i] = z;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            qh[i] = mma(qh[i], ld_frag_perm<T>(&sDO[(16 * i + lr) * LDV + 32 * ks + 4 * lg]), fS[ks]);
            kb[i] = mma(kb[i], ld_frag_perm<T>(&sU[(16 * i + lr) * LDV + 32 * ks + 4 * lg]), fD[ks]);
        }
    }
    __syncthreads();

    // ---- stage 3: T_j = (I + A_jj)^{-1}, A = diag(beta) Ak: (I - N)(I + N^2)(I + N^4)(I + N^8) --
    // q of channel cw at tokens 16 i + 4 lg + e (gated products, epilogue)
    float qv[4][4];
    {
        const __amdgpu_buffer_rsrc_t rq = tok_rsrc(p.q, p, b, h, t0, nt, K);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                qv[i][e] = buf_bf16(rq, (unsigned)((16 * i + 4 * lg + e) * rowK + cw) * 2u);
    }
    // v of token tid / 8, columns 16 (tid % 8) .. + 15 (dbeta)
    uint4 rv[2];
    {
        const __amdgpu_buffer_rsrc_t rvs = tok_rsrc(p.v, p, b, h, t0, nt, V);
        const unsigned off = (unsigned)((tid >> 3) * rowK + 16 * (tid & 7)) * 2u;
        rv[0] = buf_load16(rvs, off);
        rv[1] = buf_load16(rvs, off + 16u);
    }
    // T_j^T goes to a block of Ak^T below the diagonal (never written or read otherwise)
    auto tblock = [&](int j) {
        const int I = j < 3 ? j + 1 : 2, J = j < 3 ? 0 : 1;
        return sAkT + 16 * I * LDA + 16 * J;
    };
    if (w < 4) {
        // wave j: N = A_jj (strictly lower, so N^16 = 0).  Every factor is a
        // polynomial in N (they commute); a product P Q takes P's A operand from
        // the accumulator of P^T and Q's B operand from the accumulator of Q,
        // so both layouts are carried.
        const int j = w;
        const f32x4 bt4 = *reinterpret_cast<const f32x4*>(&sB[16 * j + 4 * lg]);
        const float btr = sB[16 * j + lr];
        f32x4 n, nt4;                              // acc(N), acc(N^T)
        {
            const f32x4 a = *reinterpret_cast<const f32x4*>(&sAkT[(16 * j + lr) * LDA + 16 * j + 4 * lg]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 4 * lg + e;         // N[rr][lr] = beta_rr Ak[rr][lr], rr > lr
                n[e] = rr > lr ? bt4[e] * a[e] : 0.f;
                const float at = sAkT[(16 * j + rr) * LDA + 16 * j + lr];
                nt4[e] = lr > rr ? btr * at : 0.f;  // N^T[rr][lr] = N[lr][rr]
            }
        }
        f32x4 id;
#pragma unroll
        for (int e = 0; e < 4; ++e) id[e] = (4 * lg + e == lr) ? 1.f : 0.f;
        const f32x4 n2 = mma16(z, nt4, n), n2t = mma16(z, n, nt4);
        const f32x4 n4 = mma16(z, n2t, n2), n4t = mma16(z, n2, n2t);
        const f32x4 n8 = mma16(z, n4t, n4);
        const f32x4 p1 = id - n, p1t = id - nt4;
        const f32x4 p2 = p1 + mma16(z, n2t, p1), p2t = p1t + mma16(z, n2, p1t);
        const f32x4 p3 = p2 + mma16(z, n4t, p2), p3t = p2t + mma16(z, n4, p2t);
        const f32x4 tj = p3 + mma16(z, p3t, n8);  // acc(T_j)
        // T_j^T as the solve reads it: row c holds column c of T_j
        *reinterpret_cast<f32x4*>(tblock(j) + lr * LDA + 4 * lg) = tj;
    }
    __syncthreads();

    // ---- stage 4: (I + A)^T dBv = dU for value column tile w; dv -------------------
    {
        f32x4 X[4];
#pragma unroll
        for (int j = 3; j >= 0; --j) {
            f32x4 acc = R[j];
#pragma unroll
            for (int i = j + 1; i < 4; ++i) {
                const f32x4 ak = *reinterpret_cast<const f32x4*>(&sAkT[(16 * j + lr) * LDA + 16 * i + 4 * lg]);
                const f32x4 bt = *reinterpret_cast<const f32x4*>(&sB[16 * i + 4 * lg]);
                acc = mma16(acc, -(ak * bt), X[i]);
            }
            X[j] = mma16(z, *reinterpret_cast<const f32x4*>(tblock(j) + lr * LDA + 4 * lg), acc);
        }
        const __amdgpu_buffer_rsrc_t rdv = tok_rsrc(p.dv, p, b, h, t0, nt, V);   // rows past nt dropped
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 16 * j + 4 * lg + e;
                const float x = X[j][e];
                sBV[s * LDV + cw] = from_f32<T>(x);
                buf_st_bf16(rdv, (unsigned)(s * rowK + cw) * 2u, sB[s] * x);
            }
    }
    __syncthreads();

    // ---- stage 5: dBk = -dBv S^T for channel tile w; dKh = diag(beta) dBk -----------
    f32x4 dkh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x4 a = z;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) a = mma(a, ld_frag_perm<T>(&sBV[(16 * i + lr) * LDV + 32 * ks + 4 * lg]), fS[ks]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = 16 * i + 4 * lg + e;
            sBK[s * LDK + cw] = from_f32<T>(-a[e]);
            dkh[i][e] = -sB[s] * a[e];
        }
    }
    __syncthreads();

    // ---- stage 6: E = -(dBv U~^T + dBk W^T), strictly lower; diag(beta) E kept split --
    {
        f32x4 eacc[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int pr = w + 8 * n;
            if (pr >= 10) break;
            int i, j;
            pair_ij(pr, i, j);
            f32x4 acc = z;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                typename FragOf<T>::type fb;
                const T* u0 = sUt + (32 * ks + 4 * lg) * LDC + 16 * j + lr;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    fb[u] = u0[u * LDC];
                    fb[4 + u] = u0[(16 + u) * LDC];
                }
                acc = mma(acc, ld_frag_perm<T>(&sBV[(16 * i + lr) * LDV + 32 * ks + 4 * lg]), fb);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc = mma(acc, ld_frag_perm<T>(&sBK[(16 * i + lr) * LDK + 32 * ks + 4 * lg]),
                          ld_frag_perm<T>(&sW[(16 * j + lr) * LDK + 32 * ks + 4 * lg]));
            eacc[n] = -acc;
        }
        __syncthreads();                          // W and U~^T are no longer read: E goes over W
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int pr = w + 8 * n;
            if (pr >= 10) break;
            int i, j;
            pair_ij(pr, i, j);
            // and dbeta's sum_r E[s][r] Ak[s][r] over this key block (16 lanes per row)
            f32x4 pe;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 16 * i + 4 * lg + e, r = 16 * j + lr;
                const float ev = r < s ? eacc[n][e] : 0.f;
                sE[s * LDA + r] = pack_hl(sB[s] * ev);
                pe[e] = r < s ? ev * sAkT[r * LDA + s] : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pe[e] += row_ror_f<8>(pe[e]);
                pe[e] += row_ror_f<4>(pe[e]);
                pe[e] += row_ror_f<2>(pe[e]);
                pe[e] += row_ror_f<1>(pe[e]);
            }
            if (lr == 0)
#pragma unroll
                for (int e = 0; e < 4; ++e) sPE[(16 * i + 4 * lg + e) * 4 + j] = pe[e];
        }
    }
    __syncthreads();

    // ---- stage 7: dbeta; the gated products and dq, dk, dG --------------------------
    {
        // eight threads per token, each on an eighth of the value and key columns
        const int s = tid >> 3, part = tid & 7;
        float acc = 0.f;
        if (s < nt) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int v = 16 * part + 8 * u;
                const typename FragOf<T>::type a = ld_frag<T>(&sBV[s * LDV + v]);
                const uint4 pv = rv[u];
                const unsigned pw[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc += to_f32(a[2 * e]) * __uint_as_float(pw[e] << 16);
                    acc += to_f32(a[2 * e + 1]) * __uint_as_float(pw[e] & 0xffff0000u);
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int c = 16 * part + 8 * u;
                const typename FragOf<T>::type a = ld_frag<T>(&sBK[s * LDK + c]), kk = ld_frag<T>(&sK[s * LDK + c]);
                float gv[8];
                ld8f(&sG[s * LDG + c], gv);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc += to_f32(a[e]) * to_f32(kk[e]) * fast_exp2(gv[e]);
            }
            // the key blocks j <= s / 16 hold the E.Ak sums of token s
            if (part <= (s >> 4)) acc += sPE[s * 4 + part];
        }
        acc += __shfl_xor(acc, 1);
        acc += __shfl_xor(acc, 2);
        acc += __shfl_xor(acc, 4);
        if (part == 0 && s < nt)
            reinterpret_cast<T*>(p.dbeta)[((size_t)b * p.T + t0 + s) * p.H + h] = from_f32<T>(acc);
    }
    f32x4 dgr[4];
    {
        // per token t = 16 i + 4 lg + e of channel cw (R_i the reference of its block):
        //   ep = e^{G_t - R_i} <= 1,  em = e^{R_i - G_t} (>= 1, below e^80 at the clamp floor)
        // and the key / query operands of the gated products, split once per block:
        //   km_i = k em (forward type),  kp_i = k ep, qp_i = q ep (transposed type)
        float kv[4][4], ep[4][4], em[4][4], gl[4][4];
        float Rr[5];
#pragma unroll
        for (int j = 0; j < 5; ++j) Rr[j] = sR[j * K + cw];
        Split4 km[4], kp[4], qp[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 a, b2, c2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * i + 4 * lg + e;
                kv[i][e] = to_f32(sK[t * LDK + cw]);
                gl[i][e] = sG[t * LDG + cw];
                ep[i][e] = fast_exp2(gl[i][e] - Rr[i]);
                em[i][e] = fast_exp2(Rr[i] - gl[i][e]);
                a[e] = kv[i][e] * em[i][e];
                b2[e] = kv[i][e] * ep[i][e];
                c2[e] = qv[i][e] * ep[i][e];
            }
            km[i] = split4(a);
            kp[i] = split4(b2);
            qp[i] = split4(c2);
        }
        // e^{R_a - R_b} (a > b, <= 1) between block references
        float xr[5][5];
#pragma unroll
        for (int a2 = 1; a2 < 5; ++a2)
#pragma unroll
            for (int b3 = 0; b3 < a2; ++b3) xr[a2][b3] = fast_exp2(Rr[a2] - Rr[b3]);
        const __amdgpu_buffer_rsrc_t rdq = tok_rsrc(p.dq, p, b, h, t0, nt, K);   // rows past nt dropped
        const __amdgpu_buffer_rsrc_t rdk = tok_rsrc(p.dk, p, b, h, t0, nt, K);
        const float RC = Rr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // forward type on token block i: Y1 = D (k gated), X1 = Et (k gated).
            // Key block j enters with k e^{R_j - G_s} and the factor e^{R_i - R_j}.
            f32x4 y1, x1;
            {
                const uint4 dw = *reinterpret_cast<const uint4*>(&sD[(16 * i + lr) * LDA + 16 * i + 4 * lg]);
                const uint4 ew = *reinterpret_cast<const uint4*>(&sE[(16 * i + lr) * LDA + 16 * i + 4 * lg]);
                y1 = mma16x3(z, unpack_hl(dw.x, dw.y, dw.z, dw.w), km[i]);
                x1 = mma16x3(z, unpack_hl(ew.x, ew.y, ew.z, ew.w), km[i]);
            }
#pragma unroll
            for (int j = 0; j < i; ++j) {
                const uint4 dw = *reinterpret_cast<const uint4*>(&sD[(16 * i + lr) * LDA + 16 * j + 4 * lg]);
                const uint4 ew = *reinterpret_cast<const uint4*>(&sE[(16 * i + lr) * LDA + 16 * j + 4 * lg]);
                const f32x4 tD = mma16x3(z, unpack_hl(dw.x, dw.y, dw.z, dw.w), km[j]);
                const f32x4 tE = mma16x3(z, unpack_hl(ew.x, ew.y, ew.z, ew.w), km[j]);
                y1 += xr[i][j] * tD;
                x1 += xr[i][j] * tE;
            }
            // transposed type on token block i: Y2 = D^T (q gated), X2 = Et^T (k gated).
            // Token block i2 enters with q e^{G_t - R_i2}; for i2 > i, the factor
            // e^{R_i2 - R_{i+1}} brings it to the reference R_{i+1}.
            f32x4 y2d, x2d, y2o = z, x2o = z;
#pragma unroll
            for (int i2 = i; i2 < 4; ++i2) {
                unsigned dwv[4], ewv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int t = 16 * i2 + 4 * lg + u;
                    dwv[u] = sD[t * LDA + 16 * i + lr];
                    ewv[u] = sE[t * LDA + 16 * i + lr];
                }
                const f32x4 tY = mma16x3(z, unpack_hl(dwv[0], dwv[1], dwv[2], dwv[3]), qp[i2]);
                const f32x4 tX = mma16x3(z, unpack_hl(ewv[0], ewv[1], ewv[2], ewv[3]), kp[i2]);
                if (i2 == i) {
                    y2d = tY;
                    x2d = tX;
                } else {
                    const float f = i2 == i + 1 ? 1.f : xr[i2][i + 1];
                    y2o += f * tY;
                    x2o += f * tX;
                }
            }
            const float gi = i < 3 ? xr[i + 1][i] : 1.f;     // e^{R_{i+1} - R_i}
            // epilogue on tokens t = 16 i + 4 lg + e, channel cw
            float colpart = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * i + 4 * lg + e;
                const float g = gl[i][e];
                const float eg = fast_exp2(g), egc = fast_exp2(RC - g);
                const float Y1 = ep[i][e] * y1[e], X1 = ep[i][e] * x1[e];
                const float Y2 = em[i][e] * (y2d[e] + gi * y2o[e]);
                const float X2 = em[i][e] * (x2d[e] + gi * x2o[e]);
                const float kk = kv[i][e], qq = qv[i][e];
                // dq = dQh e^G + Y1,  dk = (dKh e^G + X1) + dKb e^{G_C - G} + (X2 + Y2), and
                // dG = dQh q e^G + dKh k e^G - dKb k e^{G_C - G} + k (X1 - X2 - Y2) + q Y1
                //    = q dq + k ((dKh e^G + X1) - dKb e^{G_C - G} - (X2 + Y2))
                const float dq = qh[i][e] * eg + Y1;
                const float a1 = dkh[i][e] * eg + X1, bv = kb[i][e] * egc, cv = X2 + Y2;
                dgr[i][e] = qq * dq + kk * (a1 - bv - cv);
                colpart += kk * bv;
                buf_st_bf16(rdq, (unsigned)(t * rowK + cw) * 2u, dq);
                buf_st_bf16(rdk, (unsigned)(t * rowK + cw) * 2u, a1 + bv + cv);
            }
            colpart += __shfl_xor(colpart, 16);
            colpart += __shfl_xor(colpart, 32);
            if (lg == 0) sCS[i * K + cw] = colpart;
        }
    }
    __syncthreads();                              // Ak^T and D are no longer read: dG goes over them
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) sDG[(16 * i + 4 * lg + e) * LDDG + cw] = dgr[i][e];
    __syncthreads();

    // ---- stage 8: dg = mask * (reverse cumsum of dG over the chunk + the G_C terms) ---
    {
        // four threads per channel, each on a 16-token block
        const int c = tid >> 2, part = tid & 3;
        float dv16[16], sum = 0.f;
#pragma unroll
        for (int i = 15; i >= 0; --i) {
            dv16[i] = sDG[(16 * part + i) * LDDG + c];
            sum += dv16[i];
        }
        const int base = l & ~3;
        float tot = sTot[3 * K + c] + sCS[c] + sCS[K + c] + sCS[2 * K + c] + sCS[3 * K + c];
#pragma unroll
        for (int q = 3; q >= 1; --q) {
            const float sq = __shfl(sum, base + q);
            if (q > part) tot += sq;
        }
        const __amdgpu_buffer_rsrc_t rdg = tok_rsrc(p.dg, p, b, h, t0, nt, K);   // rows past nt dropped
        const unsigned pass = sM[c * 4 + part];
#pragma unroll
        for (int i = 15; i >= 0; --i) {
            tot += dv16[i];
            buf_st_bf16(rdg, (unsigned)((16 * part + i) * rowK + c) * 2u, ((pass >> i) & 1u) ? tot : 0.f);
        }
    }
}

// ---- launchers ---------------------------------------------------------------------
template <typename T, int K, int V>
static hipError_t launch_bwd_chunk_t(int stage, const BwdParams& p, hipStream_t stream) {
    const long n = (long)p.B * p.H * p.NC;
    if (n <= 0) return hipSuccess;
    if (n > 2000000000L) return hipErrorInvalidValue;
    if (stage == 0)
        // persistent, one workgroup per CU (its LDS allows no second)
        hipLaunchKernelGGL((kda_bwd_vside_kernel<T, K, V>), dim3((unsigned)(p.n_cus > 0 && p.n_cus < n ? p.n_cus : n)),
                           dim3(512), 0, stream, p);
    else if (stage == 1)
        hipLaunchKernelGGL((kda_bwd_ksolve_kernel<T, K, V>), dim3((unsigned)n), dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL((kda_bwd_kgrad_kernel<T, K, 64>), dim3((unsigned)(n * (K / 64))), dim3(512), 0, stream, p);
    return hipGetLastError();
}

bool bwd_chunk_variant_exists(int dtype, int K, int V) {
    const bool kv = (K == 64 || K == 128) && (V == 64 || V == 128);
    if (dtype == 1) return kv;
    if (dtype == 0) return K == 64 && V == 64;
    return false;
}

hipError_t launch_bwd_chunk(int stage, int dtype, int K, int V, const BwdParams& p, hipStream_t stream) {
    if (stage < 0 || stage > 2) return hipErrorInvalidValue;
    if (dtype == 1) {
        if (K == 128 && V == 128) return launch_bwd_chunk_t<bf16, 128, 128>(stage, p, stream);
        if (K == 128 && V == 64) return launch_bwd_chunk_t<bf16, 128, 64>(stage, p, stream);
        if (K == 64 && V == 128) return launch_bwd_chunk_t<bf16, 64, 128>(stage, p, stream);
        if (K == 64 && V == 64) return launch_bwd_chunk_t<bf16, 64, 64>(stage, p, stream);
    } else if (dtype == 0) {
        if (K == 64 && V == 64) return launch_bwd_chunk_t<float, 64, 64>(stage, p, stream);
    }
    return hipErrorInvalidValue;
}

bool bwd_fused_variant_exists(int dtype, int K, int V) { return dtype == 1 && K == 128 && V == 128; }

__global__ __launch_bounds__(256) void kda_to_bf16_kernel(const float* src, bf16* dst, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = (bf16)src[i];
}

hipError_t launch_to_bf16(const float* src, void* dst, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(kda_to_bf16_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream, src,
                       reinterpret_cast<bf16*>(dst), n);
    return hipGetLastError();
}

hipError_t launch_bwd_fused(const BwdParams& p, hipStream_t stream) {
    const long n = (long)p.B * p.H * p.NC;
    if (n <= 0) return hipSuccess;
    if (n > 2000000000L) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kda_bwd_fused_kernel, dim3((unsigned)n), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kda
