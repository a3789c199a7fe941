// Split chunked KDA prefill for gfx950.
//
// Intra-chunk pass: every (batch, head, chunk) at once, independent of the
// state: gate cumsum, intra-chunk similarities, the UT solve, and the chunk's
// operands of the state pass written to a workspace record.
// State pass: per (batch, head, segment, value-column block), the chunks in
// order: U = U~ - W S, O = (Q e^G) S + Mqk U, S <- Diag(e^{G_C}) S + (K e^{G_C-G})^T U.
//
// Page: "Kimi K3 — открытая модель, которая обошла закрытых лидеров рынка"
// (aiblin.ru), section "Как распараллелили последовательное обновление": the
// tokens of a chunk are handled together and only the state is passed from
// chunk to chunk; here the chunk-local part runs for all chunks side by side,
// so only the state pass is sequential.  The chunk-form algebra and the
// sub-chunk split of the gate exponents are those of the single-pass kernel.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = kChunk;

constexpr int cmax(int a, int b) { return a > b ? a : b; }

__device__ __forceinline__ void offdiag_pair(int p, int& i, int& j) {
    i = (p >= 3) ? 3 : (p >= 1) ? 2 : 1;
    j = p - i * (i - 1) / 2;
}
__device__ __forceinline__ void lower_pair(int p, int& i, int& j) {
    i = (p >= 6) ? 3 : (p >= 3) ? 2 : (p >= 1) ? 1 : 0;
    j = p - i * (i + 1) / 2;
}

template <typename T>
__device__ __forceinline__ void ld8_as_f32(const T* p, float* x) {
    typename FragOf<T>::type f = ld_frag<T>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = to_f32(f[i]);
}

// column side of block pair (i, j) for the 32-deep slab at channel c0
template <typename T, int LDK1, int K>
__device__ __forceinline__ typename FragOf<T>::type col_frag(const T* sKinv, const float* sF, int i, int j,
                                                            int lr, int c0) {
    if (i == j) return ld_frag<T>(&sKinv[(16 * j + lr) * LDK1 + c0]);
    float kv[8], f[8];
    ld8_as_f32<T>(&sKinv[(16 * j + lr) * LDK1 + c0], kv);
    ld8f(&sF[(i * (i - 1) / 2 + j) * K + c0], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) kv[e] *= f[e];
    return frag_from<T>(kv);
}

// token range [s0, s1) of sequence i of a packed batch; out-of-range offsets
// are clamped so that every access stays inside the T_total rows
__device__ __forceinline__ void seq_range(const int* cu, int i, int T_total, int& s0, int& s1) {
    s0 = min(max(cu[i], 0), T_total);
    s1 = max(s0, min(max(cu[i + 1], 0), T_total));
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));


// 4 values of T as one 8- (bf16) or 16-byte (fp32) global store
__device__ __forceinline__ void st4(bf16* p, const float* x) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (bf16)x[i];
    *reinterpret_cast<bf16x4*>(p) = r;
}
__device__ __forceinline__ void st4(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

}  // namespace

// ============================================================================
// Intra-chunk pass
// ============================================================================
// Eight waves; wave w prepares tokens [8w, 8w + 8) of the chunk, so that each
// load instruction reads whole rows (CG lanes x 16 bytes per token row) of
// q, k, g and v.  The per-channel gate cumsum crosses waves through a small
// LDS table of wave totals.  Outputs leave as whole rows too: Q e^{G} straight
// from registers, everything else staged in LDS.
// The channel-major [channel][token] LDS arrays of the intra-chunk pass keep
// token t of channel row r at column t ^ (8 ((r >> 4) & 7)): 8-token units
// are permuted per 16-row group, so that the column-wise writes of the
// preparation phase (lanes on rows 8 apart) spread over all LDS banks while
// 4- and 8-token runs stay contiguous.
__device__ __forceinline__ int swz_t(int r, int t) { return t ^ (((r >> 4) & 7) << 3); }

template <typename T, int K, int V>
struct IntraLayout {
    static constexpr int NW = 8;                 // waves
    static constexpr int NT = 64 * NW;
    static constexpr int TPW = C / NW;           // tokens per wave (8)
    static constexpr int SZ = (int)sizeof(T);
    static constexpr int PAD = 16 / SZ;
    static constexpr int LDK1 = K + PAD;         // Kd, Qd, Kinv, W: [token][channel]
    static constexpr int LDT = C + PAD;          // [channel][token]
    static constexpr int LDL = C + 4;            // solve blocks / Mqk
    static constexpr int LDD = 16;
    // key side: CG lanes of 8 channels per token row, RPI rows per
    // instruction, TPL consecutive tokens per lane; value side likewise
    static constexpr int CG = K / 8, RPI = 64 / CG, TPL = TPW / RPI;
    static constexpr int CGV = V / 8, RPIV = 64 / CGV, TPLV = TPW / RPIV;
    static constexpr int CT = K / 16, NVT = V / 16;
    static constexpr int KQ = 3 * C * LDK1 * SZ;         // Kd | Qd | Kinv, then W staging
    static constexpr int L_BYTES = C * LDL * SZ;
    static constexpr int R = L_BYTES + 4 * 16 * LDD * 4;
    static constexpr int oKQ = 0;
    static constexpr int oR = oKQ + KQ;                  // solve blocks | fp32 diagonal blocks of A (transposed)
    static constexpr int oMqk = oR + R;
    static constexpr int oKhbT = oMqk + C * LDL * SZ;    // [K][LDT] beta K e^{G}
    static constexpr int oVbT = oKhbT + K * LDT * SZ;    // [V][LDT] beta V, then U~^T
    static constexpr int oKbT = oVbT + V * LDT * SZ;     // [K][LDT] (K e^{G_C-G})^T
    static constexpr int oF = oKbT + K * LDT * SZ;       // fp32 [7][K] e^{G_b(i) - G_b(j)}; row 6: ones
    static constexpr int oWT = oF + 7 * K * 4;           // fp32 [NW][K] wave totals of clamped gates
    static constexpr int oG0 = oWT + NW * K * 4;         // fp32 [NW][K] first token's clamped gate
    static constexpr int oBeta = oG0 + NW * K * 4;       // fp32 [C]
    static constexpr int TOTAL = oBeta + C * 4;
    // per-channel table of the preparation phase, over the solve blocks (free
    // until P2): exclusive prefix before each wave [NW][K], then G_b, e^{G_b},
    // e^{G_C - G_b} of each block [4][K] each
    static constexpr int oTab = oR;
    static constexpr int TAB = (NW + 12) * K * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
    static_assert(TAB <= R, "prefix table must fit the solve-block region");
    static_assert(NT % K == 0, "whole threads per channel in the prefix table");
    static_assert(CG * RPI == 64 && RPI * TPL == TPW && TPL >= 1, "key prep mapping");
    static_assert(CGV * RPIV == 64 && RPIV * TPLV == TPW && TPLV >= 1, "value prep mapping");
    static_assert(TPW * NW == C && TPW == 8, "two waves per 16-token block");
};

template <typename T, int K, int V>
__global__ __launch_bounds__(512) void kda_intra_kernel(IntraParams p) {
    using L = IntraLayout<T, K, V>;
    constexpr int NW = L::NW, NT = L::NT;
    using Frag4 = typename Frag4Of<T>::type;
    constexpr int LDK1 = L::LDK1, LDT = L::LDT, LDL = L::LDL, LDD = L::LDD;
    constexpr int CG = L::CG, TPL = L::TPL, CGV = L::CGV, TPLV = L::TPLV;
    constexpr int CT = L::CT, NVT = L::NVT;
    constexpr int KS = K / 32;
    constexpr unsigned SZ = sizeof(T);
    constexpr RecLayout RL = rec_layout(K, V, (int)sizeof(T));

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
    T* sKd = reinterpret_cast<T*>(smem + L::oKQ);
    T* sQd = sKd + C * LDK1;
    T* sKinv = sQd + C * LDK1;
    T* sW = reinterpret_cast<T*>(smem + L::oKQ);
    T* sL = reinterpret_cast<T*>(smem + L::oR);
    float* sAd = reinterpret_cast<float*>(smem + L::oR + L::L_BYTES);
    T* sMqk = reinterpret_cast<T*>(smem + L::oMqk);
    T* sKhbT = reinterpret_cast<T*>(smem + L::oKhbT);
    T* sVbT = reinterpret_cast<T*>(smem + L::oVbT);
    T* sKbT = reinterpret_cast<T*>(smem + L::oKbT);
    float* sF = reinterpret_cast<float*>(smem + L::oF);
    float* sWT = reinterpret_cast<float*>(smem + L::oWT);
    float* sG0 = reinterpret_cast<float*>(smem + L::oG0);
    float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);
    float* tPre = reinterpret_cast<float*>(smem + L::oTab);
    float* tGb = tPre + NW * K;
    float* tEgb = tGb + 4 * K;
    float* tEcb = tEgb + 4 * K;

    const int w0 = threadIdx.x >> 6, l0 = threadIdx.x & 63;

    const T* __restrict__ qg = reinterpret_cast<const T*>(p.q);
    const T* __restrict__ kg = reinterpret_cast<const T*>(p.k);
    const T* __restrict__ vg = reinterpret_cast<const T*>(p.v);
    const T* __restrict__ gg = reinterpret_cast<const T*>(p.g);
    const T* __restrict__ bg = reinterpret_cast<const T*>(p.beta);

    // lane roles: key side channels [c0, c0 + 8) of tokens t1 .. t1 + TPL - 1;
    // value side columns [n0, n0 + 8) of tokens tv .. tv + TPLV - 1
    const int t1_ = L::TPW * w0 + TPL * (l0 / CG), tv_ = L::TPW * w0 + TPLV * (l0 / CGV);

    // beta: lane l < 8 of wave w holds that of token 8 w + l
    Pack8<T> kr[TPL], qr[TPL], gr[TPL], vr[TPLV];
    T bw;
    const unsigned rowK = (unsigned)p.H * K * SZ, rowV = (unsigned)p.H * V * SZ, rowB = (unsigned)p.H * SZ;
    const unsigned vK = (unsigned)t1_ * rowK + (unsigned)(8 * (l0 % CG)) * SZ;
    const unsigned vV = (unsigned)tv_ * rowV + (unsigned)(8 * (l0 % CGV)) * SZ;
    const int tb_ = L::TPW * w0 + l0;
    const unsigned vB = (unsigned)tb_ * rowB;
    // where an item's tokens are: first [T][H] row of head h and the number of tokens
    auto locate = [&](int item, size_t& head_row, int& nt) {
        if (p.cu_seqlens) {
            // packed batch: item = h * NC + global chunk; find its sequence
            const int h = item / p.NC, gc = item - h * p.NC;
            int t0 = 0;
            nt = 0;
            if (gc < p.chunk_off[p.N]) {
                int lo = 0, hi = p.N;              // chunk_off[lo] <= gc < chunk_off[hi]
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (p.chunk_off[mid] <= gc) lo = mid; else hi = mid;
                }
                int s0, s1;
                seq_range(p.cu_seqlens, lo, p.T, s0, s1);
                t0 = s0 + (gc - p.chunk_off[lo]) * C;
                nt = max(0, min(C, s1 - t0));
            }
            head_row = (size_t)t0 * p.H + h;
        } else {
            const int bh = item / p.NC, ci = item - bh * p.NC;
            const int b = bh / p.H, h = bh - b * p.H;
            const int t0 = ci * C;
            nt = min(C, p.T - t0);
            head_row = (size_t)(b * (size_t)p.T + t0) * p.H + h;
        }
    };
    // the loads of an item: gates and keys, queries, values and beta
    auto load_gk = [&](size_t head_row, int nt) {
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + head_row * K);
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(gg + head_row * K);
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            if (t1_ + i < nt) {
                buf_load8<T>(gr[i], rg, vK, i * rowK);
                buf_load8<T>(kr[i], rk, vK, i * rowK);
            } else {
                gr[i].zero();
                kr[i].zero();
            }
        }
    };
    auto load_q = [&](size_t head_row, int nt) {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg + head_row * K);
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            if (t1_ + i < nt) buf_load8<T>(qr[i], rq, vK, i * rowK);
            else qr[i].zero();
        }
    };
    auto load_vb = [&](size_t head_row, int nt) {
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + head_row * V);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(bg + head_row);
#pragma unroll
        for (int i = 0; i < TPLV; ++i) {
            if (tv_ + i < nt) buf_load8<T>(vr[i], rv, vV, i * rowV);
            else vr[i].zero();
        }
        if (l0 < L::TPW && tb_ < nt) buf_load1(bw, rb, vB, 0u);
        else bw = from_f32<T>(0.f);
    };

    const int G = gridDim.x;
    // the row of ones of sF (scale of the diagonal block pairs)
    for (int c = threadIdx.x; c < K; c += NT) sF[6 * K + c] = 1.f;
    size_t nrow = 0;
    int nnt = 0;
    if ((int)blockIdx.x < p.n_items) {
        locate(blockIdx.x, nrow, nnt);
        load_gk(nrow, nnt);
        load_q(nrow, nnt);
        load_vb(nrow, nnt);
    }

    for (int item = blockIdx.x; item < p.n_items; item += G) {
        unsigned char* rec = p.rec + (size_t)item * RL.bytes;
        const __amdgpu_buffer_rsrc_t rrec = make_rsrc(rec);
        // lane indices redone per item (opaque() keeps the index arithmetic
        // derived from them out of the loop preheader)
        const int tid = opaque((int)threadIdx.x);
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, lg = l >> 4, lr = l & 15;
        const int c0 = 8 * (l % CG), t1 = L::TPW * w + TPL * (l / CG);
        const int n0 = 8 * (l % CGV), tv = L::TPW * w + TPLV * (l / CGV);

        // ---- P1a: clamped log gates, in-lane and in-wave inclusive sums ----------
        float run[8], tot[8];
        float c[TPL][8];                             // clamped log2 gates, reused in P1b
        {
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                float g8[8];
                gr[i].to_f32(g8);
#pragma unroll
                for (int e = 0; e < 8; ++e) c[i][e] = clamp_gate_log2(g8[e]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < TPL; ++i) s += c[i][e];
                tot[e] = s;
            }
            // scan over the lanes holding the same channels (token order)
            float incl[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) incl[e] = tot[e];
#pragma unroll
            for (int d = CG; d < 64; d <<= 1) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float y = __shfl_up(incl[e], d);
                    if (l >= d) incl[e] += y;
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) run[e] = incl[e] - tot[e];   // in-wave sum before this lane's tokens
            // wave totals (last lanes) and the wave's first-token gates (first lanes)
            if (l >= 64 - CG) {
                st8(&sWT[w * K + c0], incl);
            }
            if (l < CG) {
                float c0v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) c0v[e] = c[0][e];
                st8(&sG0[w * K + c0], c0v);
            }
            if (l < L::TPW) sBeta[L::TPW * w + l] = to_f32(bw);
        }
        __syncthreads();

        // ---- P1t: per-channel table (prefix over waves, block references, factors) --
        {
            constexpr int P = NT / K;                     // threads per channel
            const int ch = tid % K, part = tid / K;
            float pfx[NW + 1];                            // pfx[v]: sum of the totals of waves < v
            pfx[0] = 0.f;
#pragma unroll
            for (int v = 0; v < NW; ++v) pfx[v + 1] = pfx[v] + sWT[v * K + ch];
#pragma unroll
            for (int v = 0; v < NW; ++v)
                if (v % P == part) tPre[v * K + ch] = pfx[v];
            // G_b: G at the first token of block b (the first token of wave 2 b)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (b % P == part) {
                    const float gbv = pfx[2 * b] + sG0[2 * b * K + ch];
                    tGb[b * K + ch] = gbv;
                    tEgb[b * K + ch] = fast_exp2(gbv);                 // e^{G_b}       <= 1
                    tEcb[b * K + ch] = fast_exp2(pfx[NW] - gbv);       // e^{G_C - G_b} <= 1
                }
            // e^{G_b(i) - G_b(j)} of the six off-diagonal block pairs
#pragma unroll
            for (int f = 0; f < 6; ++f)
                if (f % P == part) {
                    int bi, bj;
                    offdiag_pair(f, bi, bj);
                    const float gi = pfx[2 * bi] + sG0[2 * bi * K + ch];
                    const float gj = pfx[2 * bj] + sG0[2 * bj * K + ch];
                    sF[f * K + ch] = fast_exp2(gi - gj);
                }
            if (part == P - 1) buf_store1(rrec, (unsigned)RL.oEgc + (unsigned)ch * 4u, 0u, fast_exp2(pfx[NW]));
        }
        // value side (needs only beta): beta V, channel-major
        {
            float bv[8][TPLV];
#pragma unroll
            for (int i = 0; i < TPLV; ++i) {
                float vx[8];
                vr[i].to_f32(vx);
                const float bt = sBeta[tv + i];
#pragma unroll
                for (int e = 0; e < 8; ++e) bv[e][i] = bt * vx[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) st_small<TPLV>(&sVbT[(n0 + e) * LDT + swz_t(n0 + e, tv)], bv[e]);
        }
        __syncthreads();

        // ---- P1b: operands ---------------------------------------------------------------
        {
            float pre[8], gb[8], egb[8], ecb[8];
            const int myblk = w >> 1;
            ld8f(&tPre[w * K + c0], pre);
            ld8f(&tGb[myblk * K + c0], gb);
            ld8f(&tEgb[myblk * K + c0], egb);
            ld8f(&tEcb[myblk * K + c0], ecb);
            float kh[8][TPL], kb[8][TPL];
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const int t = t1 + i;
                float kx[8], qx[8], kd[8], ki[8], qd[8], qh[8];
                kr[i].to_f32(kx);
                qr[i].to_f32(qx);
                const float bt = sBeta[t1 + i];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    run[e] += c[i][e];
                    const float d = pre[e] + run[e] - gb[e];   // G_t - G_b in [-108, 0] (log2)
                    const float e1 = fast_exp2(d);             // e^{G_t - G_b} <= 1
                    const float e2 = fast_exp2(-d);            // e^{G_b - G_t} <= e^75
                    kd[e] = kx[e] * e1;
                    ki[e] = kx[e] * e2;
                    kh[e][i] = bt * kd[e] * egb[e];            // beta k e^{G_t}
                    kb[e][i] = ki[e] * ecb[e];                 // k e^{G_C - G_t}
                    qd[e] = qx[e] * e1;                        // q e^{G_t - G_b}
                    qh[e] = qd[e] * egb[e];                    // q e^{G_t}
                }
                st8(&sKd[t * LDK1 + c0], kd);
                st8(&sKinv[t * LDK1 + c0], ki);
                st8(&sQd[t * LDK1 + c0], qd);
                // Q e^{G}: CG lanes write one whole token row
                if constexpr (sizeof(T) == 2) {
                    const auto qf = frag_from<T>(qh);
                    buf_store16(rrec, (unsigned)RL.oQh + (unsigned)(t * K + c0) * SZ, 0u,
                                *reinterpret_cast<const uint4*>(&qf));
                } else {
                    buf_store16(rrec, (unsigned)RL.oQh + (unsigned)(t * K + c0) * SZ, 0u,
                                *reinterpret_cast<const uint4*>(&qh[0]));
                    buf_store16(rrec, (unsigned)RL.oQh + (unsigned)(t * K + c0) * SZ + 16u, 0u,
                                *reinterpret_cast<const uint4*>(&qh[4]));
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                st_small<TPL>(&sKhbT[(c0 + e) * LDT + swz_t(c0 + e, t1)], kh[e]);
                st_small<TPL>(&sKbT[(c0 + e) * LDT + swz_t(c0 + e, t1)], kb[e]);
            }
        }
        __syncthreads();

        // the raw registers are free: fetch the next item, waves 0-3 here and
        // waves 4-7 behind P2, so that half of the loads queue at a time
        __builtin_amdgcn_sched_barrier(0);
        if (item + G < p.n_items) locate(item + G, nrow, nnt);
        if (w < 4 && item + G < p.n_items) {
            load_gk(nrow, nnt);
            load_q(nrow, nnt);
            load_vb(nrow, nnt);
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- P2: diagonal blocks of A and their inverses; off-diagonal A; Mqk ----
        // wave 0: the four diagonal blocks and their inverses, and the zero
        // blocks of Mqk; waves 1-7: the off-diagonal blocks of A and the lower
        // blocks of Mqk
        if (w == 0) {
            // A_ii, transposed into sAd: sAd[i][m][r] = A_ii[r][m]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = mma(acc, ld_frag<T>(&sKd[(16 * i + lr) * LDK1 + 32 * ks + 8 * lg]),
                              ld_frag<T>(&sKinv[(16 * i + lr) * LDK1 + 32 * ks + 8 * lg]));
                const f32x4 bt = *reinterpret_cast<const f32x4*>(&sBeta[16 * i + 4 * lg]);
                f32x4 a4;
#pragma unroll
                for (int e = 0; e < 4; ++e) a4[e] = (lr < 4 * lg + e) ? bt[e] * acc[e] : 0.f;
                *reinterpret_cast<f32x4*>(&sAd[(i * 16 + lr) * LDD + 4 * lg]) = a4;
            }
            wave_lds_sync();
            // lane (block lg, column lr) of (I + A_ii)^{-1} by right-looking
            // forward substitution: when x[m] is final, remove its part from
            // every later row
            const float* At = sAd + lg * 16 * LDD;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == lr) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 15; ++m) {
                float col[16];
#pragma unroll
                for (int q4 = m / 4; q4 < 4; ++q4) {
                    const f32x4 c4 = *reinterpret_cast<const f32x4*>(&At[m * LDD + 4 * q4]);
                    col[4 * q4] = c4[0];
                    col[4 * q4 + 1] = c4[1];
                    col[4 * q4 + 2] = c4[2];
                    col[4 * q4 + 3] = c4[3];
                }
#pragma unroll
                for (int r = m + 1; r < 16; ++r) x[r] -= col[r] * x[m];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sL[(16 * lg + r) * LDL + 16 * lg + lr] = from_f32<T>(x[r]);
            // the blocks of Mqk above the diagonal are zero
#pragma unroll
            for (int q = 0; q < 6; ++q) {
                const int i = (q < 3) ? 0 : (q < 5) ? 1 : 2;
                const int j = (q < 3) ? q + 1 : (q < 5) ? q - 1 : 3;
#pragma unroll
                for (int e = 0; e < 4; ++e) sMqk[(16 * i + 4 * lg + e) * LDL + 16 * j + lr] = from_f32<T>(0.f);
            }
        } else {
            // the sixteen blocks over waves 1-7, two or three each (tasks 0-5:
            // off-diagonal blocks of -A, into the solve buffer; 6-15: blocks of
            // Mqk); every task runs branch-free: a diagonal pair scales by the
            // row of ones in sF, so that the scheduler can overlap a wave's tasks
            auto task_ops = [&](int task, typename FragOf<T>::type (&fa)[KS], typename FragOf<T>::type (&fb)[KS]) {
                int i, j;
                if (task < 6) offdiag_pair(task, i, j);
                else lower_pair(task - 6, i, j);
                const T* rowsrc = (task < 6) ? sKd : sQd;
                const int frow = (i == j) ? 6 : i * (i - 1) / 2 + j;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int cc = 32 * ks + 8 * lg;
                    fa[ks] = ld_frag<T>(&rowsrc[(16 * i + lr) * LDK1 + cc]);
                    float kv[8], f[8];
                    ld8_as_f32<T>(&sKinv[(16 * j + lr) * LDK1 + cc], kv);
                    ld8f(&sF[frow * K + cc], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) kv[e] *= f[e];
                    fb[ks] = frag_from<T>(kv);
                }
            };
            auto task_out = [&](int task, const typename FragOf<T>::type (&fa)[KS],
                                const typename FragOf<T>::type (&fb)[KS]) {
                int i, j;
                if (task < 6) offdiag_pair(task, i, j);
                else lower_pair(task - 6, i, j);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = mma(acc, fa[ks], fb[ks]);
                const f32x4 bt = *reinterpret_cast<const f32x4*>(&sBeta[16 * i + 4 * lg]);
                T* dst = (task < 6) ? sL : sMqk;
                const int r = 16 * j + lr;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s_ = 16 * i + 4 * lg + e;
                    const float val = (task < 6) ? -bt[e] * acc[e] : ((i > j || r <= s_) ? acc[e] : 0.f);
                    dst[s_ * LDL + r] = from_f32<T>(val);
                }
            };
            // per wave 1..7: tasks (t0, t1[, t2])
            const int t0 = (w <= 3) ? 2 * (w - 1) : (w == 4) ? 7 : (w == 5) ? 10 : (w == 6) ? 13 : 14;
            const int t1 = (w <= 3) ? 2 * (w - 1) + 1 : (w == 4) ? 9 : (w == 5) ? 12 : (w == 6) ? 6 : 11;
            typename FragOf<T>::type fa0[KS], fb0[KS], fa1[KS], fb1[KS];
            task_ops(t0, fa0, fb0);
            task_ops(t1, fa1, fb1);
            task_out(t0, fa0, fb0);
            task_out(t1, fa1, fb1);
            if (w >= 6) {
                const int t2 = (w == 6) ? 8 : 15;
                task_ops(t2, fa0, fb0);
                task_out(t2, fa0, fb0);
            }
        }
        __syncthreads();

        __builtin_amdgcn_sched_barrier(0);
        if (w >= 4 && item + G < p.n_items) {
            load_gk(nrow, nnt);
            load_q(nrow, nnt);
            load_vb(nrow, nnt);
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- P3: W and U~ tiles by block forward substitution -------------------------
        {
            Frag4 Ld[4], Lo[6];
#pragma unroll
            for (int i = 0; i < 4; ++i) Ld[i] = ld_frag4<T>(&sL[(16 * i + lr) * LDL + 16 * i + 4 * lg]);
#pragma unroll
            for (int q6 = 0; q6 < 6; ++q6) {
                const int i = (q6 >= 3) ? 3 : (q6 >= 1) ? 2 : 1;
                const int k = q6 - i * (i - 1) / 2;
                Lo[q6] = ld_frag4<T>(&sL[(16 * i + lr) * LDL + 16 * k + 4 * lg]);
            }
            // X = (I + A)^{-1} R for 16-column tile tl; R read from the
            // channel-major rows rhs[lr][token] of that tile
            auto solve_tile = [&](const T* rhs, int tl, f32x4* X) {
                Frag4 Xb[4];
                f32x4 R[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) R[i] = ld4_as_f32<T>(rhs + lr * LDT + swz_t(16 * tl, 16 * i + 4 * lg));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4 acc = R[i];
#pragma unroll
                    for (int k = 0; k < i; ++k) acc = mma16(acc, Lo[i * (i - 1) / 2 + k], Xb[k]);
                    X[i] = mma16(f32x4{0.f, 0.f, 0.f, 0.f}, Ld[i], frag4_from<T>(acc));
                    Xb[i] = frag4_from<T>(X[i]);
                }
            };
            // two tiles, their dependency chains interleaved
            auto solve_two = [&](const T* ra, int ta, const T* rb, int tb, f32x4* XA, f32x4* XB) {
                Frag4 Xa[4], Xc[4];
                f32x4 RA[4], RB[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    RA[i] = ld4_as_f32<T>(ra + lr * LDT + swz_t(16 * ta, 16 * i + 4 * lg));
                    RB[i] = ld4_as_f32<T>(rb + lr * LDT + swz_t(16 * tb, 16 * i + 4 * lg));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4 acca = RA[i], accb = RB[i];
#pragma unroll
                    for (int k = 0; k < i; ++k) {
                        acca = mma16(acca, Lo[i * (i - 1) / 2 + k], Xa[k]);
                        accb = mma16(accb, Lo[i * (i - 1) / 2 + k], Xc[k]);
                    }
                    XA[i] = mma16(f32x4{0.f, 0.f, 0.f, 0.f}, Ld[i], frag4_from<T>(acca));
                    XB[i] = mma16(f32x4{0.f, 0.f, 0.f, 0.f}, Ld[i], frag4_from<T>(accb));
                    Xa[i] = frag4_from<T>(XA[i]);
                    Xc[i] = frag4_from<T>(XB[i]);
                }
            };
            // tile u < CT: W columns [16 u, 16 u + 16) from beta K e^{G}; else
            // U~ tile u - CT from beta V
            auto tile_rhs = [&](int u) -> const T* {
                return u < CT ? &sKhbT[16 * u * LDT] : &sVbT[16 * (u - CT) * LDT];
            };
            auto tile_out = [&](int u, const f32x4* X) {
                if (u < CT) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sW[(16 * i + 4 * lg + e) * LDK1 + 16 * u + lr] = from_f32<T>(X[i][e]);
                } else {
                    // U~ written back over this tile's (consumed) beta V rows, transposed
                    const int vt = u - CT;
                    T* rows = &sVbT[16 * vt * LDT];
                    wave_lds_sync();
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float x4[4] = {X[i][0], X[i][1], X[i][2], X[i][3]};
                        st_small<4>(&rows[lr * LDT + swz_t(16 * vt, 16 * i + 4 * lg)], x4);
                    }
                }
            };
            static_assert(CT + NVT <= 2 * NW, "at most two tiles per wave");
            const int u0 = w, u1 = w + NW;
            if (u1 < CT + NVT) {
                f32x4 XA[4], XB[4];
                solve_two(tile_rhs(u0), u0 < CT ? u0 : u0 - CT, tile_rhs(u1), u1 < CT ? u1 : u1 - CT, XA, XB);
                tile_out(u0, XA);
                tile_out(u1, XB);
            } else if (u0 < CT + NVT) {
                f32x4 X[4];
                solve_tile(tile_rhs(u0), u0 < CT ? u0 : u0 - CT, X);
                tile_out(u0, X);
            }
        }
        __syncthreads();

        // ---- record rows out, 16 bytes at a time: W, Mqk, (K e^{G_C-G})^T, U~^T -----
        {
            constexpr int E = 16 / (int)SZ;                  // elements per piece
            constexpr int PW = K * (int)SZ / 16, PC = C * (int)SZ / 16;
            static_assert((C * PW) % NT == 0 && (C * PC) % NT == 0 && (K * PC) % NT == 0 &&
                              (V * PC) % NT == 0, "record rows split evenly over the workgroup");
#pragma unroll
            for (int j = 0; j < C * PW / NT; ++j) {
                const int pc = tid + NT * j;
                buf_store16(rrec, (unsigned)RL.oW + (unsigned)pc * 16u, 0u,
                            *reinterpret_cast<const uint4*>(&sW[(pc / PW) * LDK1 + (pc % PW) * E]));
            }
#pragma unroll
            for (int j = 0; j < C * PC / NT; ++j) {
                const int pc = tid + NT * j;
                buf_store16(rrec, (unsigned)RL.oMqk + (unsigned)pc * 16u, 0u,
                            *reinterpret_cast<const uint4*>(&sMqk[(pc / PC) * LDL + (pc % PC) * E]));
            }
#pragma unroll
            for (int j = 0; j < K * PC / NT; ++j) {
                const int pc = tid + NT * j;
                buf_store16(rrec, (unsigned)RL.oKbT + (unsigned)pc * 16u, 0u,
                            *reinterpret_cast<const uint4*>(&sKbT[(pc / PC) * LDT + swz_t(pc / PC, (pc % PC) * E)]));
            }
#pragma unroll
            for (int j = 0; j < V * PC / NT; ++j) {
                const int pc = tid + NT * j;
                buf_store16(rrec, (unsigned)RL.oUtT + (unsigned)pc * 16u, 0u,
                            *reinterpret_cast<const uint4*>(&sVbT[(pc / PC) * LDT + swz_t(pc / PC, (pc % PC) * E)]));
            }
        }
        __syncthreads();
    }
}

// ============================================================================
// State pass
// ============================================================================
template <typename T, int K, int NW_, int NTW, bool SUMMARY>
struct StateLayout {
    static constexpr int NW = NW_;                       // waves; wave w owns NTW 16-column tiles
    static constexpr int NT = 64 * NW;
    static constexpr int VB = 16 * NW * NTW;
    static constexpr int SZ = (int)sizeof(T);
    static constexpr int PAD = 16 / SZ;
    static constexpr int LDK2 = K + PAD;     // W, Qh rows
    static constexpr int LDL = C + 4;        // Mqk rows
    static constexpr int LDT = C + PAD;      // KbT, UtT rows
    static constexpr int oW = 0;
    static constexpr int oQh = oW + C * LDK2 * SZ;
    static constexpr int oMqk = oQh + C * LDK2 * SZ;
    static constexpr int oKbT = oMqk + C * LDL * SZ;
    static constexpr int oUtT = oKbT + K * LDT * SZ;     // then: per-wave output staging
    static constexpr int oEGC = oUtT + VB * LDT * SZ;
    static constexpr int TOTAL = oEGC + K * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
    static_assert(C * 16 * NTW <= 16 * NTW * LDT, "output staging must fit the wave's U~ rows");
    // 16-byte pieces of one record the workgroup loads (the summary pass
    // computes no output and skips Qh and Mqk)
    static constexpr int PW = C * K * SZ / 16;           // W
    static constexpr int PQ = SUMMARY ? 0 : C * K * SZ / 16;   // Qh
    static constexpr int PM = SUMMARY ? 0 : C * C * SZ / 16;   // Mqk
    static constexpr int PK = K * C * SZ / 16;           // KbT
    static constexpr int PU = (SUMMARY && VB > K ? VB - K : VB) * C * SZ / 16;   // U~ rows of the block
    static constexpr int PE = K * 4 / 16;                // e^{G_C}
    static constexpr int E1 = PW, E2 = E1 + PQ, E3 = E2 + PM, E4 = E3 + PK, E5 = E4 + PU;
    static constexpr int PTOT = E5 + PE;
    static constexpr int NPT = (PTOT + NT - 1) / NT;     // pieces per thread
};

// OUT: the output pass computes and stores O (false: states and snapshots only);
// GATE: o is multiplied by sigmoid of the gate input
template <typename T, int K, int NW, int NTW, bool SUMMARY, bool OUT = !SUMMARY, bool GATE = false>
__global__ __launch_bounds__(64 * NW, (NW == 4 && NTW == 1 && sizeof(T) == 2 ? 2 : 1))
void kda_state_kernel(StateParams p) {
    using L = StateLayout<T, K, NW, NTW, SUMMARY>;
    using Frag = typename FragOf<T>::type;
    constexpr int VB = L::VB;
    constexpr int LDK2 = L::LDK2, LDL = L::LDL, LDT = L::LDT;
    constexpr int KS = K / 32, CT = K / 16;
    constexpr unsigned SZ = sizeof(T);
    constexpr int NPT = L::NPT;
    // 8-wave workgroups keep 256 registers per lane: operands are loaded per tile
    constexpr bool NARROW_REGS = NW == 8 && NTW == 2;

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
    T* sW = reinterpret_cast<T*>(smem + L::oW);
    T* sQh = reinterpret_cast<T*>(smem + L::oQh);
    T* sMqk = reinterpret_cast<T*>(smem + L::oMqk);
    T* sKbT = reinterpret_cast<T*>(smem + L::oKbT);
    T* sUtT = reinterpret_cast<T*>(smem + L::oUtT);
    float* sEGC = reinterpret_cast<float*>(smem + L::oEGC);

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, lg = l >> 4, lr = l & 15;

    const int G = gridDim.x;
    const int x = blockIdx.x;
    const int lid = ((G & 7) == 0) ? (x & 7) * (G >> 3) + (x >> 3) : x;
    const int vb = lid % p.n_vb;
    const int rest = lid / p.n_vb;
    const int nseg_here = SUMMARY && !p.summary_all ? p.n_seg - 1 : p.n_seg;
    const int seg = rest % nseg_here;
    const int bh = rest / nseg_here;
    const int b = bh / p.H, h = bh % p.H;
    const int BH = p.B * p.H;
    const int V = p.V;
    // token rows of this chain: [row0, row_end) in the [rows][H] layout, and
    // its records from rec_first on
    int c_begin, c_end;
    size_t row0, row_end, rec_first;
    if (p.cu_seqlens) {
        int s0, s1;
        seq_range(p.cu_seqlens, b, p.T, s0, s1);          // b = sequence index
        row0 = (size_t)s0;
        row_end = (size_t)s1;
        c_begin = 0;
        c_end = p.chunk_off[b + 1] - p.chunk_off[b];
        rec_first = (size_t)h * p.NC + p.chunk_off[b];
    } else {
        row0 = (size_t)b * p.T;
        row_end = row0 + p.T;
        c_begin = seg * p.cps;
        c_end = min(c_begin + p.cps, p.NC);
        rec_first = (size_t)bh * p.NC;
    }

    const int col0 = vb * VB;
    const int tile0 = NTW * w;
    // summary pass: columns below K carry the transition (identity start, no
    // U~), the others the load; a workgroup may hold both kinds (a wave holds
    // one).  The U~ rows staged are those of the value columns
    // [vcol0, vcol0 + nvcol) of this workgroup.
    const bool pmode = SUMMARY && col0 + 16 * tile0 < K;
    const int vcol0 = SUMMARY ? max(col0 - K, 0) : col0;
    const int nvcol = SUMMARY ? max(0, col0 + VB - max(col0, K)) : VB;
    const int urow0 = SUMMARY ? col0 + 16 * tile0 - K - vcol0 : 16 * tile0;   // this wave's first U~ row

    const RecLayout RL = rec_layout(K, V, (int)sizeof(T));
    const unsigned char* rec0 = p.rec + rec_first * RL.bytes;

    // ---- initial state --------------------------------------------------------
    f32x4 S[NTW][CT];
    {
        const float* src = nullptr;
        if (!SUMMARY) {
            if (seg == 0) src = p.s0 ? p.s0 + (size_t)bh * K * V : nullptr;
            else src = p.seg_init + ((size_t)(seg - 1) * BH + bh) * K * V;
        }
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int col = col0 + 16 * (tile0 + j) + lr;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * ct + 4 * lg + e;
                    float v0 = 0.f;
                    if (src) v0 = src[(size_t)row * V + col];
                    else if (pmode) v0 = (row == col) ? 1.f : 0.f;
                    S[j][ct][e] = v0;
                }
        }
    }

    // ---- record loads: 16-byte pieces into registers, one chunk ahead ------------
    // piece index pc = tid + NT m over [W | Qh | Mqk | KbT | U~ rows | e^{G_C}]
    constexpr int NT = L::NT;
    uint4 pre[NPT];
    auto load_rec = [&](int ci, uint4 (&pre)[NPT]) {
        const unsigned char* rec = rec0 + (size_t)ci * RL.bytes;
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec);
#pragma unroll
        for (int m = 0; m < NPT; ++m) {
            const int pc = tid + NT * m;
            unsigned off = 0;
            bool ok = true;
            if (pc < L::E1) {
                off = (unsigned)RL.oW + (unsigned)pc * 16u;
            } else if (pc < L::E2) {
                off = (unsigned)RL.oQh + (unsigned)(pc - L::E1) * 16u;
            } else if (pc < L::E3) {
                off = (unsigned)RL.oMqk + (unsigned)(pc - L::E2) * 16u;
            } else if (pc < L::E4) {
                off = (unsigned)RL.oKbT + (unsigned)(pc - L::E3) * 16u;
            } else if (pc < L::E5) {
                ok = pc - L::E4 < nvcol * (C * (int)SZ / 16);
                off = (unsigned)RL.oUtT + (unsigned)vcol0 * C * SZ + (unsigned)(pc - L::E4) * 16u;
            } else if (pc < L::PTOT) {
                off = (unsigned)RL.oEgc + (unsigned)(pc - L::E5) * 16u;
            } else {
                ok = false;
            }
            pre[m] = ok ? buf_load16(rr, off) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_rec = [&](const uint4 (&pre)[NPT]) {
#pragma unroll
        for (int m = 0; m < NPT; ++m) {
            const int pc = tid + NT * m;
            unsigned char* dst = nullptr;
            constexpr int PRK = K * (int)SZ / 16;        // pieces per K-long row
            constexpr int PRC = C * (int)SZ / 16;        // pieces per C-long row
            if (pc < L::E1) {
                dst = smem + L::oW + (pc / PRK) * LDK2 * SZ + (pc % PRK) * 16;
            } else if (pc < L::E2) {
                const int q = pc - L::E1;
                dst = smem + L::oQh + (q / PRK) * LDK2 * SZ + (q % PRK) * 16;
            } else if (pc < L::E3) {
                const int q = pc - L::E2;
                dst = smem + L::oMqk + (q / PRC) * LDL * SZ + (q % PRC) * 16;
            } else if (pc < L::E4) {
                const int q = pc - L::E3;
                dst = smem + L::oKbT + (q / PRC) * LDT * SZ + (q % PRC) * 16;
            } else if (pc < L::E5) {
                const int q = pc - L::E4;
                dst = smem + L::oUtT + (q / PRC) * LDT * SZ + (q % PRC) * 16;
            } else if (pc < L::PTOT) {
                dst = smem + L::oEGC + (pc - L::E5) * 16;
            }
            if (dst) *reinterpret_cast<uint4*>(dst) = pre[m];
        }
    };
    const unsigned rowV = (unsigned)p.H * V * SZ;
    // one chunk of the state pass, operands in LDS
    auto step = [&](int ci) {
        const size_t trow = row0 + (size_t)ci * C;                 // first token row of the chunk
        const int nt = (int)min((size_t)C, row_end - trow);
        // the output gate's pieces of this wave's o rows, loaded before the
        // products (the stores of o must not wait for them one by one)
        constexpr int OWG = 16 * NTW, PPRG = OWG * (int)SZ / 16;
        uint4 zr[GATE ? PPRG : 1];
        if constexpr (GATE) {
            const size_t obase = (trow * p.H + h) * V + vcol0 + OWG * w;
            const __amdgpu_buffer_rsrc_t rz = make_rsrc(reinterpret_cast<const T*>(p.gate) + obase);
#pragma unroll
            for (int m = 0; m < PPRG; ++m) {
                const int pc = l + 64 * m, row = pc / PPRG, sg = pc % PPRG;
                zr[m] = row < nt ? buf_load16(rz, (unsigned)row * rowV + (unsigned)sg * 16u) : make_uint4(0, 0, 0, 0);
            }
        }
        // every phase first reads all of its LDS operands, then runs its MFMAs
        Frag Sb[NTW][KS];
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) Sb[j][ks] = frag_from_tiles<T>(S[j][2 * ks], S[j][2 * ks + 1]);
        // U = U~ - W S
        f32x4 U[NTW][4];
        if constexpr (NARROW_REGS) {
            // two waves per SIMD hide the LDS latency: operands per row tile
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                Frag aw[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) aw[ks] = ld_frag_perm<T>(&sW[(16 * ti + lr) * LDK2 + 32 * ks + 4 * lg]);
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const f32x4 ut = pmode ? f32x4{0.f, 0.f, 0.f, 0.f}
                                           : ld4_as_f32<T>(&sUtT[(urow0 + 16 * j + lr) * LDT + 16 * ti + 4 * lg]);
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) acc = mma(acc, aw[ks], Sb[j][ks]);
                    U[j][ti] = ut - acc;
                }
            }
        } else {
            Frag aw[4][KS];
            f32x4 ut[NTW][4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) aw[ti][ks] = ld_frag_perm<T>(&sW[(16 * ti + lr) * LDK2 + 32 * ks + 4 * lg]);
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
                    ut[j][ti] = pmode ? f32x4{0.f, 0.f, 0.f, 0.f}
                                      : ld4_as_f32<T>(&sUtT[(urow0 + 16 * j + lr) * LDT + 16 * ti + 4 * lg]);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) acc = mma(acc, aw[ti][ks], Sb[j][ks]);
                    U[j][ti] = ut[j][ti] - acc;
                }
        }
        Frag Ub[NTW][2];
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            Ub[j][0] = frag_from_tiles<T>(U[j][0], U[j][1]);
            Ub[j][1] = frag_from_tiles<T>(U[j][2], U[j][3]);
        }
        if constexpr (OUT) {
            // O = (Q e^G) S + Mqk U, staged in this wave's own (consumed) U~ rows
            constexpr int OW = 16 * NTW;
            T* sO = sUtT + 16 * tile0 * LDT;
            Frag aq[4][KS], am[4][2];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) aq[ti][ks] = ld_frag_perm<T>(&sQh[(16 * ti + lr) * LDK2 + 32 * ks + 4 * lg]);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (ks <= (ti >> 1)) am[ti][ks] = ld_frag_perm<T>(&sMqk[(16 * ti + lr) * LDL + 32 * ks + 4 * lg]);
            }
            f32x4 acco[NTW][4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) acc = mma(acc, aq[ti][ks], Sb[j][ks]);
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        if (ks <= (ti >> 1)) acc = mma(acc, am[ti][ks], Ub[j][ks]);
                    acco[j][ti] = acc;
                }
            wave_lds_sync();
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int j = 0; j < NTW; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sO[(16 * ti + 4 * lg + e) * OW + 16 * j + lr] = from_f32<T>(acco[j][ti][e]);
            wave_lds_sync();
            constexpr int PPR = OW * (int)SZ / 16;
            static_assert(PPR == PPRG && C * PPR == 64 * PPR, "output pieces per lane");
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(
                reinterpret_cast<T*>(p.o) + (trow * p.H + h) * V + vcol0 + OW * w);
#pragma unroll
            for (int m = 0; m < PPR; ++m) {
                const int pc = l + 64 * m, row = pc / PPR, sg = pc % PPR;
                if (row < nt) {
                    const unsigned off = (unsigned)row * rowV + (unsigned)sg * 16u;
                    uint4 ov = *reinterpret_cast<const uint4*>(&sO[row * OW + sg * (16 / (int)SZ)]);
                    if constexpr (GATE) ov = gate_piece(ov, zr[m], (const T*)nullptr);
                    buf_store16(ro, off, 0u, ov);
                }
            }
        }
        // S <- Diag(e^{G_C}) S + (K e^{G_C - G})^T U
        if constexpr (NARROW_REGS) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const f32x4 eg = *reinterpret_cast<const f32x4*>(&sEGC[16 * ct + 4 * lg]);
                Frag ak[2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) ak[ks] = ld_frag_perm<T>(&sKbT[(16 * ct + lr) * LDT + 32 * ks + 4 * lg]);
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    S[j][ct] = S[j][ct] * eg;
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) S[j][ct] = mma(S[j][ct], ak[ks], Ub[j][ks]);
                }
            }
        } else {
            Frag ak[CT][2];
            f32x4 eg[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                eg[ct] = *reinterpret_cast<const f32x4*>(&sEGC[16 * ct + 4 * lg]);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) ak[ct][ks] = ld_frag_perm<T>(&sKbT[(16 * ct + lr) * LDT + 32 * ks + 4 * lg]);
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    S[j][ct] = S[j][ct] * eg[ct];
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) S[j][ct] = mma(S[j][ct], ak[ct][ks], Ub[j][ks]);
                }
        }
    };

    if (c_begin < c_end) load_rec(c_begin, pre);
    for (int ci = c_begin; ci < c_end; ++ci) {
        store_rec(pre);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        if (ci + 1 < c_end) load_rec(ci + 1, pre);
        __builtin_amdgcn_sched_barrier(0);
        step(ci);
        if constexpr (!SUMMARY) {
            // state snapshot after every snap_every whole chunks of a sequence
            if (p.snaps && (ci + 1) % p.snap_every == 0 && row0 + (size_t)(ci + 1) * C <= row_end) {
                const int slot = (p.snap_off ? p.snap_off[b] : b * p.snap_stride) + (ci + 1) / p.snap_every - 1;
                if (slot < p.max_snaps) {
                    const size_t so = ((size_t)slot * p.H + h) * K * V;
                    if (p.snap_bf16) {
                        bf16* sd = reinterpret_cast<bf16*>(p.snaps) + so;
#pragma unroll
                        for (int j = 0; j < NTW; ++j) {
                            const int col = col0 + 16 * (tile0 + j) + lr;
#pragma unroll
                            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    sd[(size_t)(16 * ct + 4 * lg + e) * V + col] = (bf16)S[j][ct][e];
                        }
                    } else {
                        float* sd = p.snaps + so;
#pragma unroll
                        for (int j = 0; j < NTW; ++j) {
                            const int col = col0 + 16 * (tile0 + j) + lr;
#pragma unroll
                            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                                for (int e = 0; e < 4; ++e) sd[(size_t)(16 * ct + 4 * lg + e) * V + col] = S[j][ct][e];
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    float* dst = nullptr;
    size_t ld = V;
    if (!SUMMARY) {
        if (seg == p.n_seg - 1 && p.sT) dst = p.sT + (size_t)bh * K * V;
    } else if (pmode) {
        dst = p.wsP + ((size_t)seg * BH + bh) * K * K;
        ld = K;
    } else {
        dst = p.wsL + ((size_t)seg * BH + bh) * K * V;
    }
    if (dst) {
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int my_col = col0 + 16 * (tile0 + j) + lr;
            const int col = SUMMARY ? (pmode ? my_col : my_col - K) : my_col;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(size_t)(16 * ct + 4 * lg + e) * ld + col] = S[j][ct][e];
        }
    }
}

// Chunk offsets of a packed batch (one workgroup; block-wide scans of 256
// sequence lengths at a time).
__global__ __launch_bounds__(256) void kda_varlen_prep_kernel(const int* cu, int N, int T_total, int max_chunks,
                                                              int* chunk_off, int snap_len, int max_snaps,
                                                              int* snap_off) {
    __shared__ int buf[256], sbuf[256];
    __shared__ int carry, scarry;
    const int tid = threadIdx.x;
    if (tid == 0) {
        carry = 0;
        scarry = 0;
        chunk_off[0] = 0;
        if (snap_off) snap_off[0] = 0;
    }
    __syncthreads();
    for (int base = 0; base < N; base += 256) {
        const int i = base + tid;
        int c = 0, sn = 0;
        if (i < N) {
            int s0, s1;
            seq_range(cu, i, T_total, s0, s1);
            c = (s1 - s0 + C - 1) / C;
            if (snap_off) sn = (s1 - s0) / snap_len;
        }
        buf[tid] = c;
        sbuf[tid] = sn;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {
            const int add = (tid >= d) ? buf[tid - d] : 0;
            const int sadd = (tid >= d) ? sbuf[tid - d] : 0;
            __syncthreads();
            buf[tid] += add;
            sbuf[tid] += sadd;
            __syncthreads();
        }
        if (i < N) {
            chunk_off[i + 1] = min(carry + buf[tid], max_chunks);
            if (snap_off) snap_off[i + 1] = min(scarry + sbuf[tid], max_snaps);
        }
        __syncthreads();
        if (tid == 255) {
            carry = min(carry + buf[255], max_chunks);
            scarry = min(scarry + sbuf[255], max_snaps);
        }
        __syncthreads();
    }
}

hipError_t launch_varlen_prep(const int* cu_seqlens, int N, int T_total, int max_chunks, int* chunk_off,
                              int snap_every, int max_snaps, int* snap_off, hipStream_t stream) {
    hipLaunchKernelGGL(kda_varlen_prep_kernel, dim3(1), dim3(256), 0, stream, cu_seqlens, N, T_total, max_chunks,
                       chunk_off, snap_every * C, max_snaps, snap_off);
    return hipGetLastError();
}

// ---- launchers ---------------------------------------------------------------------
bool split_variant_exists(int dtype, int K, int V, int VB) {
    const bool kv = (K == 64 || K == 128) && (V == 64 || V == 128);
    if (dtype == 1) return kv && (VB == 64 || VB == 128) && VB <= V;
    if (dtype == 0) return K == 64 && V == 64 && VB == 64;
    return false;
}

template <typename T, int K, int V>
static hipError_t launch_intra_t(const IntraParams& p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((kda_intra_kernel<T, K, V>), dim3(grid), dim3(512), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_intra(int dtype, int K, int V, const IntraParams& p, int grid, hipStream_t stream) {
    if (grid <= 0) return hipSuccess;
    if (dtype == 1) {
        if (K == 128 && V == 128) return launch_intra_t<bf16, 128, 128>(p, grid, stream);
        if (K == 128 && V == 64) return launch_intra_t<bf16, 128, 64>(p, grid, stream);
        if (K == 64 && V == 128) return launch_intra_t<bf16, 64, 128>(p, grid, stream);
        if (K == 64 && V == 64) return launch_intra_t<bf16, 64, 64>(p, grid, stream);
    } else if (dtype == 0) {
        if (K == 64 && V == 64) return launch_intra_t<float, 64, 64>(p, grid, stream);
    }
    return hipErrorInvalidValue;
}

template <typename T, int K, int NW, int NTW>
static hipError_t launch_state_t(const StateParams& p, int grid, hipStream_t stream) {
    if (p.summary)
        hipLaunchKernelGGL((kda_state_kernel<T, K, NW, NTW, true>), dim3(grid), dim3(64 * NW), 0, stream, p);
    else if (p.o && p.gate)
        hipLaunchKernelGGL((kda_state_kernel<T, K, NW, NTW, false, true, true>), dim3(grid), dim3(64 * NW), 0, stream, p);
    else if (p.o)
        hipLaunchKernelGGL((kda_state_kernel<T, K, NW, NTW, false, true>), dim3(grid), dim3(64 * NW), 0, stream, p);
    else
        hipLaunchKernelGGL((kda_state_kernel<T, K, NW, NTW, false, false>), dim3(grid), dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

// VB = 16 * NW * NTW value columns per workgroup; 128 columns run as 4 waves of
// two 16-column tiles (each LDS operand fragment serves two MFMAs)
hipError_t launch_state(int dtype, int K, int VB, const StateParams& p, int grid, hipStream_t stream) {
    if (grid <= 0) return hipSuccess;
    if (dtype == 1) {
        if (K == 128 && VB == 256 && p.summary) {
            hipLaunchKernelGGL((kda_state_kernel<bf16, 128, 8, 2, true>), dim3(grid), dim3(512), 0, stream, p);
            return hipGetLastError();
        }
        if (K == 128 && VB == 128) return launch_state_t<bf16, 128, 4, 2>(p, grid, stream);
        if (K == 128 && VB == 64) return launch_state_t<bf16, 128, 4, 1>(p, grid, stream);
        if (K == 64 && VB == 128) return launch_state_t<bf16, 64, 8, 1>(p, grid, stream);
        if (K == 64 && VB == 64) return launch_state_t<bf16, 64, 4, 1>(p, grid, stream);
    } else if (dtype == 0) {
        if (K == 64 && VB == 64) return launch_state_t<float, 64, 4, 1>(p, grid, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
