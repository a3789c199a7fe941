// Chunked KDA prefill for gfx950: gate cumsum, intra-chunk similarities,
// the delta-rule triangular (UT) solve and the inter-chunk state pass, fused
// in one kernel per (batch, head, segment, value-column block).
//
// Page: "Kimi K3 — открытая модель, которая обошла закрытых лидеров рынка"
// (aiblin.ru), section "Как распараллелили последовательное обновление": the
// tokens of a chunk are handled together, then the state is handed to the
// next chunk, in parallel over heads; for long prefill with few heads a
// planner splits the sequence into segments whose transitions are computed
// side by side on one card and recombined exactly.  Section "Как хранить
// миллион токенов в памяти": the forget gate is clamped to [e^-5, 1]
// because inside a chunk one divides by the running product of gates; here
// that division only ever happens inside 16-token sub-chunks, where it is at
// most e^{75} < FLT_MAX.
//
// Chunk form (C = 64 tokens, chunk-start state S, G = in-chunk inclusive
// cumsum of the clamped log gates, per key channel):
//   A[s][r]   = beta_s sum_c k_s[c] k_r[c] e^{G_s[c]-G_r[c]}     r < s
//   Mqk[t][s] = sum_c q_t[c] k_s[c] e^{G_t[c]-G_s[c]}            s <= t
//   Tm = (I + A)^{-1},  W = Tm diag(beta) (K e^{G}),  U~ = Tm diag(beta) V
//   U  = U~ - W S
//   O  = (Q e^{G}) S + Mqk U
//   S <- Diag(e^{G_C}) S + (K e^{G_C - G})^T U
// The exponent differences inside A and Mqk are split at the first token b
// of the row's 16-token block: e^{G_s-G_r} = e^{G_s-G_b} e^{G_b-G_r}, with
// the column factor for an earlier block j taken as e^{G_{b_j}-G_r} times
// the per-channel e^{G_b-G_{b_j}} (all factors <= 1 except the in-block
// e^{G_b-G_r} <= e^{75}).
//
// One workgroup = NW waves; wave w owns the 16 value columns
// [16w, 16w+16) of the block and keeps their K x 16 fp32 state and 64 x 16
// error U in MFMA accumulator registers for the whole sequence.  Everything
// shared between waves (the key-side operands) goes through LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = kChunk;

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <typename T, int K, int NTW>
struct ChunkLayout {
    static constexpr int NW = 4;                 // waves (one per SIMD)
    static constexpr int VB = 16 * NW * NTW;     // value columns per workgroup (NTW 16-col tiles per wave)
    static constexpr int NT = 64 * NW;           // threads
    static constexpr int SZ = (int)sizeof(T);
    static constexpr int PAD = 16 / SZ;          // 16 bytes of row padding
    static constexpr int LDK1 = K + PAD;         // Kd, Qd, Kinv: [token][channel], 16-byte reads
    static constexpr int LDK2 = K + PAD;         // W, Q e^G: [token][channel], 16-byte rows
    static constexpr int LDT = C + PAD;          // [channel][token] rows
    static constexpr int LDL = C + 4;            // solve blocks / Mqk: [token][token]
    static constexpr int LDD = 16;               // fp32 diagonal blocks of A
    // prep: wave w owns CPW groups of 8 key channels for all 64 tokens; lane
    // = (group, part of TPL consecutive tokens); likewise CPWV groups of 8
    // value columns with TPLV tokens per lane
    static constexpr int CPW = K / (8 * NW);
    static constexpr int TPL = CPW;
    static constexpr int NPART = 64 / CPW;
    static constexpr int CPWV = VB / (8 * NW);
    static constexpr int TPLV = CPWV;
    // region KQ: Kd | Qd | Kinv (prep -> A/Mqk), then W (solve -> state pass)
    static constexpr int NAT1 = C * LDK1 * SZ;
    static constexpr int KQ = cmax(3 * NAT1, C * LDK2 * SZ);
    static constexpr int L_BYTES = C * LDL * SZ;
    static constexpr int R = L_BYTES + 4 * 16 * LDD * 4;
    static constexpr int oKQ = 0;
    static constexpr int oR = oKQ + KQ;                  // solve blocks | fp32 diagonals of A
    static constexpr int oMqk = oR + R;                  // [C][LDL]
    static constexpr int oQh = oMqk + C * LDL * SZ;      // [C][LDK2] Q e^{G}
    static constexpr int oKhbT = oQh + C * LDK2 * SZ;    // [K][LDT] beta K e^{G}, channel-major
    static constexpr int oKbT = oKhbT + K * LDT * SZ;    // [K][LDT] K e^{G_C-G}, channel-major
    static constexpr int oVbT = oKbT + K * LDT * SZ;     // [VB][LDT] beta V, channel-major;
                                                          // in the state pass: per-wave output staging
    static constexpr int oF = oVbT + VB * LDT * SZ;      // fp32 [6][K] e^{G_b(i) - G_b(j)}
    static constexpr int oEGC = oF + 6 * K * 4;          // fp32 [K] e^{G_C}
    static constexpr int oBeta = oEGC + K * 4;           // fp32 [C]
    static constexpr int TOTAL = oBeta + C * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
    static_assert(NW * C * 16 * NTW <= VB * LDT, "output staging must fit the beta-V buffer");
    static_assert(CPW * 8 * NW == K && (CPW == 2 || CPW == 4), "key prep mapping");
    static_assert(CPWV * 8 * NW == VB && (CPWV == 2 || CPWV == 4), "value prep mapping");
};

// lower block pairs (i >= j) of the 4 x 4 sub-chunk grid
__device__ __forceinline__ void lower_pair(int p, int& i, int& j) {
    i = (p >= 6) ? 3 : (p >= 3) ? 2 : (p >= 1) ? 1 : 0;
    j = p - i * (i + 1) / 2;
}
// strictly lower pairs (i > j): index i(i-1)/2 + j
__device__ __forceinline__ void offdiag_pair(int p, int& i, int& j) {
    i = (p >= 3) ? 3 : (p >= 1) ? 2 : 1;
    j = p - i * (i - 1) / 2;
}

template <typename T>
__device__ __forceinline__ void ld8_as_f32(const T* p, float* x) {
    typename FragOf<T>::type f = ld_frag<T>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = to_f32(f[i]);
}

// B fragment of the column side of block pair (i, j) for the 32-deep slab at
// channel c0: rows of block j of K e^{G_b(j) - G}, times e^{G_b(i) - G_b(j)}
// per channel when i > j.
template <typename T, int K>
__device__ __forceinline__ typename FragOf<T>::type col_frag(const T* sKinv, const float* sF, int i, int j,
                                                            int lr, int c0) {
    constexpr int LDK1 = K + 16 / (int)sizeof(T);
    if (i == j) return ld_frag<T>(&sKinv[(16 * j + lr) * LDK1 + c0]);
    float kv[8], f[8];
    ld8_as_f32<T>(&sKinv[(16 * j + lr) * LDK1 + c0], kv);
    ld8f(&sF[(i * (i - 1) / 2 + j) * K + c0], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) kv[e] *= f[e];
    return frag_from<T>(kv);
}

}  // namespace

template <typename T, int K, int NTW, bool SUMMARY>
__global__ __launch_bounds__(256) void kda_chunk_kernel(ChunkParams p) {
    using L = ChunkLayout<T, K, NTW>;
    constexpr int NW = L::NW;
    using Frag = typename FragOf<T>::type;
    using Frag4 = typename Frag4Of<T>::type;
    constexpr int VB = L::VB;
    constexpr int LDK1 = L::LDK1, LDK2 = L::LDK2, LDT = L::LDT, LDL = L::LDL, LDD = L::LDD;
    constexpr int CPW = L::CPW, TPL = L::TPL, NPART = L::NPART;
    constexpr int CPWV = L::CPWV, TPLV = L::TPLV;
    constexpr int KS = K / 32;                 // 32-deep slabs over key channels
    constexpr int CT = K / 16;                 // 16-row tiles of the state
    constexpr unsigned SZ = sizeof(T);

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
    T* sKd = reinterpret_cast<T*>(smem + L::oKQ);
    T* sQd = sKd + C * LDK1;
    T* sKinv = sQd + C * LDK1;
    T* sW = reinterpret_cast<T*>(smem + L::oKQ);
    T* sL = reinterpret_cast<T*>(smem + L::oR);
    float* sAd = reinterpret_cast<float*>(smem + L::oR + L::L_BYTES);
    T* sMqk = reinterpret_cast<T*>(smem + L::oMqk);
    T* sQh = reinterpret_cast<T*>(smem + L::oQh);
    T* sKhbT = reinterpret_cast<T*>(smem + L::oKhbT);
    T* sKbT = reinterpret_cast<T*>(smem + L::oKbT);
    T* sVbT = reinterpret_cast<T*>(smem + L::oVbT);
    float* sF = reinterpret_cast<float*>(smem + L::oF);
    float* sEGC = reinterpret_cast<float*>(smem + L::oEGC);
    float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, lg = l >> 4, lr = l & 15;

    // ---- which (b, h, segment, column block) this workgroup owns ----------
    // Consecutive logical ids share their inputs (same b, h, segment); they
    // are placed on the same XCD (workgroups are dealt to the 8 XCDs round
    // robin) so the shared q/k/g reads hit that XCD's L2.
    const int G = gridDim.x;
    const int x = blockIdx.x;
    const int lid = ((G & 7) == 0) ? (x & 7) * (G >> 3) + (x >> 3) : x;
    const int vb = lid % p.n_vb;
    const int rest = lid / p.n_vb;
    const int nseg_here = SUMMARY ? p.n_seg - 1 : p.n_seg;
    const int seg = rest % nseg_here;
    const int bh = rest / nseg_here;
    const int b = bh / p.H, h = bh % p.H;
    const int BH = p.B * p.H;
    const int V = p.V;
    const int n_chunks = (p.T + C - 1) / C;
    const int c_begin = seg * p.cps;
    const int c_end = min(c_begin + p.cps, n_chunks);

    // summary pass columns: [0, K) carry the transition P (start I, values 0),
    // [K, K+V) the local state L (start 0, the real values)
    const int col0 = vb * VB;
    const bool pmode = SUMMARY && col0 < K;
    const int vcol0 = SUMMARY ? (pmode ? 0 : col0 - K) : col0;
    // this lane's state columns: tile j covers block columns 16 (NTW w + j) + [0, 16)
    const int tile0 = NTW * w;

    const T* __restrict__ qg = reinterpret_cast<const T*>(p.q);
    const T* __restrict__ kg = reinterpret_cast<const T*>(p.k);
    const T* __restrict__ vg = reinterpret_cast<const T*>(p.v);
    const T* __restrict__ gg = reinterpret_cast<const T*>(p.g);
    const T* __restrict__ bg = reinterpret_cast<const T*>(p.beta);

    // prep lane roles
    const int c8l = l % CPW, part = l / CPW;
    const int c0 = 8 * (CPW * w + c8l);        // first of this lane's 8 key channels
    const int n8l = l % CPWV, pv = l / CPWV;
    const int n0 = 8 * (CPWV * w + n8l);       // first of this lane's 8 value columns

    // ---- initial state: S[j][ct] = rows 16ct + 4lg + e of tile j, column lr --
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
            for (int ct = 0; ct < CT; ++ct) {
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
    }

    // ---- raw chunk registers, loaded one chunk ahead ---------------------
    // (kept raw: converting at load time would make every load wait).
    // Global addressing: a buffer resource at the chunk's first row (scalar
    // registers), a 32-bit lane byte offset and a scalar per-token offset.
    Pack8<T> kr[TPL], qr[TPL], gr[TPL], vr[TPLV];
    T br[TPL], bvr[TPLV];
    const unsigned rowK = (unsigned)p.H * K * SZ, rowV = (unsigned)p.H * V * SZ, rowB = (unsigned)p.H * SZ;
    const unsigned vK = (unsigned)part * TPL * rowK + (unsigned)c0 * SZ;
    const unsigned vB = (unsigned)part * TPL * rowB;
    const unsigned vV = (unsigned)pv * TPLV * rowV + (unsigned)n0 * SZ;
    const unsigned vBV = (unsigned)pv * TPLV * rowB;
    auto load_chunk = [&](int ci) {
        const int t0 = ci * C;
        const int nt = min(C, p.T - t0);
        const size_t head_row = (size_t)(b * (size_t)p.T + t0) * p.H + h;   // token t0 of (b, h)
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + head_row * K);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg + head_row * K);
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(gg + head_row * K);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(bg + head_row);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + head_row * V + vcol0);
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            if (part * TPL + i < nt) {
                buf_load8<T>(kr[i], rk, vK, i * rowK);
                buf_load8<T>(gr[i], rg, vK, i * rowK);
                if (!SUMMARY) buf_load8<T>(qr[i], rq, vK, i * rowK); else qr[i].zero();
                buf_load1(br[i], rb, vB, i * rowB);
            } else {
                kr[i].zero();
                gr[i].zero();
                qr[i].zero();
                br[i] = from_f32<T>(0.f);
            }
        }
#pragma unroll
        for (int i = 0; i < TPLV; ++i) {
            if (pv * TPLV + i < nt && !pmode) {
                buf_load8<T>(vr[i], rv, vV, i * rowV);
                buf_load1(bvr[i], rb, vBV, i * rowB);
            } else {
                vr[i].zero();
                bvr[i] = from_f32<T>(0.f);
            }
        }
    };
    if (c_begin < c_end) load_chunk(c_begin);

    for (int ci = c_begin; ci < c_end; ++ci) {
        const int t0 = ci * C;
        const int nt = min(C, p.T - t0);

        // ---- P1: gate cumsum and key/query-side operands (registers -> LDS) ---
        {
            // in-lane inclusive sums over this lane's tokens, then a scan over
            // the lanes holding the same channels (parts in token order)
            float G[TPL][8];
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                float g8[8];
                gr[i].to_f32(g8);
#pragma unroll
                for (int e = 0; e < 8; ++e) G[i][e] = (i ? G[i - 1][e] : 0.f) + clamp_gate_log2(g8[e]);
            }
            float incl[8], gfirst[8], gb[8], gcum[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) incl[e] = G[TPL - 1][e];
#pragma unroll
            for (int d = CPW; d < 64; d <<= 1) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float y = __shfl_up(incl[e], d);
                    if (l >= d) incl[e] += y;
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float excl = incl[e] - G[TPL - 1][e];
#pragma unroll
                for (int i = 0; i < TPL; ++i) G[i][e] += excl;
                gfirst[e] = G[0][e];
                gcum[e] = __shfl(incl[e], (NPART - 1) * CPW + c8l);    // G at the chunk's last token
            }
            // G at the first token of a 16-token block (same channels): this
            // lane's block, and the two blocks of pair `part` of the table of
            // e^{G_b(i) - G_b(j)} (all lanes shuffle; parts >= 6 discard)
            const int myblk = (part * TPL) >> 4;
            int pi_ = 1, pj_ = 0;
            if (part < 6) offdiag_pair(part, pi_, pj_);
            const int src_b = (16 * myblk / TPL) * CPW + c8l;
            const int src_i = (16 * pi_ / TPL) * CPW + c8l;
            const int src_j = (16 * pj_ / TPL) * CPW + c8l;
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                gb[e] = __shfl(gfirst[e], src_b);
                f[e] = fast_exp2(__shfl(gfirst[e], src_i) - __shfl(gfirst[e], src_j));
            }
            if (part < 6) st8(&sF[part * K + c0], f);
            if (part == 0) {
                float f[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = fast_exp2(gcum[e]);
                st8(&sEGC[c0], f);
            }
            if (w == 0 && c8l == 0) {
#pragma unroll
                for (int i = 0; i < TPL; ++i) sBeta[part * TPL + i] = to_f32(br[i]);
            }
            float egb[8], ecb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                egb[e] = fast_exp2(gb[e]);             // e^{G_b}       <= 1
                ecb[e] = fast_exp2(gcum[e] - gb[e]);   // e^{G_C - G_b} <= 1
            }
            float kh[8][TPL], kb[8][TPL];
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const int t = part * TPL + i;
                float kx[8], kd[8], ki[8];
                kr[i].to_f32(kx);
                const float bt = to_f32(br[i]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float d = G[i][e] - gb[e];       // G_t - G_b in [-108, 0] (log2)
                    const float e1 = fast_exp2(d);         // e^{G_t - G_b} <= 1
                    const float e2 = fast_exp2(-d);        // e^{G_b - G_t} <= e^75
                    kd[e] = kx[e] * e1;
                    ki[e] = kx[e] * e2;
                    kh[e][i] = bt * kd[e] * egb[e];        // beta k e^{G_t}
                    kb[e][i] = ki[e] * ecb[e];             // k e^{G_C - G_t}
                }
                st8(&sKd[t * LDK1 + c0], kd);
                st8(&sKinv[t * LDK1 + c0], ki);
            }
            // (fence: the query side below reuses the registers of the key side)
            __builtin_amdgcn_sched_barrier(0);
            if (!SUMMARY) {
#pragma unroll
                for (int i = 0; i < TPL; ++i) {
                    const int t = part * TPL + i;
                    float qx[8], qd[8], qh[8];
                    qr[i].to_f32(qx);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        qd[e] = qx[e] * fast_exp2(G[i][e] - gb[e]);   // q e^{G_t - G_b}
                        qh[e] = qd[e] * egb[e];                        // q e^{G_t}
                    }
                    st8(&sQd[t * LDK1 + c0], qd);
                    st8(&sQh[t * LDK2 + c0], qh);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                st_small<TPL>(&sKhbT[(c0 + e) * LDT + part * TPL], kh[e]);
                st_small<TPL>(&sKbT[(c0 + e) * LDT + part * TPL], kb[e]);
            }
            // beta V, channel-major
            float bv[8][TPLV];
#pragma unroll
            for (int i = 0; i < TPLV; ++i) {
                float vx[8];
                vr[i].to_f32(vx);
                const float bt = to_f32(bvr[i]);
#pragma unroll
                for (int e = 0; e < 8; ++e) bv[e][i] = bt * vx[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) st_small<TPLV>(&sVbT[(n0 + e) * LDT + pv * TPLV], bv[e]);
        }
        __syncthreads();

        // ---- P2: A, D_i = (I + A_ii)^{-1} and Mqk --------------------------------
        if (w == 0) {
            // diagonal blocks of A (fp32), then their inverses by forward
            // substitution, one lane per (block, column); the LDS round trip
            // stays inside this wave
            f32x4 acc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i] = mma(acc[i], ld_frag<T>(&sKd[(16 * i + lr) * LDK1 + 32 * ks + 8 * lg]),
                                 ld_frag<T>(&sKinv[(16 * i + lr) * LDK1 + 32 * ks + 8 * lg]));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s_ = 16 * i + 4 * lg + e, r = 16 * i + lr;
                    sAd[(16 * i + 4 * lg + e) * LDD + lr] = (r < s_) ? sBeta[s_] * acc[i][e] : 0.f;
                }
            wave_lds_sync();
            const int i = lg, j = lr;
            float xv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float row[16];
#pragma unroll
                for (int m4 = 0; m4 < 4; ++m4) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4*>(&sAd[(i * 16 + r) * LDD + 4 * m4]);
                    row[4 * m4] = a4[0];
                    row[4 * m4 + 1] = a4[1];
                    row[4 * m4 + 2] = a4[2];
                    row[4 * m4 + 3] = a4[3];
                }
                float a = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) a -= row[m] * xv[m];
                xv[r] = a;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sL[(16 * i + r) * LDL + 16 * i + j] = from_f32<T>(xv[r]);
        } else {
            // off-diagonal blocks of A (negated, into the solve buffer), then
            // the blocks of Mqk; its blocks (0,1) and (2,3) are zero (they are
            // read by the 32-deep slabs of the output product)
            constexpr int NTASK = SUMMARY ? 6 : 18;
            for (int task = w - 1; task < NTASK; task += NW - 1) {
                if (task < 16) {
                    int i, j;
                    if (task < 6) offdiag_pair(task, i, j);
                    else lower_pair(task - 6, i, j);
                    const T* rowsrc = (task < 6) ? sKd : sQd;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int cc = 32 * ks + 8 * lg;
                        acc = mma(acc, ld_frag<T>(&rowsrc[(16 * i + lr) * LDK1 + cc]),
                                  col_frag<T, K>(sKinv, sF, i, j, lr, cc));
                    }
                    const int r = 16 * j + lr;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s_ = 16 * i + 4 * lg + e;
                        if (task < 6) sL[s_ * LDL + r] = from_f32<T>(-sBeta[s_] * acc[e]);
                        else sMqk[s_ * LDL + r] = from_f32<T>((i > j || r <= s_) ? acc[e] : 0.f);
                    }
                } else {
                    const int i = (task == 16) ? 0 : 2, j = i + 1;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sMqk[(16 * i + 4 * lg + e) * LDL + 16 * j + lr] = from_f32<T>(0.f);
                }
            }
        }
        __syncthreads();

        // ---- P3: W = (I+A)^{-1} beta K e^G and U~ = (I+A)^{-1} beta V ---------
        // block forward substitution per 16-column tile, tiles in registers:
        //   X_i = D_i (R_i - sum_{k<i} A_ik X_k)
        Frag4 Ld[4], Lo[6];
#pragma unroll
        for (int i = 0; i < 4; ++i) Ld[i] = ld_frag4<T>(&sL[(16 * i + lr) * LDL + 16 * i + 4 * lg]);
#pragma unroll
        for (int q6 = 0; q6 < 6; ++q6) {
            const int i = (q6 >= 3) ? 3 : (q6 >= 1) ? 2 : 1;
            const int k = q6 - i * (i - 1) / 2;
            Lo[q6] = ld_frag4<T>(&sL[(16 * i + lr) * LDL + 16 * k + 4 * lg]);
        }
        auto solve_tile = [&](const T* rhs, f32x4* X) {
            // rhs: channel-major row of this tile's first column; R_i read as
            // an accumulator tile (rows 16i + 4lg + e, column lr)
            Frag4 Xb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 acc = ld4_as_f32<T>(rhs + lr * LDT + 16 * i + 4 * lg);
#pragma unroll
                for (int k = 0; k < i; ++k) acc = mma16(acc, Lo[i * (i - 1) / 2 + k], Xb[k]);
                X[i] = mma16(f32x4{0.f, 0.f, 0.f, 0.f}, Ld[i], frag4_from<T>(acc));
                Xb[i] = frag4_from<T>(X[i]);
            }
        };
        for (int ct = w; ct < CT; ct += NW) {
            f32x4 X[4];
            solve_tile(&sKhbT[16 * ct * LDT], X);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sW[(16 * i + 4 * lg + e) * LDK2 + 16 * ct + lr] = from_f32<T>(X[i][e]);
        }
        f32x4 Ut[NTW][4];
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            if (!pmode) {
                solve_tile(&sVbT[16 * (tile0 + j) * LDT], Ut[j]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) Ut[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        __syncthreads();

        // fetch the next chunk behind the state pass (the scheduling fences keep
        // the loads in place, so the raw registers live only across this phase)
        __builtin_amdgcn_sched_barrier(0);
        if (ci + 1 < c_end) load_chunk(ci + 1);
        __builtin_amdgcn_sched_barrier(0);

        // ---- P4: the state pass (per wave, registers); output straight out ---
        // each key-side fragment read from LDS serves the wave's NTW tiles
        Frag Sb[NTW][KS];
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) Sb[j][ks] = frag_from_tiles<T>(S[j][2 * ks], S[j][2 * ks + 1]);
        f32x4 U[NTW][4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            f32x4 acc[NTW];
#pragma unroll
            for (int j = 0; j < NTW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const Frag a = ld_frag_perm<T>(&sW[(16 * ti + lr) * LDK2 + 32 * ks + 4 * lg]);
#pragma unroll
                for (int j = 0; j < NTW; ++j) acc[j] = mma(acc[j], a, Sb[j][ks]);
            }
#pragma unroll
            for (int j = 0; j < NTW; ++j) U[j][ti] = Ut[j][ti] - acc[j];
        }
        Frag Ub[NTW][2];
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            Ub[j][0] = frag_from_tiles<T>(U[j][0], U[j][1]);
            Ub[j][1] = frag_from_tiles<T>(U[j][2], U[j][3]);
        }
        if (!SUMMARY) {
            // this wave's 64 x 16NTW output block is staged row-major in the
            // beta-V buffer (free after the solve), then written out in
            // 16-byte pieces
            constexpr int OW = 16 * NTW;                 // staged row length
            T* sO = sVbT + w * (C * OW);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                f32x4 acc[NTW];
#pragma unroll
                for (int j = 0; j < NTW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const Frag a = ld_frag_perm<T>(&sQh[(16 * ti + lr) * LDK2 + 32 * ks + 4 * lg]);
#pragma unroll
                    for (int j = 0; j < NTW; ++j) acc[j] = mma(acc[j], a, Sb[j][ks]);
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (ks <= (ti >> 1)) {
                        const Frag a = ld_frag_perm<T>(&sMqk[(16 * ti + lr) * LDL + 32 * ks + 4 * lg]);
#pragma unroll
                        for (int j = 0; j < NTW; ++j) acc[j] = mma(acc[j], a, Ub[j][ks]);
                    }
                }
#pragma unroll
                for (int j = 0; j < NTW; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sO[(16 * ti + 4 * lg + e) * OW + 16 * j + lr] = from_f32<T>(acc[j][e]);
            }
            wave_lds_sync();
            constexpr int PPR = OW * (int)SZ / 16;       // 16-byte pieces per row
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(
                reinterpret_cast<T*>(p.o) + ((size_t)(b * (size_t)p.T + t0) * p.H + h) * V + vcol0 + OW * w);
            const size_t obase = ((size_t)(b * (size_t)p.T + t0) * p.H + h) * V + vcol0 + OW * w;
            const __amdgpu_buffer_rsrc_t rz = make_rsrc(p.gate ? reinterpret_cast<const T*>(p.gate) + obase : nullptr);
#pragma unroll
            for (int pc = l; pc < C * PPR; pc += 64) {
                const int row = pc / PPR, seg = pc % PPR;
                if (row < nt) {
                    const unsigned off = (unsigned)row * rowV + (unsigned)seg * 16u;
                    uint4 ov = *reinterpret_cast<const uint4*>(&sO[row * OW + seg * (16 / (int)SZ)]);
                    if (p.gate) ov = gate_piece(ov, buf_load16(rz, off), (const T*)nullptr);
                    buf_store16(ro, off, 0u, ov);
                }
            }
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const f32x4 eg = *reinterpret_cast<const f32x4*>(&sEGC[16 * ct + 4 * lg]);
#pragma unroll
            for (int j = 0; j < NTW; ++j) S[j][ct] = S[j][ct] * eg;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const Frag a = ld_frag_perm<T>(&sKbT[(16 * ct + lr) * LDT + 32 * ks + 4 * lg]);
#pragma unroll
                for (int j = 0; j < NTW; ++j) S[j][ct] = mma(S[j][ct], a, Ub[j][ks]);
            }
        }
        __syncthreads();
    }

    // ---- final state of this segment / column block ----------------------------
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

// Segment scan: S_{j+1} = P_j S_j + L_j, written over L_j, per (b, h) and
// 16-column block, on fp32 MFMA (16x16x4).  Wave w owns row tiles
// [TPW w, TPW w + TPW); MFMA step ks reduces over the state rows
// {(K/4) g + ks : g = 0..3} (lane group g supplies one of them), so every lane
// reads K/4 consecutive elements of its P row.  The next segment's P rows and
// L tiles are loaded while the current one is applied.
template <int K, bool REV, int NWS>
__global__ __launch_bounds__(64 * NWS) void kda_scan_kernel(ScanParams p) {
    constexpr int RT = K / 16;          // row tiles
    constexpr int TPW = RT / NWS;       // row tiles per wave
    static_assert(TPW * NWS == RT, "whole row tiles per wave");
    constexpr int KQ = K / 4;           // reduction steps
    // the state block's 16 columns, column-major (a lane reads its column's
    // 32 reduction rows with 16-byte reads and writes its 4 rows with one)
    constexpr int LDT = K + 4;
    __shared__ __attribute__((aligned(16))) float sS[16 * LDT];
    // the column blocks of one (b, h) read the same P rows: place them on one
    // XCD (workgroups are dealt to the 8 XCDs round robin) so they share its L2
    const int G = gridDim.x, x = blockIdx.x;
    const int lid = ((G & 7) == 0) ? (x & 7) * (G >> 3) + (x >> 3) : x;
    const int ncb = p.V / 16;
    const int bh = lid / ncb, cb = lid % ncb;
    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, lg = l >> 4, lr = l & 15;
    const int V = p.V;
    const size_t col = (size_t)cb * 16 + lr;
    for (int i = tid; i < K * 16; i += 64 * NWS) {
        const int row = i / 16, c = i % 16;
        sS[c * LDT + row] = p.s0 ? p.s0[((size_t)bh * K + row) * V + (size_t)cb * 16 + c] : 0.f;
    }
    // two register sets: segment j + 1's P rows and L tile are in flight
    // during step j (loads are issued as soon as a set's MFMAs have read it).
    // Past the last transition the resources are empty (the loads return zeros
    // and touch no memory): every load is issued unconditionally, so that each
    // wait counts only the older set's loads instead of draining all of them.
    float aA[TPW][KQ], aB[TPW][KQ];
    f32x4 lA[TPW], lB[TPW];
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    auto load_seg = [&](int j, float (&a)[TPW][KQ], f32x4 (&lt)[TPW]) {
        const bool live = j < p.n_seg - 1;
        const int jj = live ? j : 0;
        const int pj = REV ? p.n_seg - 1 - jj : jj;
        const __amdgpu_buffer_rsrc_t rp =
            make_rsrc_n(p.wsP + ((size_t)pj * p.BH + bh) * K * K, live ? (unsigned)(K * K * 4) : 0u);
        const __amdgpu_buffer_rsrc_t rl =
            make_rsrc_n(p.wsL + ((size_t)jj * p.BH + bh) * K * V, live ? (unsigned)(K * V * 4) : 0u);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int rt = TPW * w + t;
            if constexpr (REV) {
                // row 16 rt + lr of P^T: column 16 rt + lr of P (16 lanes read
                // 64 consecutive bytes of each row)
#pragma unroll
                for (int q = 0; q < KQ; ++q)
                    a[t][q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        rp, (int)((unsigned)((KQ * lg + q) * K + 16 * rt + lr) * 4u), 0, 0));
            } else {
                const unsigned row = (unsigned)((16 * rt + lr) * K + KQ * lg) * 4u;
#pragma unroll
                for (int q4 = 0; q4 < KQ / 4; ++q4) {
                    const u32x4 v4 = __builtin_amdgcn_raw_buffer_load_b128(rp, (int)(row + 16u * q4), 0, 0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[t][4 * q4 + e] = __uint_as_float(v4[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                lt[t][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    rl, (int)((unsigned)((16 * rt + 4 * lg + e) * V) * 4u + (unsigned)col * 4u), 0, 0));
        }
    };
    // S_{j+1} = P_j S_j + L_j with set (a, lt); then the set takes segment j + 2
    auto step = [&](int j, float (&a)[TPW][KQ], f32x4 (&lt)[TPW]) {
        // the B operands (S_j rows) are read from LDS together, ahead of the
        // MFMA chains, so the chains do not wait on each read
        float bS[KQ];
#pragma unroll
        for (int k4 = 0; k4 < KQ / 4; ++k4) {
            const f32x4 v4 = *reinterpret_cast<const f32x4*>(&sS[lr * LDT + KQ * lg + 4 * k4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) bS[4 * k4 + e] = v4[e];
        }
        __builtin_amdgcn_sched_barrier(0);
        // two independent chains per tile (even and odd reduction steps)
        f32x4 acc[TPW], acc2[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            acc[t] = lt[t];
            acc2[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < KQ; ks += 2)
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t][ks], bS[ks], acc[t], 0, 0, 0);
                acc2[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t][ks + 1], bS[ks + 1], acc2[t], 0, 0, 0);
            }
#pragma unroll
        for (int t = 0; t < TPW; ++t) acc[t] += acc2[t];
        // S_{j+1} to slot j, before the loads of segment j + 2: a wait for the
        // other set's loads then counts these stores as issued earlier and
        // need not wait for them to complete
        float* Lj = p.wsL + ((size_t)j * p.BH + bh) * K * V;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int rt = TPW * w + t;
#pragma unroll
            for (int e = 0; e < 4; ++e) Lj[(size_t)(16 * rt + 4 * lg + e) * V + col] = acc[t][e];
        }
        load_seg(j + 2, a, lt);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int rt = TPW * w + t;
            *reinterpret_cast<f32x4*>(&sS[lr * LDT + 16 * rt + 4 * lg]) = acc[t];
        }
        __syncthreads();
    };
    load_seg(0, aA, lA);
    load_seg(1, aB, lB);
    __syncthreads();
    // steps 0 .. n_seg - 2 (n_seg >= 2): step 0, then pairs (no step skipped
    // inside the loop), then the odd one left.  With step 0 ahead of the loop
    // the memory operations in flight at the loop top are the same on entry
    // and on the back edge, so its wait leaves the previous step's stores in
    // flight.
    step(0, aA, lA);
    int j = 1;
    for (; j + 2 < p.n_seg; j += 2) {
        step(j, aB, lB);
        step(j + 1, aA, lA);
    }
    if (j + 1 < p.n_seg) step(j, aB, lB);
}

__global__ __launch_bounds__(256) void kda_copy_state_kernel(const float* src, float* dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src ? src[i] : 0.f;
}

// ---- launchers ---------------------------------------------------------------------
// dtype: 0 = fp32, 1 = bf16 (kda_dtype)
bool chunk_variant_exists(int dtype, int K, int VB) {
    if (dtype == 1) return (K == 64 || K == 128) && (VB == 64 || VB == 128);
    if (dtype == 0) return K == 64 && VB == 64;
    return false;
}

template <typename T, int K, int NTW>
static hipError_t launch_chunk_t(const ChunkParams& p, int grid, hipStream_t stream) {
    if (p.summary)
        hipLaunchKernelGGL((kda_chunk_kernel<T, K, NTW, true>), dim3(grid), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((kda_chunk_kernel<T, K, NTW, false>), dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_chunk(int dtype, int K, int VB, const ChunkParams& p, int grid, hipStream_t stream) {
    if (grid <= 0) return hipSuccess;
    if (dtype == 1) {
        if (K == 128 && VB == 128) return launch_chunk_t<bf16, 128, 2>(p, grid, stream);
        if (K == 128 && VB == 64) return launch_chunk_t<bf16, 128, 1>(p, grid, stream);
        if (K == 64 && VB == 128) return launch_chunk_t<bf16, 64, 2>(p, grid, stream);
        if (K == 64 && VB == 64) return launch_chunk_t<bf16, 64, 1>(p, grid, stream);
    } else if (dtype == 0) {
        if (K == 64 && VB == 64) return launch_chunk_t<float, 64, 1>(p, grid, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_scan(int K, const ScanParams& p, hipStream_t stream) {
    const int grid = p.BH * (p.V / 16);
    if (grid <= 0 || p.n_seg < 2) return hipSuccess;
    // K = 128: eight waves of one row tile each (two waves per SIMD fill the
    // bubbles of the dependent MFMA chains); K = 64: four waves
    if (K == 128 && p.p_reverse) hipLaunchKernelGGL((kda_scan_kernel<128, true, 8>), dim3(grid), dim3(512), 0, stream, p);
    else if (K == 128) hipLaunchKernelGGL((kda_scan_kernel<128, false, 8>), dim3(grid), dim3(512), 0, stream, p);
    else if (K == 64 && p.p_reverse) hipLaunchKernelGGL((kda_scan_kernel<64, true, 4>), dim3(grid), dim3(256), 0, stream, p);
    else if (K == 64) hipLaunchKernelGGL((kda_scan_kernel<64, false, 4>), dim3(grid), dim3(256), 0, stream, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_copy_state(const float* src, float* dst, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(kda_copy_state_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, n);
    return hipGetLastError();
}

}  // namespace kda
