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

template <typename T, int K, int NW>
struct ChunkLayout {
    static constexpr int VB = 16 * NW;           // value columns per workgroup
    static constexpr int NT = 64 * NW;           // threads
    static constexpr int SZ = (int)sizeof(T);
    static constexpr int PAD = 16 / SZ;          // 16 bytes of padding per row
    static constexpr int LDK = K + PAD;          // [token][channel] rows
    static constexpr int LDT = C + PAD;          // [channel][token] rows
    static constexpr int LDA = C + 4;            // fp32 A / Tm rows
    static constexpr int LDO = VB + PAD;         // output staging rows
    static constexpr int NAT = C * LDK * SZ;     // one [C][LDK] buffer
    // region KQ: phase A = Kd | Qd | Kinv ; phase B = W | X (solve scratch) | O
    static constexpr int X_BYTES = 3 * 16 * 16 * 4;
    static constexpr int KQ_A = 3 * NAT;
    static constexpr int KQ_B = NAT + X_BYTES + C * LDO * SZ;
    static constexpr int KQ = KQ_A > KQ_B ? KQ_A : KQ_B;
    // region G: phase A = G (fp32 cumsum) ; phase B = A/Tm (fp32) | Mqk
    static constexpr int G_A = C * K * 4;
    static constexpr int G_B = C * LDA * 4 + C * LDT * SZ;
    static constexpr int GR = G_A > G_B ? G_A : G_B;
    static constexpr int oKQ = 0;
    static constexpr int oG = oKQ + KQ;
    static constexpr int oKhbT = oG + GR;               // [K][LDT] beta K e^{G}, transposed
    static constexpr int oQh = oKhbT + K * LDT * SZ;    // [C][LDK] Q e^{G}
    static constexpr int oKbT = oQh + NAT;              // [K][LDT] K e^{G_C-G}, transposed
    static constexpr int oVbT = oKbT + K * LDT * SZ;    // [VB][LDT] beta V, transposed
    static constexpr int oF = oVbT + VB * LDT * SZ;     // fp32 [6][K] block-pair gate factors
    static constexpr int oEGC = oF + 6 * K * 4;         // fp32 [K] e^{G_C}
    static constexpr int oBeta = oEGC + K * 4;          // fp32 [C]
    static constexpr int oPart = oBeta + C * 4;         // fp32 [NT] cumsum partial sums
    static constexpr int TOTAL = oPart + NT * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
    static_assert(NW >= 3, "the triangular solve needs three waves");
    static_assert(NT % K == 0 && C % (NT / K) == 0, "cumsum mapping");
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

}  // namespace

template <typename T, int K, int NW>
__global__ __launch_bounds__(64 * NW) void kda_chunk_kernel(ChunkParams p) {
    using L = ChunkLayout<T, K, NW>;
    using Frag = typename FragOf<T>::type;
    constexpr int VB = L::VB, NT = L::NT;
    constexpr int LDK = L::LDK, LDT = L::LDT, LDA = L::LDA, LDO = L::LDO;
    constexpr int NK8 = K / 8;                // 8-element packs per key row
    constexpr int NV8 = VB / 8;               // 8-element packs per value row
    constexpr int REPK = C * NK8 / NT;
    constexpr int REPV = C * NV8 / NT;
    constexpr int KS = K / 32;                // reduction slabs over key channels
    constexpr int CT = K / 16;                // 16-row tiles of the state
    static_assert(REPK * NT == C * NK8 && REPV * NT == C * NV8, "load mapping");

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
    T* sKd = reinterpret_cast<T*>(smem + L::oKQ);
    T* sQd = sKd + C * LDK;
    T* sKinv = sQd + C * LDK;
    T* sW = reinterpret_cast<T*>(smem + L::oKQ);
    float* sX = reinterpret_cast<float*>(smem + L::oKQ + L::NAT);
    T* sO = reinterpret_cast<T*>(smem + L::oKQ + L::NAT + L::X_BYTES);
    float* sG = reinterpret_cast<float*>(smem + L::oG);
    float* sA = reinterpret_cast<float*>(smem + L::oG);
    T* sMqk = reinterpret_cast<T*>(smem + L::oG + C * LDA * 4);
    T* sKhbT = reinterpret_cast<T*>(smem + L::oKhbT);
    T* sQh = reinterpret_cast<T*>(smem + L::oQh);
    T* sKbT = reinterpret_cast<T*>(smem + L::oKbT);
    T* sVbT = reinterpret_cast<T*>(smem + L::oVbT);
    float* sF = reinterpret_cast<float*>(smem + L::oF);
    float* sEGC = reinterpret_cast<float*>(smem + L::oEGC);
    float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);
    float* sPart = reinterpret_cast<float*>(smem + L::oPart);

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
    const int nseg_here = p.summary ? p.n_seg - 1 : p.n_seg;
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
    const int col0 = vb * VB;                           // first column of the block
    const bool pmode = p.summary && col0 < K;
    const int vcol0 = p.summary ? (pmode ? 0 : col0 - K) : col0;   // first value column
    const int my_col = col0 + 16 * w + lr;              // this lane's column (block space)

    const T* __restrict__ qg = reinterpret_cast<const T*>(p.q);
    const T* __restrict__ kg = reinterpret_cast<const T*>(p.k);
    const T* __restrict__ vg = reinterpret_cast<const T*>(p.v);
    const T* __restrict__ gg = reinterpret_cast<const T*>(p.g);
    const T* __restrict__ bg = reinterpret_cast<const T*>(p.beta);

    // ---- initial state: S[ct] = rows 16ct + 4lg + e, column my_col --------
    f32x4 S[CT];
    {
        const float* src = nullptr;
        if (!p.summary) {
            if (seg == 0) src = p.s0 ? p.s0 + (size_t)bh * K * V : nullptr;
            else src = p.seg_init + ((size_t)(seg - 1) * BH + bh) * K * V;
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * ct + 4 * lg + e;
                float s = 0.f;
                if (src) s = src[(size_t)row * V + my_col];
                else if (pmode) s = (row == my_col) ? 1.f : 0.f;
                S[ct][e] = s;
            }
        }
    }

    for (int ci = c_begin; ci < c_end; ++ci) {
        const int t0 = ci * C;
        const int nt = min(C, p.T - t0);

        // ---- P0: stream the chunk in ----------------------------------------
        Pack8<T> kr[REPK], qr[REPK], vr[REPV];
#pragma unroll
        for (int r = 0; r < REPK; ++r) {
            const int it = tid + r * NT;
            const int t = it / NK8, c8 = it % NK8;
            float gx[8];
            if (t < nt) {
                const size_t off = ((size_t)(b * (size_t)p.T + t0 + t) * p.H + h) * K + 8 * c8;
                kr[r].load(kg + off);
                if (!p.summary) qr[r].load(qg + off); else qr[r].zero();
                Pack8<T> gp;
                gp.load(gg + off);
                gp.to_f32(gx);
#pragma unroll
                for (int e = 0; e < 8; ++e) gx[e] = clamp_gate_log2(gx[e]);
            } else {
                kr[r].zero();
                qr[r].zero();
#pragma unroll
                for (int e = 0; e < 8; ++e) gx[e] = 0.f;
            }
            st8(&sG[t * K + 8 * c8], gx);
        }
#pragma unroll
        for (int r = 0; r < REPV; ++r) {
            const int it = tid + r * NT;
            const int t = it / NV8, n8 = it % NV8;
            if (t < nt && !pmode) {
                const size_t off = ((size_t)(b * (size_t)p.T + t0 + t) * p.H + h) * V + vcol0 + 8 * n8;
                vr[r].load(vg + off);
            } else {
                vr[r].zero();
            }
        }
        if (tid < C)
            sBeta[tid] = (tid < nt) ? ld_scalar(bg + (size_t)(b * (size_t)p.T + t0 + tid) * p.H + h) : 0.f;
        __syncthreads();

        // ---- P1: beta V (transposed) and the in-chunk gate cumsum ------------
#pragma unroll
        for (int r = 0; r < REPV; ++r) {
            const int it = tid + r * NT;
            const int t = it / NV8, n8 = it % NV8;
            float x8[8];
            vr[r].to_f32(x8);
            const float bt = sBeta[t];
#pragma unroll
            for (int e = 0; e < 8; ++e) sVbT[(8 * n8 + e) * LDT + t] = from_f32<T>(bt * x8[e]);
        }
        {
            constexpr int P = NT / K, R = C / P;
            const int c = tid % K, part = tid / K;
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < R; ++i) s += sG[(part * R + i) * K + c];
            sPart[part * K + c] = s;
            __syncthreads();
            float run = 0.f;
            for (int pp = 0; pp < part; ++pp) run += sPart[pp * K + c];
#pragma unroll
            for (int i = 0; i < R; ++i) {
                run += sG[(part * R + i) * K + c];
                sG[(part * R + i) * K + c] = run;
            }
        }
        __syncthreads();

        // ---- P2: key/query-side operands -------------------------------------
        for (int idx = tid; idx < K; idx += NT) sEGC[idx] = fast_exp2(sG[(C - 1) * K + idx]);
        for (int idx = tid; idx < 6 * K; idx += NT) {
            int i, j;
            offdiag_pair(idx / K, i, j);
            const int c = idx % K;
            sF[idx] = fast_exp2(sG[16 * i * K + c] - sG[16 * j * K + c]);
        }
#pragma unroll
        for (int r = 0; r < REPK; ++r) {
            const int it = tid + r * NT;
            const int t = it / NK8, c8 = it % NK8;
            float g8[8], gb8[8], gc8[8], kx[8], qx[8];
            ld8f(&sG[t * K + 8 * c8], g8);
            ld8f(&sG[(t & ~15) * K + 8 * c8], gb8);
            ld8f(&sG[(C - 1) * K + 8 * c8], gc8);
            kr[r].to_f32(kx);
            qr[r].to_f32(qx);
            const float bt = sBeta[t];
            float kd[8], ki[8], kh[8], kb[8], qd[8], qh[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float e0 = fast_exp2(g8[e]);              // e^{G_t}         <= 1
                const float e1 = fast_exp2(g8[e] - gb8[e]);     // e^{G_t - G_b}   <= 1
                const float e2 = fast_exp2(gb8[e] - g8[e]);     // e^{G_b - G_t}   <= e^75
                const float e3 = fast_exp2(gc8[e] - g8[e]);     // e^{G_C - G_t}   <= 1
                kd[e] = kx[e] * e1;
                ki[e] = kx[e] * e2;
                kh[e] = bt * kx[e] * e0;
                kb[e] = kx[e] * e3;
                qd[e] = qx[e] * e1;
                qh[e] = qx[e] * e0;
            }
            st8(&sKd[t * LDK + 8 * c8], kd);
            st8(&sKinv[t * LDK + 8 * c8], ki);
            if (!p.summary) {
                st8(&sQd[t * LDK + 8 * c8], qd);
                st8(&sQh[t * LDK + 8 * c8], qh);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sKhbT[(8 * c8 + e) * LDT + t] = from_f32<T>(kh[e]);
                sKbT[(8 * c8 + e) * LDT + t] = from_f32<T>(kb[e]);
            }
        }
        __syncthreads();

        // ---- P3: A and Mqk, one 16 x 16 block pair per wave at a time ---------
        // (writes region G, whose gate cumsum is no longer needed)
        for (int pi = w; pi < 10; pi += NW) {
            int i, j;
            lower_pair(pi, i, j);
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c0 = 32 * ks + 8 * lg;
                const Frag ak = ld_frag<T>(&sKd[(16 * i + lr) * LDK + c0]);
                float kv[8];
                ld8_as_f32<T>(&sKinv[(16 * j + lr) * LDK + c0], kv);
                if (i != j) {
                    float f[8];
                    ld8f(&sF[(i * (i - 1) / 2 + j) * K + c0], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) kv[e] *= f[e];
                }
                const Frag bk = frag_from<T>(kv);
                accA = mma(accA, ak, bk);
                if (!p.summary) accM = mma(accM, ld_frag<T>(&sQd[(16 * i + lr) * LDK + c0]), bk);
            }
            const int r = 16 * j + lr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 16 * i + 4 * lg + e;
                sA[s * LDA + r] = (i > j || r < s) ? sBeta[s] * accA[e] : 0.f;
                if (!p.summary) sMqk[s * LDT + r] = from_f32<T>((i > j || r <= s) ? accM[e] : 0.f);
            }
        }
        for (int idx = tid; idx < C * C; idx += NT) {
            const int s = idx / C, r = idx % C;
            if ((r >> 4) > (s >> 4)) {
                sA[s * LDA + r] = 0.f;
                if (!p.summary) sMqk[s * LDT + r] = from_f32<T>(0.f);
            }
        }
        __syncthreads();

        // ---- P4: Tm = (I + A)^{-1} in place, fp32 ------------------------------
        // diagonal 16 x 16 blocks by forward substitution, one lane per column
        if (w == 0) {
            const int i = lg, j = lr;
            float xv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) acc -= sA[(16 * i + r) * LDA + 16 * i + m] * xv[m];
                xv[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sA[(16 * i + r) * LDA + 16 * i + j] = xv[r];
        }
        __syncthreads();
        // row blocks below: Tm_ij = -D_i sum_{k=j}^{i-1} A_ik Tm_kj (fp32 MFMA)
#pragma unroll
        for (int i = 1; i < 4; ++i) {
            if (w < i) {
                const int j = w;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int kk = 16 * j; kk < 16 * i; kk += 4)
                    acc = mma4(acc, sA[(16 * i + lr) * LDA + kk + lg], sA[(kk + lg) * LDA + 16 * j + lr]);
#pragma unroll
                for (int e = 0; e < 4; ++e) sX[j * 256 + (4 * lg + e) * 16 + lr] = acc[e];
            }
            __syncthreads();
            if (w < i) {
                const int j = w;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int mm = 0; mm < 16; mm += 4)
                    acc = mma4(acc, sA[(16 * i + lr) * LDA + 16 * i + mm + lg], sX[j * 256 + (mm + lg) * 16 + lr]);
#pragma unroll
                for (int e = 0; e < 4; ++e) sA[(16 * i + 4 * lg + e) * LDA + 16 * j + lr] = -acc[e];
            }
            __syncthreads();
        }

        // ---- P5: W = Tm (beta K e^G) (shared), U~ = Tm (beta V) (per wave) ---
        Frag Tf[4][2];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks <= (ti >> 1)) {
                    float xv[8];
                    ld8f(&sA[(16 * ti + lr) * LDA + 32 * ks + 8 * lg], xv);
                    Tf[ti][ks] = frag_from<T>(xv);
                }
            }
        }
        for (int ct = w; ct < CT; ct += NW) {
            Frag bk[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) bk[ks] = ld_frag<T>(&sKhbT[(16 * ct + lr) * LDT + 32 * ks + 8 * lg]);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (ks <= (ti >> 1)) acc = mma(acc, Tf[ti][ks], bk[ks]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sW[(16 * ti + 4 * lg + e) * LDK + 16 * ct + lr] = from_f32<T>(acc[e]);
            }
        }
        f32x4 Ut[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) Ut[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!pmode) {
            Frag bv[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) bv[ks] = ld_frag<T>(&sVbT[(16 * w + lr) * LDT + 32 * ks + 8 * lg]);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (ks <= (ti >> 1)) Ut[ti] = mma(Ut[ti], Tf[ti][ks], bv[ks]);
        }
        __syncthreads();

        // ---- P6: the state pass (per wave, registers) --------------------------
        Frag Sb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) Sb[ks] = frag_from_tiles<T>(S[2 * ks], S[2 * ks + 1]);
        f32x4 U[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc = mma(acc, ld_frag_perm<T>(&sW[(16 * ti + lr) * LDK + 32 * ks + 4 * lg]), Sb[ks]);
            U[ti] = Ut[ti] - acc;
        }
        Frag Ub[2];
        Ub[0] = frag_from_tiles<T>(U[0], U[1]);
        Ub[1] = frag_from_tiles<T>(U[2], U[3]);
        if (!p.summary) {
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = mma(acc, ld_frag_perm<T>(&sQh[(16 * ti + lr) * LDK + 32 * ks + 4 * lg]), Sb[ks]);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (ks <= (ti >> 1))
                        acc = mma(acc, ld_frag_perm<T>(&sMqk[(16 * ti + lr) * LDT + 32 * ks + 4 * lg]), Ub[ks]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sO[(16 * ti + 4 * lg + e) * LDO + 16 * w + lr] = from_f32<T>(acc[e]);
            }
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const f32x4 eg = *reinterpret_cast<const f32x4*>(&sEGC[16 * ct + 4 * lg]);
            S[ct] = S[ct] * eg;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                S[ct] = mma(S[ct], ld_frag_perm<T>(&sKbT[(16 * ct + lr) * LDT + 32 * ks + 4 * lg]), Ub[ks]);
        }
        __syncthreads();

        // ---- P7: stream the chunk's output out ---------------------------------
        if (!p.summary) {
            T* og = reinterpret_cast<T*>(p.o);
#pragma unroll
            for (int r = 0; r < REPV; ++r) {
                const int it = tid + r * NT;
                const int t = it / NV8, n8 = it % NV8;
                if (t < nt) {
                    const size_t off = ((size_t)(b * (size_t)p.T + t0 + t) * p.H + h) * V + vcol0 + 8 * n8;
                    *reinterpret_cast<uint4*>(og + off) = *reinterpret_cast<const uint4*>(&sO[t * LDO + 8 * n8]);
                    if (sizeof(T) == 4)
                        *reinterpret_cast<uint4*>(og + off + 4) = *reinterpret_cast<const uint4*>(&sO[t * LDO + 8 * n8 + 4]);
                }
            }
        }
    }

    // ---- final state of this segment / column block ----------------------------
    float* dst = nullptr;
    size_t ld = V;
    if (!p.summary) {
        if (seg == p.n_seg - 1 && p.sT) dst = p.sT + (size_t)bh * K * V;
    } else if (pmode) {
        dst = p.wsP + ((size_t)seg * BH + bh) * K * K;
        ld = K;
    } else {
        dst = p.wsL + ((size_t)seg * BH + bh) * K * V;
    }
    if (dst) {
        const int col = p.summary ? (pmode ? my_col : my_col - K) : my_col;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(size_t)(16 * ct + 4 * lg + e) * ld + col] = S[ct][e];
    }
}

// Segment scan: S_{j+1} = P_j S_j + L_j, written over L_j, per (b, h) and
// 16-column block; fp32.
template <int K>
__global__ __launch_bounds__(256) void kda_scan_kernel(ScanParams p) {
    constexpr int TPR = 256 / K;        // threads per state row
    constexpr int CPT = 16 / TPR;       // columns per thread
    __shared__ float sS[K * 16];
    const int ncb = p.V / 16;
    const int bh = blockIdx.x / ncb, cb = blockIdx.x % ncb;
    const int tid = threadIdx.x;
    const int row = tid / TPR, n0 = (tid % TPR) * CPT;
    const int V = p.V;
    const size_t col = (size_t)cb * 16 + n0;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
        sS[row * 16 + n0 + i] = p.s0 ? p.s0[((size_t)bh * K + row) * V + col + i] : 0.f;
    __syncthreads();
    for (int j = 0; j + 1 < p.n_seg; ++j) {
        const float* P = p.wsP + ((size_t)j * p.BH + bh) * K * K;
        float* Lj = p.wsL + ((size_t)j * p.BH + bh) * K * V;
        float acc[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) acc[i] = Lj[(size_t)row * V + col + i];
        for (int m = 0; m < K; m += 4) {
            const float4 pm = *reinterpret_cast<const float4*>(P + (size_t)row * K + m);
            const float pv[4] = {pm.x, pm.y, pm.z, pm.w};
#pragma unroll
            for (int mm = 0; mm < 4; ++mm)
#pragma unroll
                for (int i = 0; i < CPT; ++i) acc[i] += pv[mm] * sS[(m + mm) * 16 + n0 + i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            sS[row * 16 + n0 + i] = acc[i];
            Lj[(size_t)row * V + col + i] = acc[i];
        }
        __syncthreads();
    }
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

template <typename T, int K, int NW>
static hipError_t launch_chunk_t(const ChunkParams& p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((kda_chunk_kernel<T, K, NW>), dim3(grid), dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_chunk(int dtype, int K, int VB, const ChunkParams& p, int grid, hipStream_t stream) {
    if (grid <= 0) return hipSuccess;
    if (dtype == 1) {
        if (K == 128 && VB == 128) return launch_chunk_t<bf16, 128, 8>(p, grid, stream);
        if (K == 128 && VB == 64) return launch_chunk_t<bf16, 128, 4>(p, grid, stream);
        if (K == 64 && VB == 128) return launch_chunk_t<bf16, 64, 8>(p, grid, stream);
        if (K == 64 && VB == 64) return launch_chunk_t<bf16, 64, 4>(p, grid, stream);
    } else if (dtype == 0) {
        if (K == 64 && VB == 64) return launch_chunk_t<float, 64, 4>(p, grid, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_scan(int K, const ScanParams& p, hipStream_t stream) {
    const int grid = p.BH * (p.V / 16);
    if (grid <= 0 || p.n_seg < 2) return hipSuccess;
    if (K == 128) hipLaunchKernelGGL(kda_scan_kernel<128>, dim3(grid), dim3(256), 0, stream, p);
    else if (K == 64) hipLaunchKernelGGL(kda_scan_kernel<64>, dim3(grid), dim3(256), 0, stream, p);
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
