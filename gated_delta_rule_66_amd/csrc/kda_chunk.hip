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

template <typename T, int K, int NW>
struct ChunkLayout {
    static constexpr int VB = 16 * NW;           // value columns per workgroup
    static constexpr int NT = 64 * NW;           // threads
    static constexpr int SZ = (int)sizeof(T);
    static constexpr int PAD = 16 / SZ;          // 16 bytes of row padding
    static constexpr int LDK1 = K + PAD;         // Kd, Qd, Kinv: [token][channel], 16-byte reads
    static constexpr int LDK2 = K + 4;           // W, Q e^G: [token][channel], 8/16-byte reads
    static constexpr int LDT = C + PAD;          // [channel][token] rows
    static constexpr int LDL = C + 4;            // solve blocks / Mqk: [token][token]
    static constexpr int LDD = 16;               // fp32 diagonal blocks of A
    static constexpr int LDO = VB + PAD;         // output staging rows
    // prep mappings: a thread owns 2 adjacent channels and a run of tokens
    static constexpr int CPK = K / 2, PK = NT / CPK, TPK = C / PK;
    static constexpr int CPV = VB / 2, PV = NT / CPV, TPV = C / PV;
    // region KQ: Kd | Qd | Kinv (prep -> A/Mqk), then W | O (solve -> store)
    static constexpr int NAT1 = C * LDK1 * SZ;
    static constexpr int W_BYTES = C * LDK2 * SZ;
    static constexpr int KQ = cmax(3 * NAT1, W_BYTES + C * LDO * SZ);
    // region R: prep partial sums, then the solve blocks (L) and fp32 diagonals
    static constexpr int PART_BYTES = 2 * PK * K * 4;
    static constexpr int L_BYTES = C * LDL * SZ;
    static constexpr int R = cmax(PART_BYTES, L_BYTES + 4 * 16 * LDD * 4);
    static constexpr int oKQ = 0;
    static constexpr int oR = oKQ + KQ;
    static constexpr int oMqk = oR + R;                  // [C][LDL]
    static constexpr int oQh = oMqk + C * LDL * SZ;      // [C][LDK2] Q e^{G}
    static constexpr int oKhbT = oQh + C * LDK2 * SZ;    // [K][LDT] beta K e^{G}, channel-major
    static constexpr int oKbT = oKhbT + K * LDT * SZ;    // [K][LDT] K e^{G_C-G}, channel-major
    static constexpr int oVbT = oKbT + K * LDT * SZ;     // [VB][LDT] beta V, channel-major
    static constexpr int oF = oVbT + VB * LDT * SZ;      // fp32 [6][K] e^{G_b(i) - G_b(j)}
    static constexpr int oEGC = oF + 6 * K * 4;          // fp32 [K] e^{G_C}
    static constexpr int oBeta = oEGC + K * 4;           // fp32 [C]
    static constexpr int TOTAL = oBeta + C * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
    static_assert(CPK * PK == NT && TPK * PK == C && (TPK == 4 || TPK == 8 || TPK == 16), "key prep mapping");
    static_assert(CPV * PV == NT && TPV == 8, "value prep mapping");
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

// G (log2 units) at the first token of 16-token block `blk`, for channels
// c and c+1, from the per-part sums and first values.
template <int PK, int TPK, int K>
__device__ __forceinline__ float2 block_ref(const float* sPart, const float* sFirst, int blk, int c) {
    const int pb = 16 * blk / TPK;
    float2 r = *reinterpret_cast<const float2*>(&sFirst[pb * K + c]);
    for (int pp = 0; pp < pb; ++pp) {
        const float2 s = *reinterpret_cast<const float2*>(&sPart[pp * K + c]);
        r.x += s.x;
        r.y += s.y;
    }
    return r;
}

}  // namespace

template <typename T, int K, int NW>
__global__ __launch_bounds__(64 * NW) void kda_chunk_kernel(ChunkParams p) {
    using L = ChunkLayout<T, K, NW>;
    using Frag = typename FragOf<T>::type;
    using Frag4 = typename Frag4Of<T>::type;
    constexpr int VB = L::VB;
    constexpr int LDK1 = L::LDK1, LDK2 = L::LDK2, LDT = L::LDT, LDL = L::LDL, LDD = L::LDD, LDO = L::LDO;
    constexpr int CPK = L::CPK, PK = L::PK, TPK = L::TPK;
    constexpr int CPV = L::CPV, TPV = L::TPV;
    constexpr int NV8 = VB / 8;
    constexpr int REPO = C * NV8 / L::NT;      // output store packs per thread
    constexpr int KS = K / 32;                 // 32-deep slabs over key channels
    constexpr int CT = K / 16;                 // 16-row tiles of the state

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
    T* sKd = reinterpret_cast<T*>(smem + L::oKQ);
    T* sQd = sKd + C * LDK1;
    T* sKinv = sQd + C * LDK1;
    T* sW = reinterpret_cast<T*>(smem + L::oKQ);
    T* sO = reinterpret_cast<T*>(smem + L::oKQ + L::W_BYTES);
    float* sPart = reinterpret_cast<float*>(smem + L::oR);
    float* sFirst = sPart + PK * K;
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
    const int col0 = vb * VB;
    const bool pmode = p.summary && col0 < K;
    const int vcol0 = p.summary ? (pmode ? 0 : col0 - K) : col0;
    const int my_col = col0 + 16 * w + lr;

    const T* __restrict__ qg = reinterpret_cast<const T*>(p.q);
    const T* __restrict__ kg = reinterpret_cast<const T*>(p.k);
    const T* __restrict__ vg = reinterpret_cast<const T*>(p.v);
    const T* __restrict__ gg = reinterpret_cast<const T*>(p.g);
    const T* __restrict__ bg = reinterpret_cast<const T*>(p.beta);

    // prep mapping: key side (channels 2cp, 2cp+1; tokens pk*TPK ..), value side
    const int cp = tid % CPK, pk = tid / CPK;
    const int vp = tid % CPV, pv = tid / CPV;

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

    // ---- raw chunk registers (loaded one chunk ahead) ------------------------
    // (kept raw: converting at load time would make every load wait)
    Pack2<T> kr[TPK], qr[TPK], gr[TPK], vr[TPV];
    T br[TPK];
    // global addressing: a buffer resource at the chunk's first row (scalar
    // registers), a 32-bit lane byte offset and a scalar per-token offset;
    // one chunk of one head spans far less than 2^32 bytes
    constexpr unsigned SZ = sizeof(T);
    const unsigned rowK = (unsigned)p.H * K * SZ, rowV = (unsigned)p.H * V * SZ, rowB = (unsigned)p.H * SZ;
    const unsigned vK = (unsigned)pk * TPK * rowK + 2u * cp * SZ;   // lane offsets
    const unsigned vB = (unsigned)pk * TPK * rowB;
    const unsigned vV = (unsigned)pv * TPV * rowV + 2u * vp * SZ;
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
        for (int i = 0; i < TPK; ++i) {
            const int t = pk * TPK + i;
            if (t < nt) {
                buf_load2<T>(kr[i], rk, vK, i * rowK);
                buf_load2<T>(gr[i], rg, vK, i * rowK);
                if (!p.summary) buf_load2<T>(qr[i], rq, vK, i * rowK); else qr[i].zero();
                buf_load1(br[i], rb, vB, i * rowB);
            } else {
                kr[i].zero();
                gr[i].zero();
                qr[i].zero();
                br[i] = from_f32<T>(0.f);
            }
        }
#pragma unroll
        for (int i = 0; i < TPV; ++i) {
            const int t = pv * TPV + i;
            if (t < nt && !pmode) buf_load2<T>(vr[i], rv, vV, i * rowV);
            else vr[i].zero();
        }
    };
    if (c_begin < c_end) load_chunk(c_begin);

    for (int ci = c_begin; ci < c_end; ++ci) {
        const int t0 = ci * C;
        const int nt = min(C, p.T - t0);

        // ---- P1: in-chunk gate cumsum, part totals ----------------------------
        float gl0[TPK], gl1[TPK];
        {
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int i = 0; i < TPK; ++i) {
                s0 += clamp_gate_log2(gr[i].lo());
                s1 += clamp_gate_log2(gr[i].hi());
                gl0[i] = s0;
                gl1[i] = s1;
            }
            *reinterpret_cast<float2*>(&sPart[pk * K + 2 * cp]) = make_float2(s0, s1);
            *reinterpret_cast<float2*>(&sFirst[pk * K + 2 * cp]) = make_float2(gl0[0], gl1[0]);
            if (cp == 0) {
#pragma unroll
                for (int i = 0; i < TPK; ++i) sBeta[pk * TPK + i] = to_f32(br[i]);
            }
        }
        __syncthreads();

        // ---- P2: key/query-side operands (one pass, registers -> LDS) ---------
        {
            float off0 = 0.f, off1 = 0.f, tot0 = 0.f, tot1 = 0.f;
            for (int pp = 0; pp < PK; ++pp) {
                const float2 sp = *reinterpret_cast<const float2*>(&sPart[pp * K + 2 * cp]);
                if (pp < pk) { off0 += sp.x; off1 += sp.y; }
                tot0 += sp.x;
                tot1 += sp.y;
            }
            const float2 gb = block_ref<PK, TPK, K>(sPart, sFirst, (pk * TPK) / 16, 2 * cp);
            const float egb0 = fast_exp2(gb.x), egb1 = fast_exp2(gb.y);            // e^{G_b}      <= 1
            const float ecb0 = fast_exp2(tot0 - gb.x), ecb1 = fast_exp2(tot1 - gb.y);  // e^{G_C-G_b} <= 1
            float kh0[TPK], kh1[TPK], kb0[TPK], kb1[TPK];
#pragma unroll
            for (int i = 0; i < TPK; ++i) {
                const int t = pk * TPK + i;
                const float d0 = off0 + gl0[i] - gb.x, d1 = off1 + gl1[i] - gb.y;  // G_t - G_b <= 0
                const float e10 = fast_exp2(d0), e11 = fast_exp2(d1);     // e^{G_t-G_b}
                const float e20 = fast_exp2(-d0), e21 = fast_exp2(-d1);   // e^{G_b-G_t} <= e^75
                const float k0 = kr[i].lo(), k1 = kr[i].hi();
                const float q0 = qr[i].lo(), q1 = qr[i].hi();
                const float bt = to_f32(br[i]);
                st2(&sKd[t * LDK1 + 2 * cp], k0 * e10, k1 * e11);
                st2(&sKinv[t * LDK1 + 2 * cp], k0 * e20, k1 * e21);
                if (!p.summary) {
                    st2(&sQd[t * LDK1 + 2 * cp], q0 * e10, q1 * e11);
                    st2(&sQh[t * LDK2 + 2 * cp], q0 * e10 * egb0, q1 * e11 * egb1);
                }
                kh0[i] = bt * k0 * e10 * egb0;     // beta e^{G_t}
                kh1[i] = bt * k1 * e11 * egb1;
                kb0[i] = k0 * e20 * ecb0;          // e^{G_C-G_t}
                kb1[i] = k1 * e21 * ecb1;
            }
            st_run<TPK>(&sKhbT[(2 * cp) * LDT + pk * TPK], kh0);
            st_run<TPK>(&sKhbT[(2 * cp + 1) * LDT + pk * TPK], kh1);
            st_run<TPK>(&sKbT[(2 * cp) * LDT + pk * TPK], kb0);
            st_run<TPK>(&sKbT[(2 * cp + 1) * LDT + pk * TPK], kb1);
            if (pk == 0) *reinterpret_cast<float2*>(&sEGC[2 * cp]) = make_float2(fast_exp2(tot0), fast_exp2(tot1));
            for (int pr = pk; pr < 6; pr += PK) {
                int i, j;
                offdiag_pair(pr, i, j);
                const float2 gi = block_ref<PK, TPK, K>(sPart, sFirst, i, 2 * cp);
                const float2 gj = block_ref<PK, TPK, K>(sPart, sFirst, j, 2 * cp);
                *reinterpret_cast<float2*>(&sF[pr * K + 2 * cp]) =
                    make_float2(fast_exp2(gi.x - gj.x), fast_exp2(gi.y - gj.y));
            }
            // beta V, channel-major
            float bv0[TPV], bv1[TPV];
#pragma unroll
            for (int i = 0; i < TPV; ++i) {
                const float bt = sBeta[pv * TPV + i];
                bv0[i] = bt * vr[i].lo();
                bv1[i] = bt * vr[i].hi();
            }
            st_run<TPV>(&sVbT[(2 * vp) * LDT + pv * TPV], bv0);
            st_run<TPV>(&sVbT[(2 * vp + 1) * LDT + pv * TPV], bv1);
        }
        // the raw registers are consumed: fetch the next chunk behind the compute
        // (the scheduling fence keeps the loads from being hoisted above the
        // last uses, which would hold two chunks in registers)
        __builtin_amdgcn_sched_barrier(0);
        if (ci + 1 < c_end) load_chunk(ci + 1);
        __syncthreads();

        // ---- P3: A and Mqk, one 16 x 16 block pair per wave at a time ---------
        // A's diagonal blocks go to fp32 (for the block inverses), its
        // off-diagonal blocks to the solve buffer negated; Mqk blocks (0,1)
        // and (2,3) are zero (read by the 32-deep slabs of the output).
        for (int task = w; task < 12; task += NW) {
            if (task < 10) {
                int i, j;
                lower_pair(task, i, j);
                f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int c0 = 32 * ks + 8 * lg;
                    const Frag ak = ld_frag<T>(&sKd[(16 * i + lr) * LDK1 + c0]);
                    float kv[8];
                    ld8_as_f32<T>(&sKinv[(16 * j + lr) * LDK1 + c0], kv);
                    if (i != j) {
                        float f[8];
                        ld8f(&sF[(i * (i - 1) / 2 + j) * K + c0], f);
#pragma unroll
                        for (int e = 0; e < 8; ++e) kv[e] *= f[e];
                    }
                    const Frag bk = frag_from<T>(kv);
                    accA = mma(accA, ak, bk);
                    if (!p.summary) accM = mma(accM, ld_frag<T>(&sQd[(16 * i + lr) * LDK1 + c0]), bk);
                }
                const int r = 16 * j + lr;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 16 * i + 4 * lg + e;
                    const float a = sBeta[s] * accA[e];
                    if (i == j) sAd[(i * 16 + 4 * lg + e) * LDD + lr] = (r < s) ? a : 0.f;
                    else sL[s * LDL + r] = from_f32<T>(-a);
                    if (!p.summary) sMqk[s * LDL + r] = from_f32<T>((i > j || r <= s) ? accM[e] : 0.f);
                }
            } else if (!p.summary) {
                const int i = (task == 10) ? 0 : 2, j = i + 1;
#pragma unroll
                for (int e = 0; e < 4; ++e) sMqk[(16 * i + 4 * lg + e) * LDL + 16 * j + lr] = from_f32<T>(0.f);
            }
        }
        __syncthreads();

        // ---- P4: inverses D_i = (I + A_ii)^{-1} of the diagonal blocks --------
        // forward substitution in fp32, one lane per (block, column)
        if (w == 0) {
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
                float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) acc -= row[m] * xv[m];
                xv[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sL[(16 * i + r) * LDL + 16 * i + j] = from_f32<T>(xv[r]);
        }
        __syncthreads();

        // ---- P5: W = (I+A)^{-1} beta K e^G and U~ = (I+A)^{-1} beta V ---------
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
        f32x4 Ut[4];
        if (!pmode) {
            solve_tile(&sVbT[16 * w * LDT], Ut);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) Ut[i] = f32x4{0.f, 0.f, 0.f, 0.f};
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
                acc = mma(acc, ld_frag_perm<T>(&sW[(16 * ti + lr) * LDK2 + 32 * ks + 4 * lg]), Sb[ks]);
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
                    acc = mma(acc, ld_frag_perm<T>(&sQh[(16 * ti + lr) * LDK2 + 32 * ks + 4 * lg]), Sb[ks]);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (ks <= (ti >> 1))
                        acc = mma(acc, ld_frag_perm<T>(&sMqk[(16 * ti + lr) * LDL + 32 * ks + 4 * lg]), Ub[ks]);
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
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(reinterpret_cast<T*>(p.o) + ((size_t)(b * (size_t)p.T + t0) * p.H + h) * V + vcol0);
#pragma unroll
            for (int r = 0; r < REPO; ++r) {
                const int it = tid + r * L::NT;
                const int t = it / NV8, n8 = it % NV8;
                if (t < nt) {
                    const unsigned off = (unsigned)t * rowV + 8u * n8 * SZ;
                    buf_store16(ro, off, 0, *reinterpret_cast<const uint4*>(&sO[t * LDO + 8 * n8]));
                    if (SZ == 4) buf_store16(ro, off + 16, 0, *reinterpret_cast<const uint4*>(&sO[t * LDO + 8 * n8 + 4]));
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
