// KDA backward for gfx950: gradients of the prefill with respect to q, k, v,
// the log-gates g, beta and the initial state, given dL/do and dL/dS_T.
//
// The pages give no backward; this is the chain rule applied to the
// recurrence of the page "Kimi K3 — открытая модель, которая обошла закрытых
// лидеров рынка" (aiblin.ru), section "Как хранить миллион токенов в памяти",
// token by token in reverse:
//
//   dS  += q_t do_t^T              dq_t    = S_t do_t
//   du   = dS^T k_t                dk_t    = dS u_t + S'_t dy,   dy = -beta_t du
//   dv_t = beta_t du               dbeta_t = du . (v_t - y_t)
//   dS'  = dS + k_t dy^T           da_t    = rowsum(dS' * S_{t-1})
//   dS   = Diag(a_t) dS'           dg_t    = da_t a_t [-5 <= g_t <= 0]
//
// This file holds two parts of the backward.
//
// Token-level gradients (the schedule for shapes without the two-pass
// forward, fp32 with K or V = 128).  The recurrence acts on every value
// column separately, and so does the dS recurrence; only the key-side
// gradients (dq, dk, da, dbeta) sum over the columns.  A workgroup owns one
// (b, h, 16-column block) and the whole sequence: a forward sweep that
// stores its state slice every 8 tokens, then a reverse sweep that rebuilds
// each 8-token group's states in registers from its checkpoint and applies
// the reverse steps.  Per token it writes dv for its columns and its block's
// partial sums of dq, dk, da and dbeta; a second kernel adds the blocks'
// partials in a fixed order (deterministic) and applies the gate derivative.
//
// The reverse state pass of the chunk-form backward (kda_bwd_chunk.hip).
// The forward state pass maps S to U = U~ - W S, O = Qh S + Mqk U and
// S' = Diag(e^{G_C}) S + KbT U, so its transpose maps (dS', dO) to
//   dU = Mqk^T dO + KbT^T dS'
//   dS = Diag(e^{G_C}) dS' + Qh^T dO - W^T dU
// chunk by chunk from the end of the sequence.  It runs over the forward
// plan's segments like the forward: per-segment summaries of this affine map
// (a K x K transition and a K x V load), the segment scan from dL/dS_T, then
// every segment from its incoming adjoint, writing dL/dS at each chunk
// boundary and every chunk's dU.
//
// 256 threads: thread (cg = tid & 3, rg = tid >> 2) holds rows
// [RPT rg, RPT rg + RPT) x columns [4 cg, 4 cg + 4) of the K x 16 slice.
// Sums over rows reduce across the 16 lanes of a wave that share cg (xor
// shuffles by 4 .. 32), then across the 4 waves through LDS (one barrier);
// sums over columns reduce across the 4 lanes of a row group (xor 1, 2).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int BW_VB = 16;      // value columns per workgroup
constexpr int BW_GS = 8;       // tokens per checkpoint group

template <int N>
__device__ __forceinline__ void xor_sum(float (&x)[N], int mask) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __shfl_xor(x[i], mask);
}

}  // namespace

template <typename T, int K>
__global__ __launch_bounds__(256) void kda_bwd_kernel(BwdParams p) {
    constexpr int RPT = K / 64;                 // rows per thread
    constexpr int GS = BW_GS;
    static_assert(RPT * 64 == K, "rows per thread");

    // token data of one group (fp32): k, q, alpha per key channel; v, do per column; beta
    __shared__ float sk[GS][K], sq[GS][K], sa[GS][K];
    __shared__ float sv[GS][BW_VB], sdo[GS][BW_VB], sb[GS];
    __shared__ float red[2][4][2 * BW_VB];      // row-reduction exchange, double-buffered

    const int ncb = p.V / BW_VB;
    const int bh = blockIdx.x / ncb, cb = blockIdx.x % ncb;
    const int b = bh / p.H, h = bh % p.H;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int cg = tid & 3, rg = tid >> 2;
    const int row0 = RPT * rg;
    const int col0 = cb * BW_VB + 4 * cg;       // this thread's first value column
    const int T_ = p.T, H = p.H, V = p.V;
    const size_t KV = (size_t)K * V;
    const int NG = (T_ + GS - 1) / GS;
    float* ck = p.ckpt + (size_t)bh * NG * KV;  // [NG][K][V] fp32
    int rbuf = 0;

    // sum over all K rows of x[c] (this thread's 4 columns; NV = 4 or 8 values)
    auto row_reduce = [&](auto& x) {
        xor_sum(x, 4);
        xor_sum(x, 8);
        xor_sum(x, 16);
        xor_sum(x, 32);
        constexpr int NV = sizeof(x) / sizeof(float);
        if (l < 4) {
#pragma unroll
            for (int i = 0; i < NV; ++i) red[rbuf][w][(i / 4) * BW_VB + 4 * cg + (i % 4)] = x[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = (i / 4) * BW_VB + 4 * cg + (i % 4);
            x[i] = red[rbuf][0][c] + red[rbuf][1][c] + red[rbuf][2][c] + red[rbuf][3][c];
        }
        rbuf ^= 1;
    };
    // token rows of a group: fetched into registers one group ahead, then
    // written to LDS (so that the global loads of the next group overlap the
    // current one's steps)
    constexpr int NKE = (GS * K + 255) / 256;             // key-side elements per thread
    float rk[NKE], rg_[NKE], rq[NKE], rv, rdo, rb;
    auto fetch_group = [&](int gi, bool with_q) {
        const int t0 = gi * GS;
        const int n = min(GS, T_ - t0);
#pragma unroll
        for (int m = 0; m < NKE; ++m) {
            const int e = tid + 256 * m, r = e / K, i = e % K;
            rk[m] = rg_[m] = rq[m] = 0.f;
            if (r < n) {
                const size_t tok = ((size_t)b * T_ + t0 + r) * H + h;
                rk[m] = ld_scalar(reinterpret_cast<const T*>(p.k) + tok * K + i);
                rg_[m] = ld_scalar(reinterpret_cast<const T*>(p.g) + tok * K + i);
                if (with_q) rq[m] = ld_scalar(reinterpret_cast<const T*>(p.q) + tok * K + i);
            }
        }
        rv = rdo = rb = 0.f;
        if (tid < GS * BW_VB) {
            const int r = tid / BW_VB, c = tid % BW_VB;
            if (r < n) {
                const size_t tok = ((size_t)b * T_ + t0 + r) * H + h;
                rv = ld_scalar(reinterpret_cast<const T*>(p.v) + tok * V + cb * BW_VB + c);
                if (with_q && p.d_o) rdo = ld_scalar(reinterpret_cast<const T*>(p.d_o) + tok * V + cb * BW_VB + c);
            }
        }
        if (tid < GS && tid < n) rb = ld_scalar(reinterpret_cast<const T*>(p.beta) + ((size_t)b * T_ + t0 + tid) * H + h);
    };
    auto stage_group = [&]() {
        __syncthreads();                         // the previous group's readers are done
#pragma unroll
        for (int m = 0; m < NKE; ++m) {
            const int e = tid + 256 * m, r = e / K, i = e % K;
            if (r < GS) {
                sk[r][i] = rk[m];
                sa[r][i] = fast_exp2(clamp_gate_log2(rg_[m]));
                sq[r][i] = rq[m];
            }
        }
        if (tid < GS * BW_VB) {
            sv[tid / BW_VB][tid % BW_VB] = rv;
            sdo[tid / BW_VB][tid % BW_VB] = rdo;
        }
        if (tid < GS) sb[tid] = rb;
        __syncthreads();
    };
    // one forward token on the state slice: S <- Diag(a) S + k u^T
    auto fwd_token = [&](float (&S)[RPT][4], int r) {
        float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const float a = sa[r][row0 + j], kk = sk[r][row0 + j];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                S[j][c] *= a;
                y[c] += S[j][c] * kk;
            }
        }
        row_reduce(y);
        const float bt = sb[r];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float u = bt * (sv[r][4 * cg + c] - y[c]);
#pragma unroll
            for (int j = 0; j < RPT; ++j) S[j][c] += sk[r][row0 + j] * u;
        }
    };

    // ---- forward sweep: the state before every group's first token ----------------
    float S[RPT][4];
#pragma unroll
    for (int j = 0; j < RPT; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            S[j][c] = p.s0 ? p.s0[(size_t)bh * KV + (size_t)(row0 + j) * V + col0 + c] : 0.f;
    if (NG > 1) fetch_group(0, false);
    for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            *reinterpret_cast<f32x4*>(ck + (size_t)gi * KV + (size_t)(row0 + j) * V + col0) =
                f32x4{S[j][0], S[j][1], S[j][2], S[j][3]};
        if (gi + 1 == NG) break;                 // the last group's end state is not needed
        stage_group();
        if (gi + 2 < NG) fetch_group(gi + 1, false);
        for (int r = 0; r < GS; ++r) fwd_token(S, r);
    }

    // ---- reverse sweep ---------------------------------------------------------------
    float dS[RPT][4];
#pragma unroll
    for (int j = 0; j < RPT; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            dS[j][c] = p.dsT ? p.dsT[(size_t)bh * KV + (size_t)(row0 + j) * V + col0 + c] : 0.f;
    const size_t BTH = (size_t)p.B * T_ * H;
    if (NG > 0) fetch_group(NG - 1, true);
    for (int gi = NG - 1; gi >= 0; --gi) {
        const int t0 = gi * GS;
        const int n = min(GS, T_ - t0);
        stage_group();
        if (gi > 0) fetch_group(gi - 1, true);
        // St[r] = state before token t0 + r, r = 0..n
        float St[GS + 1][RPT][4];
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const f32x4 c4 = *reinterpret_cast<const f32x4*>(ck + (size_t)gi * KV + (size_t)(row0 + j) * V + col0);
#pragma unroll
            for (int c = 0; c < 4; ++c) St[0][j][c] = c4[c];
        }
#pragma unroll
        for (int r = 0; r < GS; ++r) {
            if (r < n) {
#pragma unroll
                for (int j = 0; j < RPT; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) St[r + 1][j][c] = St[r][j][c];
                fwd_token(St[r + 1], r);
            }
        }
#pragma unroll
        for (int r = GS - 1; r >= 0; --r) {
            if (r >= n) continue;
            const size_t tok = ((size_t)b * T_ + t0 + r) * H + h;
            const float bt = sb[r];
            float dov[4], vv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                dov[c] = sdo[r][4 * cg + c];
                vv[c] = sv[r][4 * cg + c];
            }
            // dS += q do^T;  dq = S_t do (this block's columns)
            float pq[RPT];
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const float qq = sq[r][row0 + j];
                pq[j] = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    dS[j][c] += qq * dov[c];
                    pq[j] += St[r + 1][j][c] * dov[c];
                }
            }
            // y = (Diag(a) S_{t-1})^T k and du = dS^T k, over all rows
            float yd[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            float P[RPT][4];
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const float a = sa[r][row0 + j], kk = sk[r][row0 + j];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    P[j][c] = a * St[r][j][c];
                    yd[c] += P[j][c] * kk;
                    yd[4 + c] += dS[j][c] * kk;
                }
            }
            row_reduce(yd);
            float u[4], dy[4], pb = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u[c] = bt * (vv[c] - yd[c]);
                dy[c] = -bt * yd[4 + c];
                pb += yd[4 + c] * (vv[c] - yd[c]);
            }
            if (rg == 0) {
                T* dvp = reinterpret_cast<T*>(p.dv) + tok * V + col0;
#pragma unroll
                for (int c = 0; c < 4; ++c) dvp[c] = from_f32<T>(bt * yd[4 + c]);
            }
            // dk = dS u + P dy;  dS' = dS + k dy^T;  da = rowsum(dS' * S_{t-1});  dS = Diag(a) dS'
            float pk[RPT], pa[RPT];
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const float a = sa[r][row0 + j], kk = sk[r][row0 + j];
                pk[j] = 0.f;
                pa[j] = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    pk[j] += dS[j][c] * u[c] + P[j][c] * dy[c];
                    const float dP = dS[j][c] + kk * dy[c];
                    pa[j] += dP * St[r][j][c];
                    dS[j][c] = a * dP;
                }
            }
            // the block's partial sums over its 16 columns
            float cs[3 * RPT + 1];
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                cs[j] = pq[j];
                cs[RPT + j] = pk[j];
                cs[2 * RPT + j] = pa[j];
            }
            cs[3 * RPT] = pb;
            xor_sum(cs, 1);
            xor_sum(cs, 2);
            if (cg == 0) {
                const size_t base = ((size_t)cb * BTH + tok) * K + row0;
#pragma unroll
                for (int j = 0; j < RPT; ++j) {
                    p.pdq[base + j] = cs[j];
                    p.pdk[base + j] = cs[RPT + j];
                    p.pda[base + j] = cs[2 * RPT + j];
                }
                if (rg == 0) p.pdb[(size_t)cb * BTH + tok] = cs[3 * RPT];
            }
        }
    }
    if (p.ds0) {
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            *reinterpret_cast<f32x4*>(p.ds0 + (size_t)bh * KV + (size_t)(row0 + j) * V + col0) =
                f32x4{dS[j][0], dS[j][1], dS[j][2], dS[j][3]};
    }
}

// ---- reverse state pass ------------------------------------------------------------
// Workgroup (b, h, segment, block of VB = 16 NW columns); wave w owns the
// block's 16-column tile w.  Per chunk, from the segment's last: the chunk's
// W, Qh, Mqk, KbT (staged transposed, so that each MFMA operand is read along
// its reduction index), e^{G_C} and dO^T of the block's columns go to LDS;
// dU and dS follow.  dS is the adjoint of the state after the previous chunk.
template <typename T, int K, int NW>
struct BwdStateLayout {
    static constexpr int SZ = (int)sizeof(T);
    static constexpr int PAD = 16 / SZ;
    static constexpr int VB = 16 * NW;
    static constexpr int NT = 64 * NW;
    // the record's matrices are staged transposed, so that every MFMA operand
    // is read along its reduction index
    static constexpr int LDK = K + PAD;          // Kb = KbT^T: [C][LDK]
    static constexpr int LDC = kChunk + PAD;     // W^T, Qh^T [K][LDC]; Mqk^T [C][LDC]; dO^T [VB][LDC]
    static constexpr int oWT = 0;
    static constexpr int oQhT = oWT + K * LDC * SZ;
    static constexpr int oMT = oQhT + K * LDC * SZ;
    static constexpr int oKb = oMT + kChunk * LDC * SZ;
    static constexpr int oDoT = oKb + kChunk * LDK * SZ;
    static constexpr int oEgc = oDoT + VB * LDC * SZ;
    static constexpr int TOTAL = oEgc + K * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
    // 16-byte pieces staged from a record: W | Qh | Mqk | KbT | e^{G_C}.  In
    // every matrix, consecutive pieces run down a column of the source (lanes
    // then write consecutive LDS addresses of the transposed row).
    static constexpr int PRK = K * SZ / 16, PRC = kChunk * SZ / 16;
    static constexpr int E1 = kChunk * PRK, E2 = E1 + kChunk * PRK, E3 = E2 + kChunk * PRC, E4 = E3 + K * PRC;
    static constexpr int PTOT = E4 + K * 4 / 16;
    static constexpr int NPT = (PTOT + NT - 1) / NT;
    // dO: VB columns of C token rows
    static constexpr int PDR = VB * SZ / 16;     // pieces per token row
    static constexpr int NPD = (kChunk * PDR + NT - 1) / NT;
};

template <typename T, int K, int NW, bool SUMMARY>
__global__ __launch_bounds__(64 * NW) void kda_bwd_state_kernel(BwdParams p) {
    using L = BwdStateLayout<T, K, NW>;
    using Frag = typename FragOf<T>::type;
    constexpr int C = kChunk, VB = L::VB, NT = L::NT, NPT = L::NPT, NPD = L::NPD;
    constexpr int LDK = L::LDK, LDC = L::LDC, CT = K / 16, KS = K / 32;
    constexpr int SZ = L::SZ, EPP = 16 / SZ;

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
    T* sWT = reinterpret_cast<T*>(smem + L::oWT);
    T* sQhT = reinterpret_cast<T*>(smem + L::oQhT);
    T* sMT = reinterpret_cast<T*>(smem + L::oMT);
    T* sKb = reinterpret_cast<T*>(smem + L::oKb);
    T* sDoT = reinterpret_cast<T*>(smem + L::oDoT);
    const float* sEgc = reinterpret_cast<const float*>(smem + L::oEgc);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lg = l >> 4, lr = l & 15;
    const int V = p.V, NC = p.NC, T_ = p.T, H = p.H;
    // workgroup (b, h, segment, column block).  Summary: segments 1 .. n_seg - 1,
    // columns [0, K + V): the first K carry the segment's transposed transition
    // (identity start, dO taken as zero), the others its load (zero start).
    // With load_only (the chunk-form backward) only the load columns run: the
    // reverse scan takes the transposes of the forward transitions instead.
    const bool lonly = SUMMARY && p.load_only;
    const int nvb = (SUMMARY && !lonly ? K + V : V) / VB;
    const int nseg_here = SUMMARY ? p.n_seg - 1 : p.n_seg;
    // the workgroups of one (b, h) read the same records: one XCD (L2)
    const int G = gridDim.x, x = blockIdx.x;
    const int lid = ((G & 7) == 0) ? (x & 7) * (G >> 3) + (x >> 3) : x;
    // block index over [0, K + V) columns in the summary (the load blocks
    // only: shifted past the K transition columns)
    const int vb = lid % nvb + (lonly ? K / VB : 0), rest = lid / nvb;
    static_assert(K % VB == 0, "whole transition blocks");
    const int seg = (rest % nseg_here) + (SUMMARY ? 1 : 0), bh = rest / nseg_here;
    const int b = bh / p.H, h = bh % p.H;
    const int c_begin = seg * p.cps, c_end = min(c_begin + p.cps, NC);
    const size_t KV = (size_t)K * V, BH = (size_t)p.B * p.H;
    const bool pmode = SUMMARY && vb * VB < K;
    const int vcol0 = SUMMARY ? (pmode ? 0 : vb * VB - K) : vb * VB;   // first value column of the block
    const int col = (pmode ? vb * VB : vcol0) + 16 * w + lr;            // this lane's column
    const RecLayout RL = rec_layout(K, V, SZ);
    const unsigned char* rec0 = p.rec + (size_t)bh * NC * RL.bytes;

    // dS' after the segment's last chunk, accumulator layout (rows 16 ct + 4 lg + e,
    // column lr): identity / zero (summary), dL/dS_T (last segment) or the segment
    // scan's result for this segment (slot n_seg - 2 - seg)
    const float* dinit = nullptr;
    if (!SUMMARY)
        dinit = seg == p.n_seg - 1 ? (p.dsT ? p.dsT + (size_t)bh * KV : nullptr)
                                   : p.wsL + ((size_t)(p.n_seg - 2 - seg) * BH + bh) * KV;
    f32x4 dS[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * ct + 4 * lg + e;
            dS[ct][e] = dinit ? dinit[(size_t)row * V + col] : (pmode && row == col ? 1.f : 0.f);
        }

    // two register sets: the loads of chunks ci - 1 and ci - 2 are in flight
    // during chunk ci.  A chunk before the segment gets empty resources (its
    // loads return zeros and touch no memory), so that every load is issued
    // unconditionally and each wait counts only the older set's loads.
    uint4 preA[NPT], dpreA[NPD], preB[NPT], dpreB[NPD];
    auto load_chunk = [&](int ci, uint4 (&pre)[NPT], uint4 (&dpre)[NPD]) {
        const bool live = ci >= c_begin;
        const int cl = live ? ci : c_begin;
        const __amdgpu_buffer_rsrc_t rr = make_rsrc_n(rec0 + (size_t)cl * RL.bytes, live ? (unsigned)RL.bytes : 0u);
#pragma unroll
        for (int m = 0; m < NPT; ++m) {
            const int pc = tid + NT * m;
            unsigned off;
            if (pc < L::E2) {                        // W, Qh [C][K]: piece (g, t) = row t, columns EPP g ..
                const int q = pc < L::E1 ? pc : pc - L::E1;
                off = (unsigned)(pc < L::E1 ? RL.oW : RL.oQh) + (unsigned)((q % C) * L::PRK + q / C) * 16u;
            } else if (pc < L::E3) {                 // Mqk [C][C]
                const int q = pc - L::E2;
                off = (unsigned)RL.oMqk + (unsigned)((q % C) * L::PRC + q / C) * 16u;
            } else if (pc < L::E4) {                 // KbT [K][C]: piece (tg, c) = row c, tokens EPP tg ..
                const int q = pc - L::E3;
                off = (unsigned)RL.oKbT + (unsigned)((q % K) * L::PRC + q / K) * 16u;
            } else {
                off = (unsigned)RL.oEgc + (unsigned)(pc - L::E4) * 16u;
            }
            pre[m] = pc < L::PTOT ? buf_load16(rr, off) : make_uint4(0, 0, 0, 0);
        }
        const int t0 = cl * C, nt = min(C, T_ - t0);
        const T* dob = (p.d_o && !pmode && live) ? reinterpret_cast<const T*>(p.d_o) + (((size_t)b * T_ + t0) * H + h) * V + vcol0
                                                 : nullptr;
        const unsigned rowV = (unsigned)H * V * SZ;
        // the chunk's token rows of the block's columns: rows past the sequence
        // end (and a null or empty source) read as zeros
        const __amdgpu_buffer_rsrc_t rd = make_rsrc_n(dob, dob ? (unsigned)(nt - 1) * rowV + (unsigned)(VB * SZ) : 0u);
#pragma unroll
        for (int m = 0; m < NPD; ++m) {
            const int pc = tid + NT * m, t = pc % C, sg = pc / C;
            dpre[m] = pc < C * L::PDR ? buf_load16(rd, (unsigned)t * rowV + (unsigned)sg * 16u) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_chunk = [&](const uint4 (&pre)[NPT], const uint4 (&dpre)[NPD]) {
#pragma unroll
        for (int m = 0; m < NPT; ++m) {
            const int pc = tid + NT * m;
            T v[EPP];
            __builtin_memcpy(v, &pre[m], 16);
            if (pc < L::E2) {                        // W^T, Qh^T [K][LDC]
                const int q = pc < L::E1 ? pc : pc - L::E1, t = q % C, g = q / C;
                T* d = (pc < L::E1 ? sWT : sQhT) + (EPP * g) * LDC + t;
#pragma unroll
                for (int e = 0; e < EPP; ++e) d[e * LDC] = v[e];
            } else if (pc < L::E3) {                 // Mqk^T [C][LDC]
                const int q = pc - L::E2, t = q % C, g = q / C;
#pragma unroll
                for (int e = 0; e < EPP; ++e) sMT[(EPP * g + e) * LDC + t] = v[e];
            } else if (pc < L::E4) {                 // Kb [C][LDK]
                const int q = pc - L::E3, c = q % K, g = q / K;
#pragma unroll
                for (int e = 0; e < EPP; ++e) sKb[(EPP * g + e) * LDK + c] = v[e];
            } else if (pc < L::PTOT) {
                *reinterpret_cast<uint4*>(smem + L::oEgc + (pc - L::E4) * 16) = pre[m];
            }
        }
        // dO^T: element e of piece (sg, t) is column EPP sg + e of token t
#pragma unroll
        for (int m = 0; m < NPD; ++m) {
            const int pc = tid + NT * m;
            if (pc < C * L::PDR) {
                const int t = pc % C, sg = pc / C;
                T v[EPP];
                __builtin_memcpy(v, &dpre[m], 16);
#pragma unroll
                for (int e = 0; e < EPP; ++e) sDoT[(EPP * sg + e) * LDC + t] = v[e];
            }
        }
    };

    // every chunk's dU goes to p.cdU (chunk-form gradients); the adjoint
    // before chunk ci to p.adj (ci >= 1) or p.ds0; false: nothing left to do
    auto step = [&](int ci, uint4 (&pre)[NPT], uint4 (&dpre)[NPD]) -> bool {
        store_chunk(pre, dpre);
        __syncthreads();
        load_chunk(ci - 2, pre, dpre);
        Frag bdo[2], bds[KS];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) bdo[ks] = ld_frag_perm<T>(&sDoT[(16 * w + lr) * LDC + 32 * ks + 4 * lg]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bds[ks] = frag_from_tiles<T>(dS[2 * ks], dS[2 * ks + 1]);
        // -dU = -(Mqk^T dO + KbT^T dS'), 4 token tiles
        f32x4 ndU[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc = mma(acc, ld_frag_perm<T>(&sMT[(16 * ti + lr) * LDC + 32 * ks + 4 * lg]), bdo[ks]);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mma(acc, ld_frag_perm<T>(&sKb[(16 * ti + lr) * LDK + 32 * ks + 4 * lg]), bds[ks]);
            ndU[ti] = -acc;
        }
        if (!SUMMARY) {
            // per-chunk lane offsets (not hoisted out of the chunk loop: registers)
            float* du = p.cdU + ((size_t)bh * NC + ci) * kChunk * V + (size_t)(4 * opaque(lg)) * V + opaque(col);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int e = 0; e < 4; ++e) du[(size_t)(16 * ti + e) * V] = -ndU[ti][e];
            if (ci == 0 && !p.ds0) return false;
        }
        Frag bdu[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) bdu[ks] = frag_from_tiles<T>(ndU[2 * ks], ndU[2 * ks + 1]);
        // dS = Diag(e^{G_C}) dS' + Qh^T dO - W^T dU (operands read per row tile:
        // hoisting all of them would exceed the 8-wave register budget)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            __builtin_amdgcn_sched_barrier(0);
            const f32x4 eg = *reinterpret_cast<const f32x4*>(&sEgc[16 * ct + 4 * lg]);
            f32x4 acc = dS[ct] * eg;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc = mma(acc, ld_frag_perm<T>(&sQhT[(16 * ct + lr) * LDC + 32 * ks + 4 * lg]), bdo[ks]);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc = mma(acc, ld_frag_perm<T>(&sWT[(16 * ct + lr) * LDC + 32 * ks + 4 * lg]), bdu[ks]);
            dS[ct] = acc;
        }
        if (!SUMMARY) {
            // the adjoint before chunk ci: after chunk ci - 1 (bf16 where the fused
            // chunk kernel reads it), or dL/dS_0 (fp32)
            const size_t lo = (size_t)(4 * opaque(lg)) * V + opaque(col);
            if (ci > 0 && p.adj16) {
                bf16* dst = reinterpret_cast<bf16*>(p.adj16) + ((size_t)bh * NC + ci - 1) * KV + lo;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[(size_t)(16 * ct + e) * V] = (bf16)dS[ct][e];
            } else {
                float* dst = (ci > 0 ? p.adj + ((size_t)bh * NC + ci - 1) * KV : p.ds0 + (size_t)bh * KV) + lo;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[(size_t)(16 * ct + e) * V] = dS[ct][e];
            }
        }
        __syncthreads();
        return true;
    };
    load_chunk(c_end - 1, preA, dpreA);
    load_chunk(c_end - 2, preB, dpreB);
    for (int ci = c_end - 1; ci >= c_begin; ci -= 2) {
        if (!step(ci, preA, dpreA)) break;
        if (ci - 1 < c_begin || !step(ci - 1, preB, dpreB)) break;
    }
    if (SUMMARY) {
        // the segment's map, at scan slot n_seg - 1 - seg: transition [K][K] or load [K][V]
        const int slot = p.n_seg - 1 - seg;
        float* dst = pmode ? p.wsP + ((size_t)slot * BH + bh) * K * K : p.wsL + ((size_t)slot * BH + bh) * KV;
        const int ld = pmode ? K : V;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(size_t)(16 * ct + 4 * lg + e) * ld + col] = dS[ct][e];
    }
}

// dq, dk, dg, dbeta: the column blocks' partials added in block order; dg
// takes the gate derivative a [-5 <= g <= 0].  One thread per (token, head,
// channel); the thread of channel 0 also writes dbeta.
template <typename T, int K>
__global__ __launch_bounds__(256) void kda_bwd_reduce_kernel(BwdParams p) {
    const size_t BTH = (size_t)p.B * p.T * p.H;
    const int ncb = p.V / BW_VB;
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= BTH * K) return;
    const size_t tok = e / K;
    float sq = 0.f, sk = 0.f, sa = 0.f;
    for (int cb = 0; cb < ncb; ++cb) {
        const size_t o = (size_t)cb * BTH * K + e;
        sq += p.pdq[o];
        sk += p.pdk[o];
        sa += p.pda[o];
    }
    const float gv = ld_scalar(reinterpret_cast<const T*>(p.g) + e);
    const float a = fast_exp2(clamp_gate_log2(gv));
    const float dg = (gv >= -5.f && gv <= 0.f) ? sa * a : 0.f;
    reinterpret_cast<T*>(p.dq)[e] = from_f32<T>(sq);
    reinterpret_cast<T*>(p.dk)[e] = from_f32<T>(sk);
    reinterpret_cast<T*>(p.dg)[e] = from_f32<T>(dg);
    if (e % K == 0) {
        float sb = 0.f;
        for (int cb = 0; cb < ncb; ++cb) sb += p.pdb[(size_t)cb * BTH + tok];
        reinterpret_cast<T*>(p.dbeta)[tok] = from_f32<T>(sb);
    }
}

template <typename T, int K>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
    const long wgs = (long)p.B * p.H * (p.V / BW_VB);
    if (wgs > 2000000000L) return hipErrorInvalidValue;
    hipLaunchKernelGGL((kda_bwd_kernel<T, K>), dim3((unsigned)wgs), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t n = (size_t)p.B * p.T * p.H * K;
    hipLaunchKernelGGL((kda_bwd_reduce_kernel<T, K>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_bwd(int dtype, int K, const BwdParams& p, hipStream_t stream) {
    if (dtype == 1) {
        if (K == 128) return launch_bwd_t<bf16, 128>(p, stream);
        if (K == 64) return launch_bwd_t<bf16, 64>(p, stream);
    } else if (dtype == 0) {
        if (K == 128) return launch_bwd_t<float, 128>(p, stream);
        if (K == 64) return launch_bwd_t<float, 64>(p, stream);
    }
    return hipErrorInvalidValue;
}

// 64 columns per workgroup (4 waves), or 128 (8 waves: each record staged
// once per (b, h, segment) where K = V = 128)
template <typename T, int K, int NW>
static hipError_t launch_bwd_state_t(bool summary, const BwdParams& p, hipStream_t stream) {
    const long segs = summary ? p.n_seg - 1 : p.n_seg;
    const long wgs = (long)p.B * p.H * segs * ((summary && !p.load_only ? K + p.V : p.V) / (16 * NW));
    if (wgs <= 0) return hipSuccess;
    if (wgs > 2000000000L) return hipErrorInvalidValue;
    if (summary)
        hipLaunchKernelGGL((kda_bwd_state_kernel<T, K, NW, true>), dim3((unsigned)wgs), dim3(64 * NW), 0, stream, p);
    else
        hipLaunchKernelGGL((kda_bwd_state_kernel<T, K, NW, false>), dim3((unsigned)wgs), dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_bwd_state(bool summary, int dtype, int K, const BwdParams& p, hipStream_t stream) {
    if (p.NC <= 0 || (long)p.B * p.H == 0) return hipSuccess;
    if (p.V % 64 != 0 || K % 64 != 0 || p.n_seg < 1 || p.cps < 1) return hipErrorInvalidValue;
    // the 8-wave variant's blocks: (K + V) / 128 in a full summary, V / 128 in a
    // load-only summary and in the per-segment pass
    if (dtype == 1) {
        if (K == 128 && p.V == 128) return launch_bwd_state_t<bf16, 128, 8>(summary, p, stream);
        if (K == 128) return launch_bwd_state_t<bf16, 128, 4>(summary, p, stream);
        if (K == 64) return launch_bwd_state_t<bf16, 64, 4>(summary, p, stream);
    } else if (dtype == 0) {
        if (K == 64) return launch_bwd_state_t<float, 64, 4>(summary, p, stream);
    }
    return hipErrorInvalidValue;
}

size_t bwd_workspace_bytes(int B, int T, int H, int K, int V) {
    const size_t NG = (size_t)((T + BW_GS - 1) / BW_GS);
    const size_t ck = (size_t)B * H * NG * K * V * sizeof(float);
    const size_t BTH = (size_t)B * T * H;
    const size_t ncb = (size_t)(V / BW_VB);
    const size_t pd = ncb * BTH * (3 * (size_t)K + 1) * sizeof(float);
    return ((ck + 255) & ~(size_t)255) + pd;
}

}  // namespace kda
