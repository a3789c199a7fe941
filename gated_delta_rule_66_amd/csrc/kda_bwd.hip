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
// The recurrence acts on every value column separately, and so does the dS
// recurrence; only the key-side gradients (dq, dk, da, dbeta) sum over the
// columns.  A workgroup therefore owns one (b, h, 16-column block) and runs
// the whole sequence: a forward sweep that stores its state slice every 8
// tokens, then a reverse sweep that rebuilds each 8-token group's states in
// registers from its checkpoint and applies the reverse steps.  Per token it
// writes dv for its columns and its block's partial sums of dq, dk, da and
// dbeta; a second kernel adds the blocks' partials in a fixed order
// (deterministic) and applies the gate derivative.
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

size_t bwd_workspace_bytes(int B, int T, int H, int K, int V) {
    const size_t NG = (size_t)((T + BW_GS - 1) / BW_GS);
    const size_t ck = (size_t)B * H * NG * K * V * sizeof(float);
    const size_t BTH = (size_t)B * T * H;
    const size_t ncb = (size_t)(V / BW_VB);
    const size_t pd = ncb * BTH * (3 * (size_t)K + 1) * sizeof(float);
    return ((ck + 255) & ~(size_t)255) + pd;
}

}  // namespace kda
