// KDA recurrent decode step for gfx950: one read and one write of the fp32
// state per (sequence, head) and token.
//
// Page: "Kimi K3 — открытая модель, которая обошла закрытых лидеров рынка"
// (aiblin.ru), section "Как хранить миллион токенов в памяти": a fixed-size
// state S replaces the KV cache and each token rewrites it (decay by the
// clamped forget gate alpha in [e^-5, 1], then the delta-rule erase/write
// with strength beta).  Per (n, h):
//   S' = Diag(alpha) S ;  y = S'^T k ;  z = S'^T q ;  u = beta (v - y)
//   S  = S' + k u^T    ;  o = S^T q = z + (q . k) u
// The value columns are independent: a workgroup of 256 threads owns VW
// columns of one (n, h) and tiles its K x VW slice as (row group) x
// (4-column group); partial dot products over rows are combined through
// LDS, and each thread rewrites exactly the 4-column slices it read
// (coalesced 16-byte accesses along V).  The kernel is HBM-bound: 8 K V bytes
// of state traffic against 7 K V flops; the state is streamed with
// non-temporal loads and stores (it is touched once per step).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename T, int K, int V, int VW>
__global__ __launch_bounds__(256) void kda_decode_kernel(DecodeParams p) {
    constexpr int NB = V / VW;           // workgroups per (n, h)
    constexpr int CG = VW / 4;           // 4-column groups
    constexpr int RG = 256 / CG;         // row groups
    constexpr int RPT = K / RG;          // state rows per thread
    static_assert(CG * RG == 256 && RPT * RG == K, "decode tiling");
    __shared__ float red[RG][CG][9];
    __shared__ float qk_part[RG];
    __shared__ float sk[K], sq[K], sa[K];

    const int nh = blockIdx.x / NB;
    const int cb = blockIdx.x % NB;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const int col = cb * VW + 4 * cg;
    const T* qp = reinterpret_cast<const T*>(p.q) + (size_t)nh * K;
    const T* kp = reinterpret_cast<const T*>(p.k) + (size_t)nh * K;
    const T* gp = reinterpret_cast<const T*>(p.g) + (size_t)nh * K;
    const T* vp = reinterpret_cast<const T*>(p.v) + (size_t)nh * V;
    float* S = p.state + (size_t)nh * K * V;

    // the token vectors once per workgroup
    for (int r = tid; r < K; r += 256) {
        sk[r] = ld_scalar(kp + r);
        sq[r] = ld_scalar(qp + r);
        sa[r] = fast_exp2(clamp_gate_log2(ld_scalar(gp + r)));
    }
    f32x4 x[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        x[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(rg * RPT + r) * V + col));
    __syncthreads();

    float s[RPT][4], kk[RPT];
    float y[4] = {0.f, 0.f, 0.f, 0.f}, z[4] = {0.f, 0.f, 0.f, 0.f};
    float qk = 0.f;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = rg * RPT + r;
        kk[r] = sk[row];
        const float qq = sq[row], a = sa[row];
#pragma unroll
        for (int i = 0; i < 4; ++i) s[r][i] = x[r][i] * a;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            y[i] += s[r][i] * kk[r];
            z[i] += s[r][i] * qq;
        }
        qk += qq * kk[r];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        red[rg][cg][i] = y[i];
        red[rg][cg][4 + i] = z[i];
    }
    if (cg == 0) qk_part[rg] = qk;
    __syncthreads();
    float yf[4] = {0.f, 0.f, 0.f, 0.f}, zf[4] = {0.f, 0.f, 0.f, 0.f};
    float qkf = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            yf[i] += red[r][cg][i];
            zf[i] += red[r][cg][4 + i];
        }
        qkf += qk_part[r];
    }
    const float beta = ld_scalar(reinterpret_cast<const T*>(p.beta) + nh);
    float u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = beta * (ld_scalar(vp + col + i) - yf[i]);
    if (rg == 0) {
        T* op = reinterpret_cast<T*>(p.o) + (size_t)nh * V + col;
#pragma unroll
        for (int i = 0; i < 4; ++i) op[i] = from_f32<T>(zf[i] + qkf * u[i]);
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = rg * RPT + r;
        f32x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = s[r][i] + kk[r] * u[i];
        __builtin_nontemporal_store(o4, reinterpret_cast<f32x4*>(S + (size_t)row * V + col));
    }
}

// T consecutive tokens of each sequence in one launch (multi-token
// verification): the tiling of kda_decode_kernel, the state slice held in
// registers across the tokens and written once; optionally the state after
// every token (so that a caller can resume after any accepted prefix).
template <typename T, int K, int V, int VW>
__global__ __launch_bounds__(256) void kda_decode_multi_kernel(MultiDecodeParams p) {
    constexpr int NB = V / VW;
    constexpr int CG = VW / 4;
    constexpr int RG = 256 / CG;
    constexpr int RPT = K / RG;
    static_assert(CG * RG == 256 && RPT * RG == K, "decode tiling");
    __shared__ float red[RG][CG][9];
    __shared__ float qk_part[RG];
    __shared__ float sk[K], sq[K], sa[K];

    const int nh = blockIdx.x / NB;
    const int cb = blockIdx.x % NB;
    const int n = nh / p.H, h = nh % p.H;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const int col = cb * VW + 4 * cg;
    float* S = p.state + (size_t)nh * K * V;

    f32x4 x[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        x[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(rg * RPT + r) * V + col));

    for (int t = 0; t < p.T; ++t) {
        const size_t tok = ((size_t)n * p.T + t) * p.H + h;
        const T* qp = reinterpret_cast<const T*>(p.q) + tok * K;
        const T* kp = reinterpret_cast<const T*>(p.k) + tok * K;
        const T* gp = reinterpret_cast<const T*>(p.g) + tok * K;
        const T* vp = reinterpret_cast<const T*>(p.v) + tok * V;
        __syncthreads();                                   // the previous token's LDS reads are done
        for (int r = tid; r < K; r += 256) {
            sk[r] = ld_scalar(kp + r);
            sq[r] = ld_scalar(qp + r);
            sa[r] = fast_exp2(clamp_gate_log2(ld_scalar(gp + r)));
        }
        __syncthreads();
        float kk[RPT];
        float y[4] = {0.f, 0.f, 0.f, 0.f}, z[4] = {0.f, 0.f, 0.f, 0.f};
        float qk = 0.f;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int row = rg * RPT + r;
            kk[r] = sk[row];
            const float qq = sq[row], a = sa[row];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[r][i] *= a;                              // S' = Diag(alpha) S
                y[i] += x[r][i] * kk[r];
                z[i] += x[r][i] * qq;
            }
            qk += qq * kk[r];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            red[rg][cg][i] = y[i];
            red[rg][cg][4 + i] = z[i];
        }
        if (cg == 0) qk_part[rg] = qk;
        __syncthreads();
        float yf[4] = {0.f, 0.f, 0.f, 0.f}, zf[4] = {0.f, 0.f, 0.f, 0.f};
        float qkf = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                yf[i] += red[r][cg][i];
                zf[i] += red[r][cg][4 + i];
            }
            qkf += qk_part[r];
        }
        const float beta = ld_scalar(reinterpret_cast<const T*>(p.beta) + tok);
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = beta * (ld_scalar(vp + col + i) - yf[i]);
        if (rg == 0) {
            T* op = reinterpret_cast<T*>(p.o) + tok * V + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) op[i] = from_f32<T>(zf[i] + qkf * u[i]);
        }
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[r][i] += kk[r] * u[i];   // S = S' + k u^T
        if (p.step_states) {
            float* D = p.step_states + tok * K * V;
#pragma unroll
            for (int r = 0; r < RPT; ++r)
                __builtin_nontemporal_store(x[r], reinterpret_cast<f32x4*>(D + (size_t)(rg * RPT + r) * V + col));
        }
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        __builtin_nontemporal_store(x[r], reinterpret_cast<f32x4*>(S + (size_t)(rg * RPT + r) * V + col));
}

// Token-serial prefill for the sizes without chunk kernels (fp32 inputs with
// K or V = 128): the same per-token recurrence as the decode step, with the
// workgroup's state slice kept in registers from the initial state to the
// final one and the next token's operands loaded while the current one is
// applied.  Exact in fp32; no chunk parallelism, so a chain's time grows with
// its length.  Optionally o <- o * sigmoid(z) (o rounded to the input type
// first, as in the chunk kernels' fused gate).
template <typename T, int K, int V, int VW>
__global__ __launch_bounds__(256) void kda_token_fwd_kernel(TokenFwdParams p) {
    constexpr int NB = V / VW;
    constexpr int CG = VW / 4;
    constexpr int RG = 256 / CG;
    constexpr int RPT = K / RG;
    static_assert(CG * RG == 256 && RPT * RG == K && K <= 256, "token tiling");
    __shared__ float red[RG][CG][9];
    __shared__ float qk_part[RG];
    __shared__ float sk[K], sq[K], sa[K];

    const int nh = blockIdx.x / NB;
    const int cb = blockIdx.x % NB;
    const int n = nh / p.H, h = nh % p.H;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const int col = cb * VW + 4 * cg;
    // token rows [row0, row0 + len) of this chain
    size_t row0;
    int len;
    if (p.cu_seqlens) {
        const int s0 = min(max(p.cu_seqlens[n], 0), p.T);
        const int s1 = max(s0, min(max(p.cu_seqlens[n + 1], 0), p.T));
        row0 = (size_t)s0;
        len = s1 - s0;
    } else {
        row0 = (size_t)n * p.T;
        len = p.T;
    }
    const T* qg = reinterpret_cast<const T*>(p.q);
    const T* kg = reinterpret_cast<const T*>(p.k);
    const T* gg = reinterpret_cast<const T*>(p.g);
    const T* vg = reinterpret_cast<const T*>(p.v);
    const T* bg = reinterpret_cast<const T*>(p.beta);
    const T* zg = reinterpret_cast<const T*>(p.gate);

    f32x4 x[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        x[r] = p.s0 ? *reinterpret_cast<const f32x4*>(p.s0 + (size_t)nh * K * V + (size_t)(rg * RPT + r) * V + col)
                    : f32x4{0.f, 0.f, 0.f, 0.f};

    // the operands of one token: channel tid of k, q, g (tid < K); this
    // thread's four v columns and gate inputs; beta
    float pk = 0.f, pq = 0.f, pg = 0.f, pb = 0.f, pv[4], pz[4];
    auto fetch = [&](int t) {
        const size_t tok = (row0 + (size_t)t) * p.H + h;
        if (tid < K) {
            pk = ld_scalar(kg + tok * K + tid);
            pq = ld_scalar(qg + tok * K + tid);
            pg = ld_scalar(gg + tok * K + tid);
        }
        pb = ld_scalar(bg + tok);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pv[i] = ld_scalar(vg + tok * V + col + i);
            pz[i] = zg ? ld_scalar(zg + tok * V + col + i) : 0.f;
        }
    };
    if (len > 0) fetch(0);
    for (int t = 0; t < len; ++t) {
        const float ck = pk, cq = pq, cgt = pg, beta = pb;
        float cv[4], cz[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            cv[i] = pv[i];
            cz[i] = pz[i];
        }
        if (t + 1 < len) fetch(t + 1);
        __syncthreads();                                   // the previous token's LDS reads are done
        if (tid < K) {
            sk[tid] = ck;
            sq[tid] = cq;
            sa[tid] = fast_exp2(clamp_gate_log2(cgt));
        }
        __syncthreads();
        float kk[RPT];
        float y[4] = {0.f, 0.f, 0.f, 0.f}, z[4] = {0.f, 0.f, 0.f, 0.f};
        float qk = 0.f;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int row = rg * RPT + r;
            kk[r] = sk[row];
            const float qq = sq[row], a = sa[row];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[r][i] *= a;                              // S' = Diag(alpha) S
                y[i] += x[r][i] * kk[r];
                z[i] += x[r][i] * qq;
            }
            qk += qq * kk[r];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            red[rg][cg][i] = y[i];
            red[rg][cg][4 + i] = z[i];
        }
        if (cg == 0) qk_part[rg] = qk;
        __syncthreads();
        float yf[4] = {0.f, 0.f, 0.f, 0.f}, zf[4] = {0.f, 0.f, 0.f, 0.f};
        float qkf = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                yf[i] += red[r][cg][i];
                zf[i] += red[r][cg][4 + i];
            }
            qkf += qk_part[r];
        }
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = beta * (cv[i] - yf[i]);
        if (rg == 0) {
            T* op = reinterpret_cast<T*>(p.o) + ((row0 + (size_t)t) * p.H + h) * V + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float ov = zf[i] + qkf * u[i];              // o = S^T q = z + (q . k) u
                if (zg) ov = to_f32(from_f32<T>(ov)) * sigmoidf_fast(cz[i]);
                op[i] = from_f32<T>(ov);
            }
        }
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[r][i] += kk[r] * u[i];   // S = S' + k u^T
    }
    if (p.sT) {
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            *reinterpret_cast<f32x4*>(p.sT + (size_t)nh * K * V + (size_t)(rg * RPT + r) * V + col) = x[r];
    }
}

template <typename T, int K, int V>
static hipError_t launch_token_fwd_t(const TokenFwdParams& p, hipStream_t stream) {
    constexpr int VW = 64;
    hipLaunchKernelGGL((kda_token_fwd_kernel<T, K, V, VW>), dim3(p.B * p.H * (V / VW)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_token_fwd_kv(int K, int V, const TokenFwdParams& p, hipStream_t stream) {
    if (K == 128 && V == 128) return launch_token_fwd_t<T, 128, 128>(p, stream);
    if (K == 128 && V == 64) return launch_token_fwd_t<T, 128, 64>(p, stream);
    if (K == 64 && V == 128) return launch_token_fwd_t<T, 64, 128>(p, stream);
    if (K == 64 && V == 64) return launch_token_fwd_t<T, 64, 64>(p, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_token_fwd(int dtype, int K, int V, const TokenFwdParams& p, hipStream_t stream) {
    if ((long)p.B * p.H <= 0) return hipSuccess;
    if ((long)p.B * p.H * 2 > 2000000000L) return hipErrorInvalidValue;
    if (dtype == 1) return launch_token_fwd_kv<bf16>(K, V, p, stream);
    if (dtype == 0) return launch_token_fwd_kv<float>(K, V, p, stream);
    return hipErrorInvalidValue;
}

// 64 columns per workgroup: a 128-wide state is split over two workgroups
// (more of them in flight for the same bytes per step; measured faster)
template <typename T, int K, int V>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
    constexpr int VW = 64;
    hipLaunchKernelGGL((kda_decode_kernel<T, K, V, VW>), dim3(p.NH * (V / VW)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_kv(int K, int V, const DecodeParams& p, hipStream_t stream) {
    if (K == 128 && V == 128) return launch_decode_t<T, 128, 128>(p, stream);
    if (K == 128 && V == 64) return launch_decode_t<T, 128, 64>(p, stream);
    if (K == 64 && V == 128) return launch_decode_t<T, 64, 128>(p, stream);
    if (K == 64 && V == 64) return launch_decode_t<T, 64, 64>(p, stream);
    return hipErrorInvalidValue;
}

template <typename T, int K, int V>
static hipError_t launch_decode_multi_t(const MultiDecodeParams& p, hipStream_t stream) {
    constexpr int VW = 64;
    hipLaunchKernelGGL((kda_decode_multi_kernel<T, K, V, VW>), dim3(p.N * p.H * (V / VW)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_multi_kv(int K, int V, const MultiDecodeParams& p, hipStream_t stream) {
    if (K == 128 && V == 128) return launch_decode_multi_t<T, 128, 128>(p, stream);
    if (K == 128 && V == 64) return launch_decode_multi_t<T, 128, 64>(p, stream);
    if (K == 64 && V == 128) return launch_decode_multi_t<T, 64, 128>(p, stream);
    if (K == 64 && V == 64) return launch_decode_multi_t<T, 64, 64>(p, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_multi(int dtype, int K, int V, const MultiDecodeParams& p, hipStream_t stream) {
    if ((long)p.N * p.H <= 0 || p.T <= 0) return hipSuccess;
    if ((long)p.N * p.H * 2 > 2000000000L) return hipErrorInvalidValue;
    if (dtype == 1) return launch_decode_multi_kv<bf16>(K, V, p, stream);
    if (dtype == 0) return launch_decode_multi_kv<float>(K, V, p, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_decode(int dtype, int K, int V, const DecodeParams& p, hipStream_t stream) {
    if (p.NH <= 0) return hipSuccess;
    if ((long)p.NH * 2 > 2000000000L) return hipErrorInvalidValue;
    if (dtype == 1) return launch_decode_kv<bf16>(K, V, p, stream);
    if (dtype == 0) return launch_decode_kv<float>(K, V, p, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
