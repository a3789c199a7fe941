// Device-side helpers for the gfx950 KDA kernels: element types, MFMA
// fragments and their LDS loads.
//
// MFMA conventions (v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x4_f32,
// wave64): for a 16x16 output tile D = A (16 x Kred) * B (Kred x 16),
//   * accumulator / result: lane l holds D[4*(l/16) + e][l % 16], e = 0..3;
//   * an operand "fragment" covers a 32-deep slab of the reduction: lane l
//     holds 8 reduction slots for row (A) or column (B) l % 16, slots owned by
//     lane group l/16.  Any assignment of reduction indices to slots works
//     as long as A and B use the same one, so two assignments are used:
//       natural : slot (g, i) -> 8*g + i            (one 16-byte LDS read)
//       permuted: slot (g, i) -> 16*(i/4) + 4*g + i%4
//     The permuted one makes two vertically stacked result tiles, as they sit
//     in the accumulator registers, a B fragment directly (and a transposed A
//     fragment), so a state or error tile never leaves registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <typename T> struct FragOf;
template <> struct FragOf<bf16> { typedef bf16x8 type; };
template <> struct FragOf<float> { typedef f32x8 type; };

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// ---- MFMA: acc += A * B over one 32-deep slab --------------------------------
__device__ __forceinline__ f32x4 mma(f32x4 acc, bf16x8 a, bf16x8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x4 acc, f32x8 a, f32x8 b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
    return acc;
}
// ---- MFMA over a 16-deep slab (16x16x16 bf16 / four 16x16x4 fp32) --------------
// Slot (g, i) of lane l holds reduction index 4*g + i (g = l/16): a result tile
// in accumulator layout is a B operand of this shape as it stands.
template <typename T> struct Frag4Of;
template <> struct Frag4Of<bf16> { typedef bf16x4 type; };
template <> struct Frag4Of<float> { typedef f32x4 type; };

__device__ __forceinline__ f32x4 mma16(f32x4 acc, bf16x4 a, bf16x4 b) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x4 acc, f32x4 a, f32x4 b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
    return acc;
}
template <typename T> __device__ __forceinline__ typename Frag4Of<T>::type frag4_from(f32x4 x);
template <> __device__ __forceinline__ bf16x4 frag4_from<bf16>(f32x4 x) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (bf16)x[i];
    return r;
}
template <> __device__ __forceinline__ f32x4 frag4_from<float>(f32x4 x) { return x; }
// 4 consecutive elements (8-byte aligned for bf16, 16 for fp32)
template <typename T> __device__ __forceinline__ typename Frag4Of<T>::type ld_frag4(const T* p) {
    return *reinterpret_cast<const typename Frag4Of<T>::type*>(p);
}
template <typename T> __device__ __forceinline__ f32x4 ld4_as_f32(const T* p) {
    typename Frag4Of<T>::type f = ld_frag4<T>(p);
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = to_f32(f[i]);
    return r;
}

// ---- fragment construction ----------------------------------------------------
template <typename T> __device__ __forceinline__ typename FragOf<T>::type frag_from(const float* x);
template <> __device__ __forceinline__ bf16x8 frag_from<bf16>(const float* x) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (bf16)x[i];
    return r;
}
template <> __device__ __forceinline__ f32x8 frag_from<float>(const float* x) {
    f32x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = x[i];
    return r;
}

// two stacked accumulator tiles -> one permuted-slot fragment
template <typename T>
__device__ __forceinline__ typename FragOf<T>::type frag_from_tiles(f32x4 top, f32x4 bot) {
    float x[8] = {top[0], top[1], top[2], top[3], bot[0], bot[1], bot[2], bot[3]};
    return frag_from<T>(x);
}

// natural slots: 8 consecutive elements (16-byte aligned for bf16, 32 for f32)
template <typename T> __device__ __forceinline__ typename FragOf<T>::type ld_frag(const T* p);
template <> __device__ __forceinline__ bf16x8 ld_frag<bf16>(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}
template <> __device__ __forceinline__ f32x8 ld_frag<float>(const float* p) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    f32x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[4 + i] = b[i]; }
    return r;
}

// permuted slots: elements p[0..3] and p[16..19]
template <typename T> __device__ __forceinline__ typename FragOf<T>::type ld_frag_perm(const T* p);
template <> __device__ __forceinline__ bf16x8 ld_frag_perm<bf16>(const bf16* p) {
    bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
    bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16);
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[4 + i] = b[i]; }
    return r;
}
template <> __device__ __forceinline__ f32x8 ld_frag_perm<float>(const float* p) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 16);
    f32x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[4 + i] = b[i]; }
    return r;
}

// 8 consecutive fp32 values from LDS (16-byte aligned)
// The value unchanged, hidden from the optimiser: index arithmetic derived
// from it is redone where it is used instead of being hoisted out of a
// persistent loop and kept live (or spilled) across the whole body.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

__device__ __forceinline__ void ld8f(const float* p, float* x) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
}

// ---- 2-element (channel pair) global / LDS I/O in the input dtype ------------
template <typename T> struct Pack2;
template <> struct Pack2<bf16> {
    uint32_t d;
    __device__ __forceinline__ void load(const bf16* p) { d = *reinterpret_cast<const uint32_t*>(p); }
    __device__ __forceinline__ void zero() { d = 0u; }
    __device__ __forceinline__ float lo() const { return __uint_as_float(d << 16); }
    __device__ __forceinline__ float hi() const { return __uint_as_float(d & 0xffff0000u); }
};
template <> struct Pack2<float> {
    float2 d;
    __device__ __forceinline__ void load(const float* p) { d = *reinterpret_cast<const float2*>(p); }
    __device__ __forceinline__ void zero() { d = make_float2(0.f, 0.f); }
    __device__ __forceinline__ float lo() const { return d.x; }
    __device__ __forceinline__ float hi() const { return d.y; }
};
__device__ __forceinline__ void st2(bf16* p, float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r;
    r[0] = (bf16)a;
    r[1] = (bf16)b;
    *reinterpret_cast<bf16x2*>(p) = r;
}
__device__ __forceinline__ void st2(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
}
// N consecutive values stored as N elements of T (N * sizeof(T) >= 8 bytes,
// aligned to min(16, N * sizeof(T)))
template <int N> __device__ __forceinline__ void st_run(bf16* p, const float* x) {
    static_assert(N % 4 == 0, "run length");
    if constexpr (N % 8 == 0) {
#pragma unroll
        for (int j = 0; j < N; j += 8) {
            bf16x8 r;
#pragma unroll
            for (int i = 0; i < 8; ++i) r[i] = (bf16)x[j + i];
            *reinterpret_cast<bf16x8*>(p + j) = r;
        }
    } else {
#pragma unroll
        for (int j = 0; j < N; j += 4) {
            bf16x4 r;
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] = (bf16)x[j + i];
            *reinterpret_cast<bf16x4*>(p + j) = r;
        }
    }
}
template <int N> __device__ __forceinline__ void st_run(float* p, const float* x) {
    static_assert(N % 4 == 0, "run length");
#pragma unroll
    for (int j = 0; j < N; j += 4)
        *reinterpret_cast<float4*>(p + j) = make_float4(x[j], x[j + 1], x[j + 2], x[j + 3]);
}

// ---- buffer (descriptor-based) global access -------------------------------------
// A raw buffer resource over a chunk's base address: the base lives in scalar
// registers and every lane adds only a 32-bit byte offset, plus a wave-uniform
// scalar offset per load.  No range clamping (records = 0xffffffff); callers
// mask out-of-range rows themselves.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xffffffff, 0x00020000);
}
// a resource over the first `bytes` bytes at base: loads at or past the end
// return zeros (range checking of raw buffer accesses), so conditional reads
// need no branch; bytes = 0 (e.g. a null source) reads zeros only
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_n(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <typename T> __device__ __forceinline__ void buf_load2(Pack2<T>& x, __amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff);
template <> __device__ __forceinline__ void buf_load2<bf16>(Pack2<bf16>& x, __amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    x.d = __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
template <> __device__ __forceinline__ void buf_load2<float>(Pack2<float>& x, __amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
    x.d = make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
}
// one element, kept raw (converted when used)
__device__ __forceinline__ void buf_load1(bf16& x, __amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    const unsigned short u = __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
    x = __builtin_bit_cast(bf16, u);
}
__device__ __forceinline__ void buf_load1(float& x, __amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}
template <typename T> struct Pack8;
template <typename T> __device__ __forceinline__ void buf_load8(Pack8<T>& x, __amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff);
__device__ __forceinline__ void buf_store1(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, bf16 x) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void buf_store1(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, uint4 v) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 x = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)voff, (int)soff, 0);
}

// ---- 8-element global I/O in the input dtype ---------------------------------
// A "pack" is 8 consecutive input elements: 16 bytes of bf16 or 32 of fp32.
template <typename T> struct Pack8;
template <> struct Pack8<bf16> {
    uint4 d;
    __device__ __forceinline__ void load(const bf16* p) { d = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ void zero() { d = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ void to_f32(float* x) const {
        const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct Pack8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    __device__ __forceinline__ void zero() { a = make_float4(0, 0, 0, 0); b = a; }
    __device__ __forceinline__ void to_f32(float* x) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
};

template <> __device__ __forceinline__ void buf_load8<bf16>(Pack8<bf16>& x, __amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    x.d = make_uint4(v[0], v[1], v[2], v[3]);
}
template <> __device__ __forceinline__ void buf_load8<float>(Pack8<float>& x, __amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff + 16, (int)soff, 0);
    x.a = make_float4(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]), __uint_as_float(a[3]));
    x.b = make_float4(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[2]), __uint_as_float(b[3]));
}

// N (1, 2, 4 or a multiple of 4) consecutive values stored as elements of T
template <int N> __device__ __forceinline__ void st_small(bf16* p, const float* x) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    if constexpr (N == 1) {
        *p = (bf16)x[0];
    } else if constexpr (N == 2) {
        bf16x2 r;
        r[0] = (bf16)x[0];
        r[1] = (bf16)x[1];
        *reinterpret_cast<bf16x2*>(p) = r;
    } else {
        st_run<N>(p, x);
    }
}
template <int N> __device__ __forceinline__ void st_small(float* p, const float* x) {
    if constexpr (N == 1) {
        *p = x[0];
    } else if constexpr (N == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
    } else {
        st_run<N>(p, x);
    }
}

// store 8 fp32 values as 8 elements of T (16-byte aligned for bf16)
__device__ __forceinline__ void st8(bf16* p, const float* x) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (bf16)x[i];
    *reinterpret_cast<bf16x8*>(p) = r;
}
__device__ __forceinline__ void st8(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// ---- wave-level LDS exchange ------------------------------------------------------
// Lanes of one wave that hand data to each other through LDS: the wave's LDS
// operations execute in order, so a compiler fence (no hardware wait) between
// the writes and the reads is enough.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- scalar math ---------------------------------------------------------------
constexpr float kLog2e = 1.4426950408889634f;

// exp2 on the hardware transcendental unit (v_exp_f32)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// forget-gate clamp in log space: log alpha in [-5, 0]; returned in log2 units
__device__ __forceinline__ float clamp_gate_log2(float g) {
    return fminf(fmaxf(g, -5.0f), 0.0f) * kLog2e;
}

__device__ __forceinline__ float ld_scalar(const bf16* p) { return (float)*p; }
__device__ __forceinline__ float ld_scalar(const float* p) { return *p; }

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned voff) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Output gate on one 16-byte piece of o (input dtype): o * sigmoid(z), z of
// the same layout; both widened to fp32, the product rounded once.
__device__ __forceinline__ float sigmoidf_fast(float z) {
    return __builtin_amdgcn_rcpf(1.f + fast_exp2(-1.4426950408889634f * z));
}
__device__ __forceinline__ uint4 gate_piece(uint4 o, uint4 z, const bf16*) {
    const uint32_t ow[4] = {o.x, o.y, o.z, o.w}, zw[4] = {z.x, z.y, z.z, z.w};
    float r[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = __uint_as_float(ow[i] << 16) * sigmoidf_fast(__uint_as_float(zw[i] << 16));
        r[2 * i + 1] = __uint_as_float(ow[i] & 0xffff0000u) * sigmoidf_fast(__uint_as_float(zw[i] & 0xffff0000u));
    }
    const bf16x8 b = frag_from<bf16>(r);
    return *reinterpret_cast<const uint4*>(&b);
}
__device__ __forceinline__ uint4 gate_piece(uint4 o, uint4 z, const float*) {
    return make_uint4(__float_as_uint(__uint_as_float(o.x) * sigmoidf_fast(__uint_as_float(z.x))),
                      __float_as_uint(__uint_as_float(o.y) * sigmoidf_fast(__uint_as_float(z.y))),
                      __float_as_uint(__uint_as_float(o.z) * sigmoidf_fast(__uint_as_float(z.z))),
                      __float_as_uint(__uint_as_float(o.w) * sigmoidf_fast(__uint_as_float(z.w))));
}

}  // namespace kda
