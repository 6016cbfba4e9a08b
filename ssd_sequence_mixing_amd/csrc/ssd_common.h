// Device-side helpers shared by the libssd kernels (gfx950 / CDNA4 only).
//
// Global memory is read and written through raw buffer resources: every
// access carries a byte range, and the hardware returns zero for loads and
// drops stores outside it. The kernels build one resource per batch element
// (its X / B / C / Y slab), so tokens past the end of a sequence read as zero
// and are never written, which is how a partial last chunk is handled.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Word 3 of a raw (unstructured) buffer resource on the gfx9 family.
constexpr int kRsrcWord3 = 0x00020000;
// An offset beyond every range a kernel builds: loads return 0, stores drop.
constexpr uint32_t kOOB = 0x80000000u;

// Offset `off`, or one past every range when `bad`: bit 31 is set, and every
// range a kernel builds is under 2 GiB. Arithmetic rather than a select, so
// the compiler keeps one load instead of branching around two.
__device__ __forceinline__ uint32_t oob_if(bool bad, uint32_t off) {
    return off | ((uint32_t)bad << 31);
}

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

__device__ __forceinline__ u32x4 buf_ld128(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_ld64(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_ld32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t buf_ld16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
// The same with a scalar (wave-uniform) offset added: voff per lane, soff per wave.
__device__ __forceinline__ u32x4 buf_ld128s(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ void buf_st128s(u32x4 v, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, 0);
}
__device__ __forceinline__ void buf_st64s(u32x2 v, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, 0);
}
__device__ __forceinline__ void buf_st128(u32x4 v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_st64(u32x2 v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_st32(uint32_t v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_st16(uint16_t v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32). The kernels keep log-decays in
// base 2, so every decay factor is one instruction. exp2(-inf) = 0 and
// exp2(0) = 1 exactly.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

// The step-size prologue of a Mamba-2 layer, optionally fused into the core.
// mode 0: dt = raw + bias; 1: dt = softplus(raw + bias); 2: dt = softplus(raw)
// + bias (the bias after the softplus, as the Mamba explainer page's
// training-stability notes write it). softplus(x) = log(1 + e^x) = log1p(u),
// u = e^x from the hardware's 2^x: for u < 1/32 the series u - u^2/2 + u^3/3
// - u^4/4 + u^5/5 (truncation below u^5/6 < 2e-9 relative), else ln 2 log2(1 + u)
// with the hardware's log2 (rounding 1 + u costs under 3e-6 relative there);
// x itself above 20, where e^{-x} is below fp32 resolution.
constexpr float kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float softplus_f32(float x) {
    if (x > 20.f) return x;
    const float u = __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
    if (u < 0.03125f) return u * (1.f - u * (0.5f - u * (1.f / 3.f - u * (0.25f - u * 0.2f))));
    return kLn2 * __builtin_amdgcn_logf(1.f + u);
}
__device__ __forceinline__ float dt_prologue(float raw, float bias, int mode) {
    if (mode == 1) return softplus_f32(raw + bias);
    if (mode == 2) return softplus_f32(raw) + bias;
    return raw + bias;
}

// The output gate: y * silu(z) = y * z / (1 + e^{-z}).
__device__ __forceinline__ float silu_gate(float y, float z) { return y * (z / (1.f + expf(-z))); }

// ---------------------------------------------------------------------------
// Storage-type traits. A "fragment" is the 8 consecutive K-elements one lane
// contributes to a 16x16x32 matrix-core product.
//
// Matrix-core layout used throughout (v_mfma_f32_16x16x32_bf16 on gfx950):
//   lane l = 16*kg + r (r = l % 16, kg = l / 16)
//   A operand: A[r][8*kg + e], e = 0..7         (row r, 8 consecutive k)
//   B operand: B[8*kg + e][r], e = 0..7         (column r, 8 consecutive k)
//   D result : D[4*kg + i][r], i = 0..3         (4 consecutive rows, column r)
// For fp32 storage the same per-lane fragments feed eight
// v_mfma_f32_16x16x4_f32 products, product e taking element e of every lane:
// that covers k = 8*kg + e for all kg and e, the same 32-long sum.
// ---------------------------------------------------------------------------
template <typename T> struct Traits;

template <> struct Traits<bf16> {
    static constexpr int kBytes = 2;
    typedef bf16x8 frag;
    __device__ static __forceinline__ frag load_frag(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(bf16x8, buf_ld128(r, off));
    }
    __device__ static __forceinline__ frag load_frag_s(rsrc_t r, uint32_t voff, uint32_t soff) {
        return __builtin_bit_cast(bf16x8, buf_ld128s(r, voff, soff));
    }
    __device__ static __forceinline__ frag lds_frag(const bf16 *p) {
        return *reinterpret_cast<const bf16x8 *>(p);
    }
    __device__ static __forceinline__ float to_f32(bf16 v) { return (float)v; }
    __device__ static __forceinline__ bf16 from_f32(float v) { return (bf16)v; }
    __device__ static __forceinline__ float frag_get(const frag &f, int e) { return (float)f[e]; }
    __device__ static __forceinline__ void frag_set(frag &f, int e, float v) { f[e] = (bf16)v; }
    __device__ static __forceinline__ f32x4 mma(const frag &a, const frag &b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Traits<float> {
    static constexpr int kBytes = 4;
    typedef f32x8 frag;
    __device__ static __forceinline__ frag load_frag(rsrc_t r, uint32_t off) {
        u32x4 lo = buf_ld128(r, off);
        u32x4 hi = buf_ld128(r, off + 16);
        f32x4 a = __builtin_bit_cast(f32x4, lo), b = __builtin_bit_cast(f32x4, hi);
        frag f;
        f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
        f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
        return f;
    }
    __device__ static __forceinline__ frag load_frag_s(rsrc_t r, uint32_t voff, uint32_t soff) {
        u32x4 lo = buf_ld128s(r, voff, soff);
        u32x4 hi = buf_ld128s(r, voff + 16, soff);
        f32x4 a = __builtin_bit_cast(f32x4, lo), b = __builtin_bit_cast(f32x4, hi);
        frag f;
        f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
        f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
        return f;
    }
    __device__ static __forceinline__ frag lds_frag(const float *p) {
        const f32x4 *q = reinterpret_cast<const f32x4 *>(p);
        f32x4 a = q[0], b = q[1];
        frag f;
        f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
        f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
        return f;
    }
    __device__ static __forceinline__ float to_f32(float v) { return v; }
    __device__ static __forceinline__ float from_f32(float v) { return v; }
    __device__ static __forceinline__ float frag_get(const frag &f, int e) { return f[e]; }
    __device__ static __forceinline__ void frag_set(frag &f, int e, float v) { f[e] = v; }
    __device__ static __forceinline__ f32x4 mma(const frag &a, const frag &b, f32x4 c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
        return c;
    }
};

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

}  // namespace ssd
