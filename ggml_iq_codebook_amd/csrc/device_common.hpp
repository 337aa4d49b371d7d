// device_common.hpp -- small device helpers shared by the HIP kernels of
// libiqcodec.so: fp16 conversion, bf16 operand splitting, status reporting,
// block geometry, reading weights of every storage type as fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "iq_codec.h"

namespace iqk {

constexpr int kWave = 64;
constexpr int kBlockElems = 256;

// float32 -> IEEE binary16 bits, round to nearest, ties to even, done with
// integer operations so the result does not depend on the FP mode registers.
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f)
{
    const uint32_t x = __float_as_uint(f);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const uint32_t a = x & 0x7fffffffu;
    if (a >= 0x7f800000u) return sign | 0x7c00u | (a > 0x7f800000u ? 0x200u : 0u);
    if (a >= 0x477ff000u) return sign | 0x7c00u;          // rounds past 65504
    if (a < 0x38800000u) {                                 // binary16 subnormal range
        // a = 1.m * 2^(E-127); the subnormal mantissa is value * 2^24.
        const int E = (int)(a >> 23);
        if (E < 102) return sign;                          // below half of 2^-24
        const uint32_t m = (a & 0x7fffffu) | 0x800000u;    // 24-bit significand
        const int shift = 126 - E;                         // value*2^24 = m >> shift
        const uint32_t q = m >> shift;
        const uint32_t rem = m & ((1u << shift) - 1u);
        const uint32_t half = 1u << (shift - 1);
        const uint32_t r = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
        return sign | r;
    }
    const uint32_t h = ((((a >> 23) - 112u) << 10) | ((a & 0x7fffffu) >> 13));
    const uint32_t rem = a & 0x1fffu;
    return sign | (h + ((rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ? 1u : 0u));
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h)
{
    const uint32_t e = (h >> 10) & 0x1fu;
    const uint32_t m = h & 0x3ffu;
    float v;
    if (e == 0) v = (float)m * 5.9604644775390625e-8f;     // m * 2^-24, exact
    else if (e == 31) v = __uint_as_float(0x7f800000u | (m << 13));
    else v = __uint_as_float(((e + 112u) << 23) | (m << 13));
    return (h & 0x8000u) ? -v : v;
}

// First data error of a call: only a zero status is replaced.  The pointer
// and the code pass through an empty asm so that the atomic's operands are
// formed here, on this rare path, and not held (or spilled) for the whole
// kernel.  report() then uses the pointer as a global-memory pointer, so the
// atomic is a global one; report_generic() leaves it generic (a flat atomic,
// which the compiler also counts as a pending LDS access).  The atomic only
// runs on errors, but the choice changes the code generated around it: the
// IQ1 kernels measured 3 % faster on IQ1_M with the generic form, the IQ2_XS
// kernel 1.5 % faster with the global one.
__device__ __forceinline__ void report(int32_t* status, int code)
{
    uint64_t p = reinterpret_cast<uint64_t>(status);
    __asm__ volatile("" : "+s"(p), "+v"(code));
    typedef __attribute__((address_space(1))) int32_t global_i32;
    int32_t expected = 0;
    __atomic_compare_exchange_n(reinterpret_cast<global_i32*>(p), &expected, code, false,
                                __ATOMIC_RELAXED, __ATOMIC_RELAXED);
}

__device__ __forceinline__ void report_generic(int32_t* status, int code)
{
    __asm__ volatile("" : "+s"(status), "+v"(code));
    atomicCAS(status, 0, code);
}

__device__ __forceinline__ bool finite_f32(float v)
{
    return (__float_as_uint(v) & 0x7f800000u) != 0x7f800000u;
}

// bf16 operands of the matrix cores: the exact three-way split of an fp32
// value into bf16 parts, so that products with bf16-exact values are exact.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Part p (0, 1, 2) of the exact three-way bf16 split of v: v = hi + mid + lo,
// each part the leading 8 significant bits of what the earlier parts leave
// (truncation: hi keeps v's top 8 bits, v - hi is exact with at most 16
// significant bits, mid keeps its top 8, and the last 8 fit lo exactly).
// Half the instructions of a split by rounding to nearest, and the same sum.
__device__ __forceinline__ uint32_t split_part(float v, int p)
{
    const uint32_t u0 = __float_as_uint(v);
    const float r1 = v - __uint_as_float(u0 & 0xffff0000u);
    const uint32_t u1 = __float_as_uint(r1);
    const float r2 = r1 - __uint_as_float(u1 & 0xffff0000u);
    const uint32_t u2 = __float_as_uint(r2);
    return (p == 0 ? u0 : (p == 1 ? u1 : u2)) >> 16;
}

__device__ __forceinline__ v8bf as_v8bf(uint4 u)
{
    return __builtin_bit_cast(v8bf, u);
}

// 32 x 32 matrix tiles (v_mfma_f32_32x32x16_bf16): lane l supplies row and
// column l%32 of its operands with K elements 8*(l/32) .. +7, and holds rows
// 8*(v/4) + 4*(l/32) + v%4 of column l%32 of the result in v = 0..15.
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f mfma32(v8bf a, v8bf b, v16f c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Exchange with the lane 1 or 2 away inside a quad (DPP quad_perm): no
// address register, unlike a shuffle.
template <int kCtrl>
__device__ __forceinline__ float quad_xchg(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                                                 0xf, 0xf, false));
}
template <int kCtrl>
__device__ __forceinline__ int quad_xchg(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xf, 0xf, false);
}
template <int kCtrl>
__device__ __forceinline__ double quad_xchg(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)quad_xchg<kCtrl>((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)quad_xchg<kCtrl>((int)(uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
constexpr int kQuadXor1 = 0xb1, kQuadXor2 = 0x4e;

// One 256-value block of the weight in its storage type (iq_dtype_t), read as
// fp32: bf16 and fp16 convert exactly, fp64 rounds to nearest even.  quad(q)
// reads values 4q..4q+3, group(g, v) values 8g..8g+7, one(i) value i (the
// block start is 16-byte aligned in every type).
template <int kDT>
struct WeightBlock;

template <>
struct WeightBlock<IQ_DTYPE_F32> {
    const float* p;
    __device__ __forceinline__ WeightBlock(const void* base, int64_t blk)
        : p(static_cast<const float*>(base) + blk * kBlockElems) {}
    __device__ __forceinline__ float one(int i) const { return p[i]; }
    __device__ __forceinline__ float4 quad(int q) const
    {
        return reinterpret_cast<const float4*>(p)[q];
    }
    __device__ __forceinline__ void group(int g, float (&v)[8]) const
    {
        const float4* xp = reinterpret_cast<const float4*>(p + g * 8);
        const float4 a = xp[0], b = xp[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

template <>
struct WeightBlock<IQ_DTYPE_BF16> {
    const uint16_t* p;
    __device__ __forceinline__ WeightBlock(const void* base, int64_t blk)
        : p(static_cast<const uint16_t*>(base) + blk * kBlockElems) {}
    __device__ __forceinline__ static float lo(uint32_t u) { return __uint_as_float(u << 16); }
    __device__ __forceinline__ static float hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
    __device__ __forceinline__ float one(int i) const { return lo(p[i]); }
    __device__ __forceinline__ float4 quad(int q) const
    {
        const uint2 u = reinterpret_cast<const uint2*>(p)[q];
        return make_float4(lo(u.x), hi(u.x), lo(u.y), hi(u.y));
    }
    __device__ __forceinline__ void group(int g, float (&v)[8]) const
    {
        const uint4 u = reinterpret_cast<const uint4*>(p)[g];
        v[0] = lo(u.x); v[1] = hi(u.x); v[2] = lo(u.y); v[3] = hi(u.y);
        v[4] = lo(u.z); v[5] = hi(u.z); v[6] = lo(u.w); v[7] = hi(u.w);
    }
};

template <>
struct WeightBlock<IQ_DTYPE_F16> {
    const uint16_t* p;
    __device__ __forceinline__ WeightBlock(const void* base, int64_t blk)
        : p(static_cast<const uint16_t*>(base) + blk * kBlockElems) {}
    __device__ __forceinline__ static float cv(uint32_t h)
    {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
    }
    __device__ __forceinline__ float one(int i) const { return cv(p[i]); }
    __device__ __forceinline__ float4 quad(int q) const
    {
        const uint2 u = reinterpret_cast<const uint2*>(p)[q];
        return make_float4(cv(u.x), cv(u.x >> 16), cv(u.y), cv(u.y >> 16));
    }
    __device__ __forceinline__ void group(int g, float (&v)[8]) const
    {
        const uint4 u = reinterpret_cast<const uint4*>(p)[g];
        v[0] = cv(u.x); v[1] = cv(u.x >> 16); v[2] = cv(u.y); v[3] = cv(u.y >> 16);
        v[4] = cv(u.z); v[5] = cv(u.z >> 16); v[6] = cv(u.w); v[7] = cv(u.w >> 16);
    }
};

template <>
struct WeightBlock<IQ_DTYPE_F64> {
    const double* p;
    __device__ __forceinline__ WeightBlock(const void* base, int64_t blk)
        : p(static_cast<const double*>(base) + blk * kBlockElems) {}
    __device__ __forceinline__ float one(int i) const { return (float)p[i]; }
    __device__ __forceinline__ float4 quad(int q) const
    {
        const double2* dp = reinterpret_cast<const double2*>(p) + 2 * q;
        const double2 a = dp[0], b = dp[1];
        return make_float4((float)a.x, (float)a.y, (float)b.x, (float)b.y);
    }
    __device__ __forceinline__ void group(int g, float (&v)[8]) const
    {
        const float4 a = quad(2 * g), b = quad(2 * g + 1);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

}  // namespace iqk
