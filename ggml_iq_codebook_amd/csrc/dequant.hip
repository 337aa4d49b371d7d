// dequant.hip -- decode of IQ1_S / IQ2_XS payloads to fp32 on gfx950.
//
// Decode rule (NVIDIA Model-Optimizer, "Add IQ tests and release notes" #2450,
// code review, worked example): IQ1_S value = d*(2k+1)*(q + delta) with
// delta = -1/8 when bit 15 of the sub-block's qh word is set, entry index =
// low byte | 3 high bits from qh; IQ2_XS value = d*(2k+1)*sign*q, the group's
// 8th sign implied by even parity of its 7-bit mask.  Every product is exact in
// fp32 (d has 11 significant bits, 2k+1 at most 5, q + delta at most 4).
//
// HBM-bound streaming kernel: a wave per 256-value block, a lane per 4
// consecutive values (half a group), so every store instruction of a wave
// writes one contiguous KiB, with non-temporal stores.  The lane reads the few payload bytes its group
// needs (the 64 lanes of a block share one 50 to 74-byte record, served by the
// L1) and one float4 of its grid entry (the grid, at most 64 KiB, stays in
// L2/L1).
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace iqk {
namespace {

constexpr int kThreads = 256;

// The values are written once and not read again by this kernel: a
// non-temporal store (measured 9 % faster than a plain one on the 4096 x 4096
// decodes).
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_streaming(float* out, int64_t quad, float4 v)
{
    __builtin_nontemporal_store(f4v{v.x, v.y, v.z, v.w}, reinterpret_cast<f4v*>(out) + quad);
}

// Lane t of the launch covers values 4t..4t+3: block t/64, group (t%64)/2,
// half t%2 of the group.
__global__ __launch_bounds__(kThreads) void dequant_iq1s_kernel(const uint8_t* __restrict__ packed,
                                                                const float* __restrict__ grid, int n,
                                                                float* __restrict__ out,
                                                                int32_t* status, int64_t nquads)
{
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= nquads) return;
    const int64_t blk = t >> 6;
    const int g = (int)(t >> 1) & 31;
    const int h = (int)t & 1;
    const int sub = g >> 2, l = g & 3;
    const uint8_t* b = packed + blk * 50;
    const uint32_t dh = (uint32_t)b[0] | ((uint32_t)b[1] << 8);
    const uint32_t qh = (uint32_t)b[34 + 2 * sub] | ((uint32_t)b[35 + 2 * sub] << 8);
    const int e = (int)b[2 + 4 * sub + l] | (int)(((qh >> (3 * l)) & 7u) << 8);
    const int k = (int)((qh >> 12) & 7u);
    const float delta = (qh >> 15) ? -0.125f : 0.125f;
    const float s = f16_bits_to_f32(dh) * (float)(2 * k + 1);
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (e < n) {
        const float4 q = reinterpret_cast<const float4*>(grid + 8 * e)[h];
        v = make_float4(s * (q.x + delta), s * (q.y + delta), s * (q.z + delta), s * (q.w + delta));
    } else if (h == 0) {
        report(status, IQ_ERR_CODE);
    }
    store_streaming(out, t, v);
}

__global__ __launch_bounds__(kThreads) void dequant_iq2xs_kernel(const uint8_t* __restrict__ packed,
                                                                 const float* __restrict__ grid, int n,
                                                                 float* __restrict__ out,
                                                                 int32_t* status, int64_t nquads)
{
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= nquads) return;
    const int64_t blk = t >> 6;
    const int g = (int)(t >> 1) & 31;
    const int h = (int)t & 1;
    const int m = g >> 1;
    const uint8_t* b = packed + blk * 74;
    const uint32_t dh = (uint32_t)b[0] | ((uint32_t)b[1] << 8);
    const uint32_t code = (uint32_t)b[2 + 2 * g] | ((uint32_t)b[3 + 2 * g] << 8);
    const int e = (int)(code & 0x1ffu);
    const uint32_t mask = code >> 9;
    const uint32_t sb = b[66 + (m >> 1)];
    const int k = (int)((m & 1) ? (sb >> 4) : (sb & 15u));
    const float s = f16_bits_to_f32(dh) * (float)(2 * k + 1);
    // the 8 signs (the 8th from even parity of the 7-bit mask), this half's 4
    const uint32_t signs = (mask | ((__popc(mask) & 1u) << 7)) >> (4 * h);
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (e < n) {
        const float4 q = reinterpret_cast<const float4*>(grid + 8 * e)[h];
        v = make_float4(((signs & 1u) ? -s : s) * q.x, ((signs & 2u) ? -s : s) * q.y,
                        ((signs & 4u) ? -s : s) * q.z, ((signs & 8u) ? -s : s) * q.w);
    } else if (h == 0) {
        report(status, IQ_ERR_CODE);
    }
    store_streaming(out, t, v);
}

// IQ1_M (#2525 IQ1_M codec body): d's fp16 bits from the top nibbles of the
// four scale words; the 3-bit local scale of the group's scale group; the
// group's nibble gives the 3 high index bits and the shift.
__global__ __launch_bounds__(kThreads) void dequant_iq1m_kernel(const uint8_t* __restrict__ packed,
                                                                const float* __restrict__ grid, int n,
                                                                float* __restrict__ out,
                                                                int32_t* status, int64_t nquads)
{
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= nquads) return;
    const int64_t blk = t >> 6;
    const int g = (int)(t >> 1) & 31;
    const int h = (int)t & 1;
    const int m = g >> 1;
    const uint8_t* b = packed + blk * 56;
    uint32_t sc[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) sc[w] = (uint32_t)b[48 + 2 * w] | ((uint32_t)b[49 + 2 * w] << 8);
    // d's fp16 bits, nibble w (bits 4w..4w+3) in the top 4 bits of word w
    uint32_t dh = 0u;
#pragma unroll
    for (int w = 0; w < 4; ++w) dh |= (sc[w] >> 12) << (4 * w);
    const int k = (int)((sc[m >> 2] >> (3 * (m & 3))) & 7u);
    const uint32_t nib = ((uint32_t)b[32 + (g >> 1)] >> (4 * (g & 1))) & 0xfu;
    const int e = (int)b[g] | (int)((nib & 7u) << 8);
    const float delta = (nib & 8u) ? -0.125f : 0.125f;
    const float s = f16_bits_to_f32(dh) * (float)(2 * k + 1);
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (e < n) {
        const float4 q = reinterpret_cast<const float4*>(grid + 8 * e)[h];
        v = make_float4(s * (q.x + delta), s * (q.y + delta), s * (q.z + delta), s * (q.w + delta));
    } else if (h == 0) {
        report(status, IQ_ERR_CODE);
    }
    store_streaming(out, t, v);
}

}  // namespace

hipError_t launch_dequant(int fmt, const uint8_t* packed, const float* grid, int grid_size,
                          float* out, int32_t* status, const BlockGeom& g, hipStream_t stream)
{
    const int64_t nquads = g.nblocks * 64;
    const int64_t wgs = (nquads + kThreads - 1) / kThreads;
    if (fmt == IQ_FMT_IQ1_S)
        hipLaunchKernelGGL(dequant_iq1s_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                           packed, grid, grid_size, out, status, nquads);
    else if (fmt == IQ_FMT_IQ1_M)
        hipLaunchKernelGGL(dequant_iq1m_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                           packed, grid, grid_size, out, status, nquads);
    else
        hipLaunchKernelGGL(dequant_iq2xs_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                           packed, grid, grid_size, out, status, nquads);
    return hipGetLastError();
}

}  // namespace iqk
