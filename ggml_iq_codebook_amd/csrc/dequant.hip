// dequant.hip -- decode of IQ1_S / IQ2_XS payloads to fp32 on gfx950.
//
// Decode rule (NVIDIA Model-Optimizer, "Add IQ tests and release notes" #2450,
// code review, worked example): IQ1_S value = d*(2k+1)*(q + delta) with
// delta = -1/8 when bit 15 of the sub-block's qh word is set, entry index =
// low byte | 3 high bits from qh; IQ2_XS value = d*(2k+1)*sign*q, the group's
// 8th sign implied by even parity of its 7-bit mask.  Every product is exact in
// fp32 (d has 11 significant bits, 2k+1 at most 5, q + delta at most 4).
//
// HBM-bound streaming kernel: one lane per 8-value group, two float4 stores
// per lane (coalesced 32-byte runs); the payload bytes of a block are read by
// 32 consecutive lanes and the grid (<= 64 KiB) stays in L2/L1.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace iqk {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void dequant_iq1s_kernel(const uint8_t* __restrict__ packed,
                                                                const float* __restrict__ grid, int n,
                                                                float* __restrict__ out,
                                                                int32_t* status, int64_t ngroups)
{
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= ngroups) return;
    const int64_t blk = gid >> 5;
    const int g = (int)(gid & 31);
    const int sub = g >> 2, l = g & 3;
    const uint8_t* b = packed + blk * 50;
    const uint32_t dh = (uint32_t)b[0] | ((uint32_t)b[1] << 8);
    const uint32_t qh = (uint32_t)b[34 + 2 * sub] | ((uint32_t)b[35 + 2 * sub] << 8);
    const int e = (int)b[2 + 4 * sub + l] | (int)(((qh >> (3 * l)) & 7u) << 8);
    const int k = (int)((qh >> 12) & 7u);
    const float delta = (qh >> 15) ? -0.125f : 0.125f;
    const float s = f16_bits_to_f32(dh) * (float)(2 * k + 1);
    float v[8];
    if (e < n) {
        const float4* q4 = reinterpret_cast<const float4*>(grid + 8 * e);
        const float4 q0 = q4[0], q1 = q4[1];
        v[0] = s * (q0.x + delta); v[1] = s * (q0.y + delta);
        v[2] = s * (q0.z + delta); v[3] = s * (q0.w + delta);
        v[4] = s * (q1.x + delta); v[5] = s * (q1.y + delta);
        v[6] = s * (q1.z + delta); v[7] = s * (q1.w + delta);
    } else {
        report(status, IQ_ERR_CODE);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
    float4* o = reinterpret_cast<float4*>(out + gid * 8);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

__global__ __launch_bounds__(kThreads) void dequant_iq2xs_kernel(const uint8_t* __restrict__ packed,
                                                                 const float* __restrict__ grid, int n,
                                                                 float* __restrict__ out,
                                                                 int32_t* status, int64_t ngroups)
{
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= ngroups) return;
    const int64_t blk = gid >> 5;
    const int g = (int)(gid & 31);
    const int m = g >> 1;
    const uint8_t* b = packed + blk * 74;
    const uint32_t dh = (uint32_t)b[0] | ((uint32_t)b[1] << 8);
    const uint32_t code = (uint32_t)b[2 + 2 * g] | ((uint32_t)b[3 + 2 * g] << 8);
    const int e = (int)(code & 0x1ffu);
    const uint32_t mask = code >> 9;
    const uint32_t sb = b[66 + (m >> 1)];
    const int k = (int)((m & 1) ? (sb >> 4) : (sb & 15u));
    const float s = f16_bits_to_f32(dh) * (float)(2 * k + 1);
    const uint32_t signs = mask | ((__popc(mask) & 1u) << 7);
    float v[8];
    if (e < n) {
        const float4* q4 = reinterpret_cast<const float4*>(grid + 8 * e);
        const float4 q0 = q4[0], q1 = q4[1];
        const float q[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (((signs >> j) & 1u) ? -s : s) * q[j];
    } else {
        report(status, IQ_ERR_CODE);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
    float4* o = reinterpret_cast<float4*>(out + gid * 8);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// IQ1_M (#2525 IQ1_M codec body): d reassembled from the top nibbles of the
// four scale words; the 3-bit local scale of the group's scale group; the
// group's nibble gives the 3 high index bits and the shift.
__global__ __launch_bounds__(kThreads) void dequant_iq1m_kernel(const uint8_t* __restrict__ packed,
                                                                const float* __restrict__ grid, int n,
                                                                float* __restrict__ out,
                                                                int32_t* status, int64_t ngroups)
{
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= ngroups) return;
    const int64_t blk = gid >> 5;
    const int g = (int)(gid & 31);
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
    float v[8];
    if (e < n) {
        const float4* q4 = reinterpret_cast<const float4*>(grid + 8 * e);
        const float4 q0 = q4[0], q1 = q4[1];
        v[0] = s * (q0.x + delta); v[1] = s * (q0.y + delta);
        v[2] = s * (q0.z + delta); v[3] = s * (q0.w + delta);
        v[4] = s * (q1.x + delta); v[5] = s * (q1.y + delta);
        v[6] = s * (q1.z + delta); v[7] = s * (q1.w + delta);
    } else {
        report(status, IQ_ERR_CODE);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
    float4* o = reinterpret_cast<float4*>(out + gid * 8);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

}  // namespace

hipError_t launch_dequant(int fmt, const uint8_t* packed, const float* grid, int grid_size,
                          float* out, int32_t* status, const BlockGeom& g, hipStream_t stream)
{
    const int64_t ngroups = g.nblocks * 32;
    const int64_t wgs = (ngroups + kThreads - 1) / kThreads;
    if (fmt == IQ_FMT_IQ1_S)
        hipLaunchKernelGGL(dequant_iq1s_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                           packed, grid, grid_size, out, status, ngroups);
    else if (fmt == IQ_FMT_IQ1_M)
        hipLaunchKernelGGL(dequant_iq1m_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                           packed, grid, grid_size, out, status, ngroups);
    else
        hipLaunchKernelGGL(dequant_iq2xs_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                           packed, grid, grid_size, out, status, ngroups);
    return hipGetLastError();
}

}  // namespace iqk
