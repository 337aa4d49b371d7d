// iq1s_encode.hip -- importance-weighted exhaustive codebook search for IQ1_S
// on gfx950.
//
// The format (NVIDIA Model-Optimizer, "Add IQ tests and release notes" #2450,
// code review; "Weight the IQ1 encoders by the square root of GPTQ's Hessian
// diagonal" #2723): a 256-value block has an fp16 scale d predicted as
// (amax/16.875)*0.61; each group of 8 values is s*(q + delta) with q one of up
// to 2048 ternary grid entries; the 4 groups of a 32-value sub-block share the
// local scale s = d*(2k+1), k = 0..7, and delta = +-1/8.  The codes minimise
// sum w*(x - s*(q+delta))^2, lowest index winning ties.
//
// Kernel layout (MI355X-first, not the CUDA prior art's one-block-per-row):
//  * one lane = one 8-value group, a 64-lane wave = two 256-value blocks,
//    a 512-thread workgroup = 16 blocks; weights and importance are read once,
//    two float4 per lane, fully coalesced;
//  * the grid (64 KiB for 2048 entries) is staged once per workgroup in LDS
//    (160 KiB per CU on CDNA4) and read as wave-uniform broadcasts;
//  * per (group, entry) the three weighted dot products A = sum wx*q,
//    M = sum w*q, N = sum w*|q| give U(delta) = sum w*(q+delta)^2 and
//    V(delta) = sum wx*(q+delta); the key of local scale s_k is
//    s_k*U - 2V (the error divided by s_k, minus a constant), one FMA each;
//  * the 16 per-choice minima are tracked by value only (v_min3 over two
//    entries); the 32-entry chunk that last lowered each minimum is recorded,
//    and after the sub-block's choice is known each lane rescans only its
//    winning chunk with the identical instruction sequence to recover the
//    lowest entry index whose key equals the minimum;
//  * the 4 lanes of a sub-block sum their minima with xor-shuffles (identical
//    in every lane), pick the lowest-cost choice, and the block is packed in
//    LDS and stored as 16-bit words.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace iqk {
namespace {

constexpr int kBlocksPerWave = 2;
constexpr int kWavesPerWG = 8;
constexpr int kBlocksPerWG = kBlocksPerWave * kWavesPerWG;   // 16
constexpr int kThreads = kWave * kWavesPerWG;                 // 512
constexpr int kChunk = 32;                                    // entries per tracking chunk
constexpr int kMaxGrid = 2048;
constexpr int kBlockBytes = 50;

struct Iq1sArgs {
    const float* w;
    const float* imp;
    const float* grid;
    const uint16_t* scales;
    const int32_t* choices;
    uint8_t* out;
    int32_t* status;
    BlockGeom g;
    int grid_size;
};

struct GroupTerms {
    float up, um;     // U(+1/8), U(-1/8)
    float vnp, vnm;   // -2*V(+1/8), -2*V(-1/8)
};

// Terms of one grid entry for one group.  Used by the sweep and the rescan, so
// both produce bit-identical keys.
__device__ __forceinline__ GroupTerms entry_terms(const float4* __restrict__ sg, int e,
                                                  const float (&wx)[8], const float (&w)[8],
                                                  float w64, float b4)
{
    const float4 q0 = sg[2 * e];
    const float4 q1 = sg[2 * e + 1];
    const float q[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    float A = wx[0] * q[0];
    float M = w[0] * q[0];
    float N = w[0] * fabsf(q[0]);
#pragma unroll
    for (int j = 1; j < 8; ++j) {
        A = __builtin_fmaf(wx[j], q[j], A);
        M = __builtin_fmaf(w[j], q[j], M);
        N = __builtin_fmaf(w[j], fabsf(q[j]), N);
    }
    // U(delta) = N + 2*delta*M + delta^2*W,  V(delta) = A + delta*B
    const float T = N + w64;
    GroupTerms t;
    t.up = __builtin_fmaf(M, 0.25f, T);
    t.um = __builtin_fmaf(M, -0.25f, T);
    t.vnp = __builtin_fmaf(A, -2.0f, -b4);
    t.vnm = __builtin_fmaf(A, -2.0f, b4);
    return t;
}

__global__ __launch_bounds__(kThreads) void iq1s_encode_kernel(Iq1sArgs a)
{
    __shared__ float4 sgrid[kMaxGrid * 2];
    __shared__ uint16_t sout16[kBlocksPerWG * kBlockBytes / 2];
    __shared__ int sgrid_bad;
    uint8_t* sout = reinterpret_cast<uint8_t*>(sout16);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int n = a.grid_size;
    const int nchunks = (n + kChunk - 1) / kChunk;
    const int npad = nchunks * kChunk;

    if (tid == 0) sgrid_bad = 0;
    for (int i = tid; i < kBlocksPerWG * kBlockBytes / 2; i += kThreads) sout16[i] = 0;
    __syncthreads();
    // Stage the grid; entries past the end repeat the last one (their keys can
    // never beat the real entry, which comes first).
    {
        const float4* gsrc = reinterpret_cast<const float4*>(a.grid);
        int bad = 0;
        for (int i = tid; i < npad * 2; i += kThreads) {
            const int e = i >> 1;
            const int src = e < n ? e : n - 1;
            const float4 v = gsrc[2 * src + (i & 1)];
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bad |= !(vv[j] == 0.0f || vv[j] == 1.0f || vv[j] == -1.0f);
            sgrid[i] = v;
        }
        if (bad) sgrid_bad = 1;
    }
    __syncthreads();
    const bool grid_bad = sgrid_bad != 0;
    if (grid_bad && tid == 0) report(a.status, IQ_ERR_GRID);

    const int slot = wave * kBlocksPerWave + (lane >> 5);     // block slot in this WG
    const int64_t blk = (int64_t)blockIdx.x * kBlocksPerWG + slot;
    const bool valid = blk < a.g.nblocks;
    const int g = lane & 31;                                   // group in block
    const int sub = g >> 2;                                    // sub-block
    const int lq = g & 3;                                      // group in sub-block

    float x[8], w[8];
    if (valid) {
        const float4* xp = reinterpret_cast<const float4*>(a.w + blk * kBlockElems + g * 8);
        const float4 x0 = xp[0], x1 = xp[1];
        x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
        x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
        if (a.imp) {
            const int64_t bt = blk / a.g.blocks_per_batch;
            const int64_t cb = blk % a.g.blocks_per_row;
            const float4* wp = reinterpret_cast<const float4*>(a.imp + bt * a.g.cols + cb * kBlockElems + g * 8);
            const float4 w0 = wp[0], w1 = wp[1];
            w[0] = w0.x; w[1] = w0.y; w[2] = w0.z; w[3] = w0.w;
            w[4] = w1.x; w[5] = w1.y; w[6] = w1.z; w[7] = w1.w;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = 1.0f;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) { x[j] = 0.0f; w[j] = 1.0f; }
    }

    // Input checks: a non-finite weight or a negative / non-finite importance
    // value zeroes the whole block and is reported.
    int err = 0;
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (!finite_f32(x[j])) err = IQ_ERR_NONFINITE;
        amax = fmaxf(amax, fabsf(x[j]));
    }
    if (!err) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (!(w[j] >= 0.0f) || !finite_f32(w[j])) err = IQ_ERR_IMPORTANCE;
    }
    if (err && valid) report(a.status, err);
    const uint64_t bad_lanes = __ballot(err != 0);
    const uint32_t bad_half = (lane >> 5) ? (uint32_t)(bad_lanes >> 32) : (uint32_t)bad_lanes;

    // Block amax over the 32 lanes of this half-wave.
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));

    // Super-block scale: fp32 divide, fp32 multiply (no contraction), fp16 RNE.
    uint32_t dh;
    if (a.scales) {
        dh = valid ? (uint32_t)a.scales[blk] : 0u;
    } else {
        const float t = amax / 16.875f;
        const float u = t * 0.61f;
        dh = f32_to_f16_bits(u);
    }
    bool scale_bad = ((dh & 0x7c00u) == 0x7c00u) || ((dh & 0x8000u) && (dh & 0x7fffu));
    dh &= 0x7fffu;
    if (scale_bad && valid && g == 0 && bad_half == 0) report(a.status, IQ_ERR_SCALE_RANGE);
    const float d = scale_bad ? 0.0f : f16_bits_to_f32(dh);

    // Forced choice of this sub-block, if any.
    int forced = -1;
    if (a.choices && valid) {
        forced = a.choices[blk * 8 + sub];
        if (forced < 0 || forced > 15) {
            if (lq == 0) report(a.status, IQ_ERR_ARG);
            forced = -2;
        }
    }
    const uint64_t badc_lanes = __ballot(forced == -2);
    const uint32_t badc_half = (lane >> 5) ? (uint32_t)(badc_lanes >> 32) : (uint32_t)badc_lanes;

    const bool zero_block = !valid || grid_bad || bad_half != 0 || scale_bad || dh == 0u ||
                            badc_half != 0;

    // Per-group sums.
    float wx[8];
    float W = 0.0f, B = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        wx[j] = w[j] * x[j];
        W += w[j];
        B += wx[j];
    }
    const float w64 = W * 0.015625f;
    const float b4 = B * 0.25f;
    float s[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) s[k] = d * (float)(2 * k + 1);

    // Sweep: value-only minima of the 16 choices, chunk of the last improvement.
    float best[16], snap[16];
    int chunk_of[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) { best[c] = __builtin_inff(); snap[c] = best[c]; chunk_of[c] = 0; }

    for (int ch = 0; ch < nchunks; ++ch) {
        const int e0 = ch * kChunk;
#pragma unroll 2
        for (int e = e0; e < e0 + kChunk; e += 2) {
            const GroupTerms t0 = entry_terms(sgrid, e, wx, w, w64, b4);
            const GroupTerms t1 = entry_terms(sgrid, e + 1, wx, w, w64, b4);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float p0 = __builtin_fmaf(s[k], t0.up, t0.vnp);
                const float p1 = __builtin_fmaf(s[k], t1.up, t1.vnp);
                best[k] = fminf(fminf(best[k], p0), p1);
                const float m0 = __builtin_fmaf(s[k], t0.um, t0.vnm);
                const float m1 = __builtin_fmaf(s[k], t1.um, t1.vnm);
                best[8 + k] = fminf(fminf(best[8 + k], m0), m1);
            }
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            chunk_of[c] = best[c] < snap[c] ? ch : chunk_of[c];
            snap[c] = best[c];
        }
    }

    // Sub-block cost of each choice: s_k * (sum of the 4 groups' minima); the
    // xor-butterfly gives the same float sum in all 4 lanes.
    int cstar = 0;
    float cbest = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        float v = best[c];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        const float cost = s[c & 7] * v;
        if (c == 0 || cost < cbest) { cbest = cost; cstar = c; }
    }
    if (forced >= 0) cstar = forced;

    // Rescan the winning chunk of the chosen choice for the lowest entry index.
    float target = best[0];
    int tchunk = chunk_of[0];
#pragma unroll
    for (int c = 1; c < 16; ++c)
        if (cstar == c) { target = best[c]; tchunk = chunk_of[c]; }
    const int kstar = cstar & 7;
    const int dbit = cstar >> 3;
    float sk = s[0];
#pragma unroll
    for (int k = 1; k < 8; ++k)
        if (kstar == k) sk = s[k];
    int found = -1;
    {
        const int e0 = tchunk * kChunk;
        for (int i = 0; i < kChunk; ++i) {
            const GroupTerms t = entry_terms(sgrid, e0 + i, wx, w, w64, b4);
            const float key = dbit ? __builtin_fmaf(sk, t.um, t.vnm) : __builtin_fmaf(sk, t.up, t.vnp);
            if (found < 0 && key == target) found = e0 + i;
        }
    }
    int idx = found < 0 ? 0 : (found < n ? found : n - 1);

    // Pack: low byte per group, qh word per sub-block, d per block.
    int hi = ((idx >> 8) & 7) << (3 * lq);
    hi |= __shfl_xor(hi, 1);
    hi |= __shfl_xor(hi, 2);
    if (!zero_block) {
        uint8_t* ob = sout + slot * kBlockBytes;
        ob[2 + 4 * sub + lq] = (uint8_t)(idx & 0xff);
        if (lq == 0) {
            const uint32_t qh = (uint32_t)hi | ((uint32_t)kstar << 12) | ((uint32_t)dbit << 15);
            ob[34 + 2 * sub] = (uint8_t)(qh & 0xff);
            ob[35 + 2 * sub] = (uint8_t)(qh >> 8);
        }
        if (g == 0) {
            ob[0] = (uint8_t)(dh & 0xff);
            ob[1] = (uint8_t)(dh >> 8);
        }
    }
    __syncthreads();
    // Coalesced store of this workgroup's blocks as 16-bit words.
    const int64_t first = (int64_t)blockIdx.x * kBlocksPerWG;
    const int64_t left = a.g.nblocks - first;
    const int nb = left < kBlocksPerWG ? (int)left : kBlocksPerWG;
    uint16_t* o16 = reinterpret_cast<uint16_t*>(a.out + first * kBlockBytes);
    for (int i = tid; i < nb * (kBlockBytes / 2); i += kThreads) o16[i] = sout16[i];
}

}  // namespace

hipError_t launch_iq1s_encode(const float* w, const float* imp, const float* grid, int grid_size,
                              const uint16_t* scales, const int32_t* choices, uint8_t* out,
                              int32_t* status, const BlockGeom& g, hipStream_t stream)
{
    Iq1sArgs a{w, imp, grid, scales, choices, out, status, g, grid_size};
    const int64_t wgs = (g.nblocks + kBlocksPerWG - 1) / kBlocksPerWG;
    hipLaunchKernelGGL(iq1s_encode_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace iqk
