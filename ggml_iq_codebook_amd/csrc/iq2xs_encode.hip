// iq2xs_encode.hip -- importance-weighted codebook search for IQ2_XS on
// gfx950, with two epilogues: the packed payload, and the top-C candidates
// that feed the local-Hessian choice search.
//
// The format (NVIDIA Model-Optimizer, "Add IQ tests and release notes" #2450,
// code review; "Register each GGML IQ format once" #2525, IQ2_S commit body,
// "What's distinctive about it"): a 74-byte block holds an fp16 scale d, 32
// 16-bit codes (9-bit grid index + 7-bit sign mask; the 8th sign of a group is
// implied by even parity, so the weakest element's sign is flipped when the
// input has an odd number of negatives) and 16 four-bit local scales, one per
// 16 values.  Each group of 8 is s*sign*q with q from a 512-entry magnitude
// grid and s = d*(2k+1), k = 0..15, shared by the 2 groups of a scale group;
// the codes minimise sum w*(x - s*sign*q)^2 with the lowest index winning.
// For the candidates, the 16 local scales of every scale group are ordered by
// their (cost, k) and the first top_c are emitted with their codes and error
// vectors xhat - x ("[2/4] Encode every GGML IQ choice in one pass" #3159).
//
// Kernel layout: one lane = one group, a wave = two blocks, a 512-thread
// workgroup = 16 blocks.  The grid and its squares are staged in LDS (32 KiB).
// Per (group, entry): P = sum (w*sign*x)*q and N = sum w*q^2, 16 keys
// s_k*N - 2P (one FMA each), value-only minima with chunked index recovery as
// in the IQ1_S kernel; the two lanes of a scale group add their minima with an
// xor-shuffle.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace iqk {
namespace {

constexpr int kBlocksPerWave = 2;
constexpr int kWavesPerWG = 8;
constexpr int kBlocksPerWG = kBlocksPerWave * kWavesPerWG;   // 16
constexpr int kThreads = kWave * kWavesPerWG;                 // 512
constexpr int kChunk = 32;
constexpr int kMaxGrid = 512;
constexpr int kBlockBytes = 74;

struct Iq2xsArgs {
    const float* w;
    const float* imp;
    const float* grid;
    const uint16_t* scales;
    const int32_t* choices;
    uint8_t* out;            // encode: packed payload
    float* cand_err;         // candidates
    int32_t* cand_choice;
    uint16_t* cand_codes;
    int32_t* status;
    BlockGeom g;
    int grid_size;
    int top_c;
};

struct EntryTerms {
    float pn;   // -2 * sum (w*sign*x) * q
    float n;    // sum w * q^2
};

// Terms of one grid entry; shared by the sweep and the rescan so both give
// bit-identical keys.  sg holds, per entry, q[0..7] then q^2[0..7].
__device__ __forceinline__ EntryTerms entry_terms(const float4* __restrict__ sg, int e,
                                                  const float (&wxs)[8], const float (&w)[8])
{
    const float4 a0 = sg[4 * e], a1 = sg[4 * e + 1], b0 = sg[4 * e + 2], b1 = sg[4 * e + 3];
    const float q[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float q2[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    float P = wxs[0] * q[0];
    float N = w[0] * q2[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
        P = __builtin_fmaf(wxs[j], q[j], P);
        N = __builtin_fmaf(w[j], q2[j], N);
    }
    EntryTerms t;
    t.pn = -2.0f * P;
    t.n = N;
    return t;
}

// Lowest entry index of choice k whose key equals the sweep's minimum: rescan
// the chunk that last lowered that minimum with the sweep's own arithmetic.
__device__ __forceinline__ int rescan(const float4* __restrict__ sg, int k, const float (&best)[16],
                                      const int (&chunk_of)[16], const float (&s)[16],
                                      const float (&wxs)[8], const float (&w)[8], int n)
{
    float target = best[0];
    int tchunk = chunk_of[0];
    float sk = s[0];
#pragma unroll
    for (int c = 1; c < 16; ++c)
        if (k == c) { target = best[c]; tchunk = chunk_of[c]; sk = s[c]; }
    int found = -1;
    const int e0 = tchunk * kChunk;
    for (int i = 0; i < kChunk; ++i) {
        const EntryTerms t = entry_terms(sg, e0 + i, wxs, w);
        const float key = __builtin_fmaf(sk, t.n, t.pn);
        if (found < 0 && key == target) found = e0 + i;
    }
    return found < 0 ? 0 : (found < n ? found : n - 1);
}

template <bool kCandidates>
__global__ __launch_bounds__(kThreads) void iq2xs_kernel(Iq2xsArgs a)
{
    __shared__ float4 sgrid[kMaxGrid * 4];
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
    if (!kCandidates)
        for (int i = tid; i < kBlocksPerWG * kBlockBytes / 2; i += kThreads) sout16[i] = 0;
    __syncthreads();
    {
        const float4* gsrc = reinterpret_cast<const float4*>(a.grid);
        int bad = 0;
        for (int i = tid; i < npad * 2; i += kThreads) {
            const int e = i >> 1;
            const int src = e < n ? e : n - 1;
            const float4 v = gsrc[2 * src + (i & 1)];
            bad |= !(v.x >= 0.0f && v.y >= 0.0f && v.z >= 0.0f && v.w >= 0.0f);
            bad |= !(finite_f32(v.x) && finite_f32(v.y) && finite_f32(v.z) && finite_f32(v.w));
            sgrid[4 * e + (i & 1)] = v;
            sgrid[4 * e + 2 + (i & 1)] = make_float4(v.x * v.x, v.y * v.y, v.z * v.z, v.w * v.w);
        }
        if (bad) sgrid_bad = 1;
    }
    __syncthreads();
    const bool grid_bad = sgrid_bad != 0;
    if (grid_bad && tid == 0) report(a.status, IQ_ERR_GRID);

    const int slot = wave * kBlocksPerWave + (lane >> 5);
    const int64_t blk = (int64_t)blockIdx.x * kBlocksPerWG + slot;
    const bool valid = blk < a.g.nblocks;
    const int g = lane & 31;          // group in block
    const int m = g >> 1;             // scale group
    const int h = g & 1;              // group in scale group

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

#pragma unroll
    for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));

    uint32_t dh;
    if (!kCandidates && a.scales) {
        dh = valid ? (uint32_t)a.scales[blk] : 0u;
    } else {
        const float t = amax / 155.0f;
        const float u = t * 0.61f;
        dh = f32_to_f16_bits(u);
    }
    const bool scale_bad = ((dh & 0x7c00u) == 0x7c00u) || ((dh & 0x8000u) && (dh & 0x7fffu));
    dh &= 0x7fffu;
    if (scale_bad && valid && g == 0 && bad_half == 0) report(a.status, IQ_ERR_SCALE_RANGE);
    const float d = scale_bad ? 0.0f : f16_bits_to_f32(dh);

    int forced = -1;
    if (!kCandidates && a.choices && valid) {
        forced = a.choices[blk * 16 + m];
        if (forced < 0 || forced > 15) {
            if (h == 0) report(a.status, IQ_ERR_ARG);
            forced = -2;
        }
    }
    const uint64_t badc_lanes = __ballot(forced == -2);
    const uint32_t badc_half = (lane >> 5) ? (uint32_t)(badc_lanes >> 32) : (uint32_t)badc_lanes;
    const bool bad_block = !valid || grid_bad || bad_half != 0 || scale_bad || badc_half != 0;
    const bool zero_scale = dh == 0u;

    // Signs: input signs, the weakest element (smallest (w*x)*x, lowest index)
    // flipped when the count of negatives is odd.
    float wx[8];
    int negmask = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        wx[j] = w[j] * x[j];
        if (x[j] < 0.0f) negmask |= 1 << j;
    }
    if (__popc(negmask) & 1) {
        int jw = 0;
        float wk = wx[0] * x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) {
            const float v = wx[j] * x[j];
            if (v < wk) { wk = v; jw = j; }
        }
        negmask ^= 1 << jw;
    }
    const int mask7 = negmask & 0x7f;
    float wxs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) wxs[j] = ((negmask >> j) & 1) ? -wx[j] : wx[j];

    float s[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) s[k] = d * (float)(2 * k + 1);

    float best[16], snap[16];
    int chunk_of[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) { best[k] = __builtin_inff(); snap[k] = best[k]; chunk_of[k] = 0; }

    for (int ch = 0; ch < nchunks; ++ch) {
        const int e0 = ch * kChunk;
#pragma unroll 2
        for (int e = e0; e < e0 + kChunk; e += 2) {
            const EntryTerms t0 = entry_terms(sgrid, e, wxs, w);
            const EntryTerms t1 = entry_terms(sgrid, e + 1, wxs, w);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const float k0 = __builtin_fmaf(s[k], t0.n, t0.pn);
                const float k1 = __builtin_fmaf(s[k], t1.n, t1.pn);
                best[k] = fminf(fminf(best[k], k0), k1);
            }
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            chunk_of[k] = best[k] < snap[k] ? ch : chunk_of[k];
            snap[k] = best[k];
        }
    }

    // Scale-group cost of every local scale (same float sum in both lanes).
    float cost[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        float v = best[k];
        v += __shfl_xor(v, 1);
        cost[k] = s[k] * v;
    }

    if (!kCandidates) {
        int kstar = 0;
        float cb = cost[0];
#pragma unroll
        for (int k = 1; k < 16; ++k)
            if (cost[k] < cb) { cb = cost[k]; kstar = k; }
        if (forced >= 0) kstar = forced;
        const int idx = rescan(sgrid, kstar, best, chunk_of, s, wxs, w, n);
        // byte 66 + m/2 holds scale group m in its low (even m) or high (odd m) nibble
        const int kodd = __shfl_xor(kstar, 2);
        if (!bad_block && !zero_scale) {
            uint8_t* ob = sout + slot * kBlockBytes;
            const uint32_t code = (uint32_t)idx | ((uint32_t)mask7 << 9);
            ob[2 + 2 * g] = (uint8_t)(code & 0xff);
            ob[3 + 2 * g] = (uint8_t)(code >> 8);
            if ((g & 3) == 0) ob[66 + (m >> 1)] = (uint8_t)(kstar | (kodd << 4));
            if (g == 0) {
                ob[0] = (uint8_t)(dh & 0xff);
                ob[1] = (uint8_t)(dh >> 8);
            }
        }
        __syncthreads();
        const int64_t first = (int64_t)blockIdx.x * kBlocksPerWG;
        const int64_t left = a.g.nblocks - first;
        const int nb = left < kBlocksPerWG ? (int)left : kBlocksPerWG;
        uint16_t* o16 = reinterpret_cast<uint16_t*>(a.out + first * kBlockBytes);
        for (int i = tid; i < nb * (kBlockBytes / 2); i += kThreads) o16[i] = sout16[i];
    } else {
        // Top-C local scales by (cost, k); a zero scale makes every choice decode
        // to zero with entry 0 and no signs, so the order is k = 0, 1, ...
        const int C = a.top_c;
        int used = 0;
        for (int r = 0; r < C; ++r) {
            int kr = -1;
            float cr = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const bool free_k = !((used >> k) & 1);
                const bool better = zero_scale ? (kr < 0) : (kr < 0 || cost[k] < cr);
                if (free_k && better) { kr = k; cr = cost[k]; }
            }
            used |= 1 << kr;
            int idx = rescan(sgrid, kr, best, chunk_of, s, wxs, w, n);
            int msk = mask7;
            float sg[8];
            if (zero_scale) {
                idx = 0;
                msk = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) sg[j] = 1.0f;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) sg[j] = ((negmask >> j) & 1) ? -1.0f : 1.0f;
            }
            if (valid) {
                const int64_t base = (blk * 16 + m) * C + r;     // [block][m][r]
                float ev[8];
                if (bad_block) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) ev[j] = 0.0f;
                } else {
                    float sk = s[0];
#pragma unroll
                    for (int c = 1; c < 16; ++c)
                        if (kr == c) sk = s[c];
                    const float4 q0 = sgrid[4 * idx], q1 = sgrid[4 * idx + 1];
                    const float q[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
                    for (int j = 0; j < 8; ++j) ev[j] = (sk * sg[j]) * q[j] - x[j];
                }
                float4* ep = reinterpret_cast<float4*>(a.cand_err + base * 16 + h * 8);
                ep[0] = make_float4(ev[0], ev[1], ev[2], ev[3]);
                ep[1] = make_float4(ev[4], ev[5], ev[6], ev[7]);
                if (h == 0) a.cand_choice[base] = kr;
                if (a.cand_codes)
                    a.cand_codes[base * 2 + h] =
                        bad_block ? (uint16_t)0 : (uint16_t)(idx | (msk << 9));
            }
        }
    }
}

}  // namespace

hipError_t launch_iq2xs_encode(const float* w, const float* imp, const float* grid, int grid_size,
                               const uint16_t* scales, const int32_t* choices, uint8_t* out,
                               int32_t* status, const BlockGeom& g, hipStream_t stream)
{
    Iq2xsArgs a{w, imp, grid, scales, choices, out, nullptr, nullptr, nullptr, status, g,
                grid_size, 0};
    const int64_t wgs = (g.nblocks + kBlocksPerWG - 1) / kBlocksPerWG;
    hipLaunchKernelGGL(iq2xs_kernel<false>, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_iq2xs_candidates(const float* w, const float* imp, const float* grid,
                                   int grid_size, int top_c, float* cand_err, int32_t* cand_choice,
                                   uint16_t* cand_codes, int32_t* status, const BlockGeom& g,
                                   hipStream_t stream)
{
    Iq2xsArgs a{w, imp, grid, nullptr, nullptr, nullptr, cand_err, cand_choice, cand_codes,
                status, g, grid_size, top_c};
    const int64_t wgs = (g.nblocks + kBlocksPerWG - 1) / kBlocksPerWG;
    hipLaunchKernelGGL(iq2xs_kernel<true>, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace iqk
