// iq1s_encode.hip -- importance-weighted exhaustive codebook search for IQ1_S
// on gfx950, with the weighted dot products on the matrix cores.
//
// The format (NVIDIA Model-Optimizer, "Add IQ tests and release notes" #2450,
// code review; "Weight the IQ1 encoders by the square root of GPTQ's Hessian
// diagonal" #2723): a 256-value block has an fp16 scale d predicted as
// (amax/16.875)*0.61; each group of 8 values is s*(q + delta) with q one of up
// to 2048 ternary grid entries; the 4 groups of a 32-value sub-block share the
// local scale s = d*(2k+1), k = 0..7, and delta = +-1/8.  The codes minimise
// sum w*(x - s*(q+delta))^2, lowest index winning ties.
//
// For a group and a grid entry the error is, up to a constant,
//   s^2 * U(delta) - 2 s * V(delta),  U(delta) = sum w*(q+delta)^2,
//   V(delta) = sum wx*(q+delta).
// U(+1/8), U(-1/8), -2V(+1/8) and -2V(-1/8) for 16 grid entries x 16 groups
// are four small products [16 entries x 8] x [8 x 16 groups], run as
// v_mfma_f32_16x16x32_bf16: the entry side (q+delta)^2 and q is exact in bf16
// (values like 81/64 need 7 mantissa bits), the group side (w and -2*w*x) is
// split into three bf16 parts whose sum is exactly the fp32 value, so the
// products are exact and only the fp32 accumulation rounds; the constant
// -2*delta*sum(wx) of V enters as the accumulator input.  Everything is
// divided by the block scale d (the V side carries 1/d), so the key of local
// scale s_k = d*(2k+1) is (2k+1)*U - 2V/d: one FMA with a literal multiplier
// (v_fmamk_f32, two register operands, which pairs well with v_min3 in the
// dual-issue VALU); the choice cost of a sub-block is (2k+1) times the sum of
// its groups' minima (the common factor d^2 dropped).  The VALU keeps
// value-only minima (v_min3 over two entries).
//
// Layout: a wave owns 16 groups (half a block): matrix column j = lane%16 is
// group j; the lane's four accumulator rows are 4*(lane/16)+r of every
// 16-entry tile, so the four lanes of a column cover disjoint quarters of the
// grid.  A 1024-thread workgroup runs 16 waves = 8 blocks per pass and 2
// passes (16 blocks), with the grid staged once in LDS as bf16 ((q+1/8)^2,
// (q-1/8)^2 and q, 96 KiB; one workgroup per CU, 4 waves per SIMD).
// Index recovery: each lane records the 128-entry chunk that last lowered each
// of its 16 minima; once the sub-block's choice is fixed, the lane rescans its
// 32 entries of that chunk on the VALU (fp32 dot products) and takes the lowest
// entry of least key; the four lanes of a column then keep the one whose
// matrix-core minimum is least (lowest index on equal minima).
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace iqk {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWavesPerWG = 16;
constexpr int kThreads = kWave * kWavesPerWG;        // 1024
constexpr int kBlocksPerPass = kWavesPerWG / 2;      // two waves per block
constexpr int kPasses = 2;
constexpr int kBlocksPerWG = kBlocksPerPass * kPasses;   // 16
constexpr int kTile = 16;                            // grid entries per matrix tile
constexpr int kChunkTiles = 8;                       // tiles per tracking chunk
constexpr int kChunk = kTile * kChunkTiles;          // 128 entries
constexpr int kMaxGrid = 2048;
constexpr int kBlockBytes = 50;

struct Iq1sArgs {
    const float* w;
    const float* imp;
    const float* grid;
    const uint16_t* scales;
    const int32_t* choices;
    uint8_t* out;            // payload: [nblocks][50]; every choice: [16][nblocks][50]; may be
                             // NULL for the fake-quant output
    float* xhat;             // fake quant: decoded values [nblocks][256]
    float* cand_err;         // candidates: [nblocks][8][top_c][32]
    int32_t* cand_choice;    // [nblocks][8][top_c]
    uint16_t* cand_codes;    // NULL or [nblocks][8][top_c][4]
    int32_t* status;
    BlockGeom g;
    int grid_size;
    int top_c;
};

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Part p (0, 1, 2) of the exact three-way bf16 split of v: v = hi + mid + lo.
__device__ __forceinline__ uint32_t split_part(float v, int p)
{
    const uint32_t hi = bf16_bits(v);
    const float r1 = v - bf16_to_f32(hi);
    const uint32_t mid = bf16_bits(r1);
    const float r2 = r1 - bf16_to_f32(mid);
    return p == 0 ? hi : (p == 1 ? mid : bf16_bits(r2));
}

__device__ __forceinline__ v8bf as_v8bf(uint4 u)
{
    return __builtin_bit_cast(v8bf, u);
}

// The 8 values and importance weights of group g of a block (zeros and ones
// for a rejected block, so the sweep stays finite).
__device__ __forceinline__ void load_group(const float* xblk, const float* wblk, int g, bool zero,
                                           float (&x)[8], float (&w)[8])
{
    if (zero) {
#pragma unroll
        for (int j = 0; j < 8; ++j) { x[j] = 0.0f; w[j] = 1.0f; }
        return;
    }
    const float4* xp = reinterpret_cast<const float4*>(xblk + g * 8);
    const float4 x0 = xp[0], x1 = xp[1];
    x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
    x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
    if (wblk) {
        const float4* wp = reinterpret_cast<const float4*>(wblk + g * 8);
        const float4 w0 = wp[0], w1 = wp[1];
        w[0] = w0.x; w[1] = w0.y; w[2] = w0.z; w[3] = w0.w;
        w[4] = w1.x; w[5] = w1.y; w[6] = w1.z; w[7] = w1.w;
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = 1.0f;
    }
}

// VALU rescan for choice cs = k + 8*deltabit: the lowest of this lane's
// entries of chunk tchunk with the least key (2k+1)*U - 2V/d, recomputed in
// fp32 from the group's values and weights (read again from memory rather
// than held through the sweep).
__device__ __forceinline__ int rescan(const uint4* __restrict__ sq, int tchunk, int kb, int cs,
                                      const float* xblk, const float* wblk, int g, bool zero_block,
                                      float w64, float b4, float inv_d)
{
    float x[8], w[8];
    __asm__ volatile("" ::: "memory");
    load_group(xblk, wblk, g, zero_block, x, w);
    const float mk = (float)(2 * (cs & 7) + 1);
    const float dl = (cs >> 3) ? -0.25f : 0.25f;      // 2*delta
    const float bd = (cs >> 3) ? b4 : -b4;
    int idx = -1;
    float vbest = 0.0f;
    for (int tt = 0; tt < kChunkTiles; ++tt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = (tchunk * kChunkTiles + tt) * kTile + 4 * kb + r;
            const uint4 u = sq[e + tchunk];
            const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
            float A = 0.0f, M = 0.0f, N = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float q = bf16_to_f32((uu[j >> 1] >> (16 * (j & 1))) & 0xffffu);
                A = __builtin_fmaf(w[j] * x[j], q, A);
                M = __builtin_fmaf(w[j], q, M);
                N = __builtin_fmaf(w[j], fabsf(q), N);
            }
            const float U = __builtin_fmaf(M, dl, N + w64);
            const float key = __builtin_fmaf(U, mk, __builtin_fmaf(A, -2.0f, bd) * inv_d);
            if (idx < 0 || key < vbest) { vbest = key; idx = e; }
        }
    }
    return idx;
}

template <int kMode>
__global__ __launch_bounds__(kThreads) void iq1s_encode_kernel(Iq1sArgs a)
{
    // Payloads staged in LDS: one per block, or one per block and choice.
    constexpr int kPayloads = kMode == kModeEvery ? 16 : 1;
    // Entry e sits at e + e/kChunk: one spare slot per 128-entry chunk, so the
    // lanes of a rescan that read different chunks (512 words apart without
    // the slot, a multiple of the 64 banks) spread over the banks.
    constexpr int kSlots = kMaxGrid + kMaxGrid / kChunk;
    __shared__ uint4 sp[kSlots];         // (q[0..7] + 1/8)^2 as bf16
    __shared__ uint4 sm[kSlots];         // (q[0..7] - 1/8)^2 as bf16
    __shared__ uint4 sq[kSlots];         // q[0..7] as bf16
    __shared__ uint16_t sout16[kPayloads * kBlocksPerWG * kBlockBytes / 2];
    __shared__ int sgrid_bad;
    uint8_t* sout = reinterpret_cast<uint8_t*>(sout16);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int n = a.grid_size;
    const int nchunks = (n + kChunk - 1) / kChunk;
    const int npad = nchunks * kChunk;

    if (tid == 0) sgrid_bad = 0;
    if (kMode != kModeCandidates)
        for (int i = tid; i < kPayloads * kBlocksPerWG * kBlockBytes / 2; i += kThreads) sout16[i] = 0;
    __syncthreads();
    // Stage the grid as bf16 (exact for ternary values); entries past the end
    // repeat the last one, which always comes first in index order.
    {
        const float4* gsrc = reinterpret_cast<const float4*>(a.grid);
        int bad = 0;
        for (int e = tid; e < npad; e += kThreads) {
            const int src = e < n ? e : n - 1;
            const float4 v0 = gsrc[2 * src], v1 = gsrc[2 * src + 1];
            const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            uint32_t h[8], hp[8], hm[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                bad |= !(v[t] == 0.0f || v[t] == 1.0f || v[t] == -1.0f);
                h[t] = bf16_bits(v[t]);
                const float p = v[t] + 0.125f, m = v[t] - 0.125f;
                hp[t] = bf16_bits(p * p);          // exact: 81/64, 1/64, 49/64
                hm[t] = bf16_bits(m * m);
            }
            const int at = e + e / kChunk;
            sq[at] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                  h[4] | (h[5] << 16), h[6] | (h[7] << 16));
            sp[at] = make_uint4(hp[0] | (hp[1] << 16), hp[2] | (hp[3] << 16),
                                  hp[4] | (hp[5] << 16), hp[6] | (hp[7] << 16));
            sm[at] = make_uint4(hm[0] | (hm[1] << 16), hm[2] | (hm[3] << 16),
                                  hm[4] | (hm[5] << 16), hm[6] | (hm[7] << 16));
        }
        if (bad) sgrid_bad = 1;
    }
    __syncthreads();
    const bool grid_bad = sgrid_bad != 0;
    if (grid_bad && tid == 0) report(a.status, IQ_ERR_GRID);

    const int col = lane & 15;          // matrix column = group within the half block
    const int kb = lane >> 4;           // K slice of the operands / row quarter of the result
    const int half = wave & 1;
    const int g = half * 16 + col;      // group in block
    const int sub = g >> 2;
    const int lq = g & 3;

    for (int pass = 0; pass < kPasses; ++pass) {
        const int slot = pass * kBlocksPerPass + (wave >> 1);
        const int64_t blk = (int64_t)blockIdx.x * kBlocksPerWG + slot;
        if (blk >= a.g.nblocks) continue;                      // wave-uniform
        const int64_t bt = blk / a.g.blocks_per_batch;
        const int64_t cb = blk % a.g.blocks_per_row;
        const float* xblk = a.w + blk * kBlockElems;
        const float* wblk = a.imp ? a.imp + bt * a.g.cols + cb * kBlockElems : nullptr;

        // Whole-block checks and amax (each lane reads 4 of the 256 values).
        int err = 0;
        float amax = 0.0f;
        {
            const float4 xv = reinterpret_cast<const float4*>(xblk)[lane];
            const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (!finite_f32(xs[t])) err = IQ_ERR_NONFINITE;
                amax = fmaxf(amax, fabsf(xs[t]));
            }
            if (wblk && !err) {
                const float4 wv = reinterpret_cast<const float4*>(wblk)[lane];
                const float ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (!(ws[t] >= 0.0f) || !finite_f32(ws[t])) err = IQ_ERR_IMPORTANCE;
            }
        }
        if (err && half == 0) report(a.status, err);
        const bool block_bad = __ballot(err != 0) != 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));

        uint32_t dh;
        if (a.scales) {
            dh = (uint32_t)a.scales[blk];
        } else {
            const float t = amax / 16.875f;
            const float u = t * 0.61f;
            dh = f32_to_f16_bits(u);
        }
        const bool scale_bad = ((dh & 0x7c00u) == 0x7c00u) || ((dh & 0x8000u) && (dh & 0x7fffu));
        dh &= 0x7fffu;
        if (scale_bad && !block_bad && half == 0 && lane == 0) report(a.status, IQ_ERR_SCALE_RANGE);
        const float d = scale_bad ? 0.0f : f16_bits_to_f32(dh);

        // Forced choices: every wave of the block checks all 8 of them.
        int forced = -1;
        bool choice_bad = false;
        if (kMode != kModeEvery && a.choices) {
            const int cv = lane < 8 ? a.choices[blk * 8 + lane] : 0;
            const bool bad = cv < 0 || cv > 15;
            if (bad && half == 0) report(a.status, IQ_ERR_ARG);
            choice_bad = __ballot(bad) != 0;
            forced = a.choices[blk * 8 + sub];
        }
        const bool zero_block = grid_bad || block_bad || scale_bad || dh == 0u || choice_bad;
        if (choice_bad) forced = -1;

        // The lane's group: values, weights, sums, and its K slice of the
        // three-way bf16 split of -2*w*x and w (slice 3 is zero padding).
        float x[8], w[8];
        load_group(xblk, wblk, g, zero_block, x, w);
        const float inv_d = zero_block ? 1.0f : 1.0f / d;
        float W = 0.0f, B = 0.0f;
        uint32_t bwx[8], bw[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float wxj = w[j] * x[j];
            W += w[j];
            B += wxj;
            bwx[j] = kb < 3 ? split_part(-2.0f * (wxj * inv_d), kb) : 0u;
            bw[j] = kb < 3 ? split_part(w[j], kb) : 0u;
        }
        const v8bf opn2wx = as_v8bf(make_uint4(bwx[0] | (bwx[1] << 16), bwx[2] | (bwx[3] << 16),
                                               bwx[4] | (bwx[5] << 16), bwx[6] | (bwx[7] << 16)));
        const v8bf opw = as_v8bf(make_uint4(bw[0] | (bw[1] << 16), bw[2] | (bw[3] << 16),
                                            bw[4] | (bw[5] << 16), bw[6] | (bw[7] << 16)));
        const float w64 = W * 0.015625f;
        const float b4 = B * 0.25f;
        const float b4d = b4 * inv_d;
        const v4f cnp = {-b4d, -b4d, -b4d, -b4d};     // -2*(+1/8)*B/d
        const v4f cnm = {b4d, b4d, b4d, b4d};         // -2*(-1/8)*B/d

        // Sweep.
        // chunk_of: 4-bit chunk index of choice c in bits 4*(c%8) of word c/8.
        float best[16], snap[16];
        uint32_t chunk_of[2] = {0u, 0u};
#pragma unroll
        for (int c = 0; c < 16; ++c) { best[c] = __builtin_inff(); snap[c] = best[c]; }
        const v4f zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int ch = 0; ch < nchunks; ++ch) {
            for (int tt = 0; tt < kChunkTiles; ++tt) {
                const int at = (ch * kChunkTiles + tt) * kTile + col + ch;
                const v8bf ap = as_v8bf(sp[at]);
                const v8bf am = as_v8bf(sm[at]);
                const v8bf aq = as_v8bf(sq[at]);
                const v4f up = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, opw, zero4, 0, 0, 0);
                const v4f um = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, opw, zero4, 0, 0, 0);
                const v4f vnp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, opn2wx, cnp, 0, 0, 0);
                const v4f vnm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, opn2wx, cnm, 0, 0, 0);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float mk = (float)(2 * k + 1);
                    const float p0 = __builtin_fmaf(up[0], mk, vnp[0]);
                    const float p1 = __builtin_fmaf(up[1], mk, vnp[1]);
                    const float p2 = __builtin_fmaf(up[2], mk, vnp[2]);
                    const float p3 = __builtin_fmaf(up[3], mk, vnp[3]);
                    const float m0 = __builtin_fmaf(um[0], mk, vnm[0]);
                    const float m1 = __builtin_fmaf(um[1], mk, vnm[1]);
                    const float m2 = __builtin_fmaf(um[2], mk, vnm[2]);
                    const float m3 = __builtin_fmaf(um[3], mk, vnm[3]);
                    best[k] = fminf(best[k], fminf(fminf(fminf(p0, p1), p2), p3));
                    best[8 + k] = fminf(best[8 + k], fminf(fminf(fminf(m0, m1), m2), m3));
                }
            }
            const uint32_t chrep = (uint32_t)ch * 0x11111111u;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const uint32_t m = best[c] < snap[c] ? (0xfu << (4 * (c & 7))) : 0u;
                chunk_of[c >> 3] = (chunk_of[c >> 3] & ~m) | (chrep & m);
                snap[c] = best[c];
            }
        }

        // Sub-block choice: per group, the least minimum of its four lanes; per
        // sub-block, s_k times the sum over its four groups (identical float sum
        // in every lane of the sub-block).
        int cstar = 0;
        float cbest = 0.0f;
        float cost[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            float m = best[c];
            m = fminf(m, __shfl_xor(m, 16));
            m = fminf(m, __shfl_xor(m, 32));
            float v = m + __shfl_xor(m, 1);
            v += __shfl_xor(v, 2);
            cost[c] = (float)(2 * (c & 7) + 1) * v;
            if (c == 0 || cost[c] < cbest) { cbest = cost[c]; cstar = c; }
        }
        if (forced >= 0) cstar = forced;
        // Candidates: the top_c choices by (cost, c); with a zero scale every
        // choice decodes to zero with entry 0, so the order is c = 0, 1, ...
        const bool rejected = grid_bad || block_bad || scale_bad || choice_bad;
        const bool zero_scale = !rejected && dh == 0u;
        int used = 0;

        // Entry of choice cs for this lane's group: the lane rescans its
        // entries of the chunk that holds its minimum of that choice, then the
        // lane of the column whose matrix-core minimum is least is kept; the
        // payload takes the low byte per group, the qh word per sub-block and
        // d per block.
        const int nloop = kMode == kModeEvery ? 16 : (kMode == kModeCandidates ? a.top_c : 1);
        for (int it = 0; it < nloop; ++it) {
            int cs = kMode == kModeEvery ? it : cstar;
            if (kMode == kModeCandidates) {
                int cr = -1;
                float vr = 0.0f;
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const bool better = zero_scale ? (cr < 0) : (cr < 0 || cost[c] < vr);
                    if (!((used >> c) & 1) && better) { cr = c; vr = cost[c]; }
                }
                used |= 1 << cr;
                cs = cr;
            }
            float lane_min = best[0];
#pragma unroll
            for (int c = 1; c < 16; ++c)
                if (cs == c) lane_min = best[c];
            const int tchunk = (int)((chunk_of[cs >> 3] >> (4 * (cs & 7))) & 0xfu);
            int idx = rescan(sq, tchunk, kb, cs, xblk, wblk, g, zero_block, w64, b4, inv_d);
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) {
                const float om = __shfl_xor(lane_min, o);
                const int oi = __shfl_xor(idx, o);
                if (om < lane_min || (om == lane_min && oi < idx)) { lane_min = om; idx = oi; }
            }
            idx = idx < n ? idx : n - 1;
            if (kMode == kModeCandidates) {
                // One lane per group writes its 8 errors xhat - x (xhat exact
                // in fp32, one rounding), its entry and, once per sub-block,
                // the choice.
                if (zero_scale) idx = 0;
                if (kb == 0) {
                    const int64_t base = (blk * 8 + sub) * a.top_c + it;     // [block][sub][r]
                    float xo[8], wo[8];
                    load_group(xblk, wblk, g, rejected, xo, wo);
                    const float sk = f16_bits_to_f32(dh) * (float)(2 * (cs & 7) + 1);
                    const float delta = (cs >> 3) ? -0.125f : 0.125f;
                    const uint4 u = sq[idx + idx / kChunk];
                    const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
                    float ev[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float q = bf16_to_f32((uu[j >> 1] >> (16 * (j & 1))) & 0xffffu);
                        ev[j] = rejected ? 0.0f : sk * (q + delta) - xo[j];
                    }
                    float4* ep = reinterpret_cast<float4*>(a.cand_err + base * 32 + lq * 8);
                    ep[0] = make_float4(ev[0], ev[1], ev[2], ev[3]);
                    ep[1] = make_float4(ev[4], ev[5], ev[6], ev[7]);
                    if (lq == 0) a.cand_choice[base] = cs;
                    if (a.cand_codes) a.cand_codes[base * 4 + lq] = rejected ? (uint16_t)0 : (uint16_t)idx;
                }
                continue;
            }
            int hi = ((idx >> 8) & 7) << (3 * lq);
            hi |= __shfl_xor(hi, 1);
            hi |= __shfl_xor(hi, 2);
            if (!zero_block && kb == 0) {
                uint8_t* ob = sout + (it * kBlocksPerWG + slot) * kBlockBytes;
                ob[2 + 4 * sub + lq] = (uint8_t)(idx & 0xff);
                if (lq == 0) {
                    const uint32_t qh = (uint32_t)hi | ((uint32_t)cs << 12);
                    ob[34 + 2 * sub] = (uint8_t)(qh & 0xff);
                    ob[35 + 2 * sub] = (uint8_t)(qh >> 8);
                }
                if (g == 0) {
                    ob[0] = (uint8_t)(dh & 0xff);
                    ob[1] = (uint8_t)(dh >> 8);
                }
            }
            if (kMode == kModeFake && kb == 0) {
                // The decoded group, d*(2k+1)*(q + delta) with the payload's
                // fields (a zero block decodes as the all-zero payload does;
                // a rejected block is written as zeros).
                const uint32_t dz = zero_block ? 0u : dh;
                const int ez = zero_block ? 0 : idx;
                const int cz = zero_block ? 0 : cs;
                const float sk = f16_bits_to_f32(dz) * (float)(2 * (cz & 7) + 1);
                const float delta = (cz >> 3) ? -0.125f : 0.125f;
                const uint4 u = sq[ez + ez / kChunk];
                const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
                const bool rejected = grid_bad || block_bad || scale_bad || choice_bad;
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float q = bf16_to_f32((uu[j >> 1] >> (16 * (j & 1))) & 0xffffu);
                    v[j] = rejected ? 0.0f : sk * (q + delta);
                }
                float4* o = reinterpret_cast<float4*>(a.xhat + blk * kBlockElems + g * 8);
                o[0] = make_float4(v[0], v[1], v[2], v[3]);
                o[1] = make_float4(v[4], v[5], v[6], v[7]);
            }
        }
    }
    if (kMode != kModeCandidates && a.out) {
        __syncthreads();
        const int64_t first = (int64_t)blockIdx.x * kBlocksPerWG;
        const int64_t left = a.g.nblocks - first;
        const int nb = left < kBlocksPerWG ? (int)left : kBlocksPerWG;
        for (int cs = 0; cs < kPayloads; ++cs) {
            uint16_t* o16 = reinterpret_cast<uint16_t*>(a.out + (cs * a.g.nblocks + first) * kBlockBytes);
            const uint16_t* s16 = sout16 + cs * kBlocksPerWG * (kBlockBytes / 2);
            for (int i = tid; i < nb * (kBlockBytes / 2); i += kThreads) o16[i] = s16[i];
        }
    }
}

}  // namespace

hipError_t launch_iq1s_encode(const float* w, const float* imp, const float* grid, int grid_size,
                              const uint16_t* scales, const int32_t* choices, uint8_t* out,
                              float* xhat, int mode, int32_t* status, const BlockGeom& g,
                              hipStream_t stream)
{
    Iq1sArgs a{w, imp, grid, scales, choices, out, xhat, nullptr, nullptr, nullptr, status, g,
               grid_size, 0};
    const int64_t wgs = (g.nblocks + kBlocksPerWG - 1) / kBlocksPerWG;
    if (mode == kModeEvery)
        hipLaunchKernelGGL(iq1s_encode_kernel<kModeEvery>, dim3((unsigned)wgs), dim3(kThreads), 0,
                           stream, a);
    else if (mode == kModeFake)
        hipLaunchKernelGGL(iq1s_encode_kernel<kModeFake>, dim3((unsigned)wgs), dim3(kThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(iq1s_encode_kernel<kModePayload>, dim3((unsigned)wgs), dim3(kThreads), 0,
                           stream, a);
    return hipGetLastError();
}

hipError_t launch_iq1s_candidates(const float* w, const float* imp, const float* grid,
                                  int grid_size, int top_c, float* cand_err, int32_t* cand_choice,
                                  uint16_t* cand_codes, int32_t* status, const BlockGeom& g,
                                  hipStream_t stream)
{
    Iq1sArgs a{w, imp, grid, nullptr, nullptr, nullptr, nullptr, cand_err, cand_choice, cand_codes,
               status, g, grid_size, top_c};
    const int64_t wgs = (g.nblocks + kBlocksPerWG - 1) / kBlocksPerWG;
    hipLaunchKernelGGL(iq1s_encode_kernel<kModeCandidates>, dim3((unsigned)wgs), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace iqk
