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
// With the signs fixed, the error of a group and an entry is, up to a
// constant, s^2*N - 2s*P with N = sum w*q^2 and P = sum (w*sign*x)*q.  P and
// N for 16 entries x 16 groups are two [16 x 8] x [8 x 16] products on the
// matrix cores.  When every grid value and its square are exact in bf16 (the
// odd-integer grids {1,3,5} among them), each is one v_mfma_f32_16x16x32_bf16
// with the group side split in three bf16 parts whose sum is the fp32 value,
// so the products are exact; any other magnitude grid is used as given with
// fp32 operands (two v_mfma_f32_16x16x4_f32 each, four times the matrix-core
// time).  Dividing by d, the key of local scale k is (2k+1)*N - 2P/d: one FMA
// with a literal multiplier; the choice cost of a scale group is (2k+1) times
// the sum of its two groups' minima.
//
// Two kernels.  The payload encode (iq2xs_payload_wide_kernel, below) runs
// 32 x 32 matrix tiles with a wave per block.  The other outputs (every
// choice, fake quant, candidates) run iq2xs_kernel with 16 x 16 tiles.
//
// Layout of iq2xs_kernel: a wave owns 16 groups (half a block); matrix
// column j = lane%16 is group j, the lane's accumulator rows are entries
// 4*(lane/16)+r of each 16-entry tile.  A 1024-thread workgroup runs 8 blocks per pass and 2 passes
// per set of 16 blocks; the workgroups are persistent (one per CU) and stage
// the grid once in LDS (q and q^2 as fp32 and as bf16, and a padded fp32 copy
// for the rescans: 85 KiB).  Value-only minima (v_min3); each lane records
// the chunk that last lowered each minimum; the lane of each column whose
// matrix-core minimum is least is found, and the four lanes of the column
// split its entries of that chunk and rescan them on the VALU (lowest entry
// of least key).
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace iqk {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWavesPerWG = 16;
constexpr int kThreads = kWave * kWavesPerWG;        // 1024
constexpr int kBlocksPerPass = kWavesPerWG / 2;
constexpr int kPasses = 2;
constexpr int kBlocksPerWG = kBlocksPerPass * kPasses;   // 16
constexpr int kTile = 16;
constexpr int kMaxGrid = 512;
constexpr int kBlockBytes = 74;

struct Iq2xsArgs {
    const void* w;           // weights in the storage type the kernel is built for
    const float* imp;
    const float* grid;
    const uint16_t* scales;
    const int32_t* choices;
    uint8_t* out;            // payload [nblocks][74], every choice [16][nblocks][74]; may be
                             // NULL for the fake-quant output
    float* xhat;             // fake quant: decoded values [nblocks][256]
    float* cand_err;         // candidates
    int32_t* cand_choice;
    uint16_t* cand_codes;
    int32_t* status;
    BlockGeom g;
    int grid_size;
    int top_c;
};

template <class XB>
__device__ __forceinline__ void load_group(const XB& xb, const float* wblk, int g, bool zero,
                                           float (&x)[8], float (&w)[8])
{
    if (zero) {
#pragma unroll
        for (int j = 0; j < 8; ++j) { x[j] = 0.0f; w[j] = 1.0f; }
        return;
    }
    xb.group(g, x);
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

// Input signs with the weakest element (smallest (w*x)*x, lowest index)
// flipped when the count of negatives is odd.  Bit j set = element j negative.
__device__ __forceinline__ int group_signs(const float (&x)[8], const float (&w)[8])
{
    int neg = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (x[j] < 0.0f) neg |= 1 << j;
    if (__popc(neg) & 1) {
        int jw = 0;
        float wk = (w[0] * x[0]) * x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) {
            const float v = (w[j] * x[j]) * x[j];
            if (v < wk) { wk = v; jw = j; }
        }
        neg ^= 1 << jw;
    }
    return neg;
}

// True when v and v*v are both exact in bf16 (then v*v is exact in fp32 too:
// at most 16 significant bits, and the range keeps it normal).
__device__ __forceinline__ bool bf16_exact_with_square(float v)
{
    const bool range = v == 0.0f || (v >= 0x1p-60f && v <= 0x1p60f);
    const float v2 = v * v;
    return range && bf16_to_f32(bf16_bits(v)) == v && bf16_to_f32(bf16_bits(v2)) == v2;
}

// One matrix tile of P' = -2P/d and N: the 16 keys (2k+1)*N + P' of the
// lane's 4 entries folded into the running minima.
__device__ __forceinline__ void fold_tile(const v4f& pn, const v4f& nn, float (&best)[16])
{
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const float mk = (float)(2 * k + 1);
        const float k0 = __builtin_fmaf(nn[0], mk, pn[0]);
        const float k1 = __builtin_fmaf(nn[1], mk, pn[1]);
        const float k2 = __builtin_fmaf(nn[2], mk, pn[2]);
        const float k3 = __builtin_fmaf(nn[3], mk, pn[3]);
        best[k] = fminf(best[k], fminf(fminf(fminf(k0, k1), k2), k3));
    }
}

// After chunk ch: record ch (4 bits at bits 4*(k%8) of word k/8) for every
// minimum that it lowered.
__device__ __forceinline__ void track_chunk(int ch, const float (&best)[16], float (&snap)[16],
                                            uint32_t (&chunk_of)[2])
{
    const uint32_t chrep = (uint32_t)ch * 0x11111111u;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const uint32_t msk = best[k] < snap[k] ? (0xfu << (4 * (k & 7))) : 0u;
        chunk_of[k >> 3] = (chunk_of[k >> 3] & ~msk) | (chrep & msk);
        snap[k] = best[k];
    }
}

// Weighted squared error of a group against s*sign*q in fp64, from its
// definition: sum of w*(x - s*sign*q)^2.
__device__ __forceinline__ double group_error64(const float (&x)[8], const float (&w)[8], int neg,
                                                const float* q, double s)
{
    double e = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const double sq = s * (double)q[j];
        const double r = (double)x[j] - (((neg >> j) & 1) ? -sq : sq);
        e += (double)w[j] * r * r;
    }
    return e;
}

// Per-entry fp32 copy of the grid for the VALU rescans: q[0..7], q^2[0..7],
// padded to 18 floats so the four entries the four lanes of a column read
// together (4 apart) fall in different LDS banks.
constexpr int kEntryStride = 18;
// Tracking chunks are 32 or 64 entries, a multiple of the 64 LDS banks apart
// at that stride, so lanes rescanning different chunks would all hit the same
// banks; every chunk therefore starts 2 floats later than the stride alone
// puts it.
template <int kChunk>
__device__ __forceinline__ int entry_off(int e) { return kEntryStride * e + 2 * (e / kChunk); }

// VALU rescan for local scale k: positions p0 .. p0+np-1 of the entries one
// lane of a column covers in chunk `chunk` (position p = tile p/4 of the
// chunk, row 4*kbs + p%4): the lowest entry with the least key
// (2k+1)*N - 2P/d.  Returns the entry, writes its key.
template <int kChunkTiles>
__device__ __forceinline__ int rescan(const float* __restrict__ sg, int chunk, int kbs, int p0,
                                      int np, int k, const float (&wxs)[8], const float (&w)[8],
                                      float inv_d, float* key_out)
{
    const float mk = (float)(2 * k + 1);
    int idx = -1;
    float vbest = 0.0f;
    for (int pp = p0; pp < p0 + np; ++pp) {
        const int e = (chunk * kChunkTiles + (pp >> 2)) * kTile + 4 * kbs + (pp & 3);
        const float2* p = reinterpret_cast<const float2*>(sg + entry_off<kChunkTiles * kTile>(e));
        float q[8], q2[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float2 u = p[t], v = p[4 + t];
            q[2 * t] = u.x; q[2 * t + 1] = u.y;
            q2[2 * t] = v.x; q2[2 * t + 1] = v.y;
        }
        float P = 0.0f, N = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            P = __builtin_fmaf(wxs[j], q[j], P);
            N = __builtin_fmaf(w[j], q2[j], N);
        }
        const float key = __builtin_fmaf(N, mk, (-2.0f * P) * inv_d);
        if (idx < 0 || key < vbest) { vbest = key; idx = e; }
    }
    *key_out = vbest;
    return idx;
}

// kMode: EncodeMode; kDT: the weight's iq_dtype_t.
template <int kMode, int kDT>
__global__ __launch_bounds__(kThreads) void iq2xs_kernel(Iq2xsArgs a)
{
    constexpr bool kCandidates = kMode == kModeCandidates;
    constexpr int kPayloads = kMode == kModeEvery ? 16 : 1;
    // Tiles per tracking chunk.  Recording chunks costs the sweep about 4
    // instructions per choice and chunk; each pick rescans one lane's
    // entries of a chunk, 4 per tile.  One pick per group (payload, fake
    // quant): 8 tiles (128 entries); top_c picks (candidates): 4; 16 picks
    // (every choice): 2.
    constexpr int kChunkTiles = kCandidates ? 4 : (kMode == kModeEvery ? 2 : 8);
    constexpr int kChunk = kTile * kChunkTiles;

    __shared__ float sgrid[kMaxGrid * kEntryStride + 2 * (kMaxGrid / 32)];  // q[0..7], q^2[0..7]
    __shared__ float2 sq[kMaxGrid * 4];                 // entry e, slice kb: (q[kb], q[kb+4])
    __shared__ float2 sq2[kMaxGrid * 4];                // same for q^2
    __shared__ uint4 sbq[kMaxGrid];                     // entry e: q[0..7] as bf16
    __shared__ uint4 sbq2[kMaxGrid];                    // entry e: q^2[0..7] as bf16
    __shared__ int sgrid_inexact;
    __shared__ uint16_t sout16[kPayloads * kBlocksPerWG * kBlockBytes / 2];
    __shared__ int sgrid_bad;
    uint8_t* sout = reinterpret_cast<uint8_t*>(sout16);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int n = a.grid_size;
    const int nchunks = (n + kChunk - 1) / kChunk;
    const int npad = nchunks * kChunk;

    if (tid == 0) { sgrid_bad = 0; sgrid_inexact = 0; }
    if (!kCandidates)
        for (int i = tid; i < kPayloads * kBlocksPerWG * kBlockBytes / 2; i += kThreads) sout16[i] = 0;
    __syncthreads();
    {
        int bad = 0, inexact = 0;
        // One (entry, slice) pair per thread: consecutive threads write
        // consecutive LDS words.
        for (int i = tid; i < npad * 4; i += kThreads) {
            const int e = i >> 2, t = i & 3;
            const int src = e < n ? e : n - 1;
            const float a0 = a.grid[8 * src + 2 * t], a1 = a.grid[8 * src + 2 * t + 1];
            const float b0 = a.grid[8 * src + t], b1 = a.grid[8 * src + t + 4];
            bad |= !(a0 >= 0.0f && finite_f32(a0) && a1 >= 0.0f && finite_f32(a1));
            float2* ge = reinterpret_cast<float2*>(sgrid + entry_off<kChunk>(e));
            ge[t] = make_float2(a0, a1);
            ge[4 + t] = make_float2(a0 * a0, a1 * a1);
            sq[i] = make_float2(b0, b1);
            sq2[i] = make_float2(b0 * b0, b1 * b1);
            // Word t of the bf16 rows: elements 2t and 2t+1.
            inexact |= !(bf16_exact_with_square(a0) && bf16_exact_with_square(a1));
            reinterpret_cast<uint32_t*>(sbq)[i] = bf16_bits(a0) | (bf16_bits(a1) << 16);
            reinterpret_cast<uint32_t*>(sbq2)[i] = bf16_bits(a0 * a0) | (bf16_bits(a1 * a1) << 16);
        }
        if (bad) sgrid_bad = 1;
        if (inexact) sgrid_inexact = 1;
    }
    __syncthreads();
    const bool grid_bad = sgrid_bad != 0;
    const bool grid_exact = sgrid_inexact == 0;     // workgroup-uniform
    if (grid_bad && tid == 0) report(a.status, IQ_ERR_GRID);

    const int col = lane & 15;
    const int kb = lane >> 4;
    const int half = wave & 1;
    const int g = half * 16 + col;          // group in block
    const int m = g >> 1;                   // scale group
    const int h = g & 1;                    // group in scale group

    // Persistent workgroups: the grid is staged once, then each workgroup
    // takes every gridDim.x-th set of 16 blocks.
    const int64_t nsets = (a.g.nblocks + kBlocksPerWG - 1) / kBlocksPerWG;
    for (int64_t set = blockIdx.x; set < nsets; set += gridDim.x) {
    if (set != blockIdx.x) __syncthreads();     // the previous set's payloads are out
    for (int pass = 0; pass < kPasses; ++pass) {
        const int slot = pass * kBlocksPerPass + (wave >> 1);
        const int64_t blk = set * kBlocksPerWG + slot;
        if (blk >= a.g.nblocks) continue;                      // wave-uniform
        const int64_t bt = blk / a.g.blocks_per_batch;
        const int64_t cb = blk % a.g.blocks_per_row;
        const WeightBlock<kDT> xb(a.w, blk);
        const float* wblk = a.imp ? a.imp + bt * a.g.cols + cb * kBlockElems : nullptr;

        int err = 0;
        float amax = 0.0f;
        {
            const float4 xv = xb.quad(lane);
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
        if (!kCandidates && a.scales) {
            dh = (uint32_t)a.scales[blk];
        } else {
            const float t = amax / 155.0f;
            const float u = t * 0.61f;
            dh = f32_to_f16_bits(u);
        }
        const bool scale_bad = ((dh & 0x7c00u) == 0x7c00u) || ((dh & 0x8000u) && (dh & 0x7fffu));
        dh &= 0x7fffu;
        if (scale_bad && !block_bad && half == 0 && lane == 0) report(a.status, IQ_ERR_SCALE_RANGE);
        const float d = scale_bad ? 0.0f : f16_bits_to_f32(dh);

        int forced = -1;
        bool choice_bad = false;
        if ((kMode == kModePayload || kMode == kModeFake) && a.choices) {
            int ln = lane;                  // opaque: the address is formed here, not hoisted
            __asm__ volatile("" : "+v"(ln));
            const int cv = ln < 16 ? a.choices[blk * 16 + ln] : 0;
            const bool bad = cv < 0 || cv > 15;
            if (bad && half == 0) report(a.status, IQ_ERR_ARG);
            choice_bad = __ballot(bad) != 0;
            forced = choice_bad ? -1 : a.choices[blk * 16 + m];
        }
        const bool bad_block = grid_bad || block_bad || scale_bad || choice_bad;
        const bool zero_scale = dh == 0u;
        const bool skip = bad_block || zero_scale;

        // The lane's group: values, weights and signs.
        float x[8], w[8];
        load_group(xb, wblk, g, skip, x, w);
        const int neg = group_signs(x, w);
        const float inv_d = skip ? 1.0f : 1.0f / d;

        // Sweep.
        float best[16], snap[16];
        uint32_t chunk_of[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < 16; ++k) { best[k] = __builtin_inff(); snap[k] = best[k]; }
        const v4f zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
        if (grid_exact) {
            // The lane's K slice kb of the group side: part kb of the exact
            // three-way bf16 split of -2*(w*sign*x)/d and of w, for all 8
            // elements (slice 3 is zero padding).
            uint32_t hp[8], hw[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float v = w[j] * x[j];
                if ((neg >> j) & 1) v = -v;
                v = -2.0f * (v * inv_d);
                hp[j] = kb < 3 ? split_part(v, kb) : 0u;
                hw[j] = kb < 3 ? split_part(w[j], kb) : 0u;
            }
            const v8bf opp = as_v8bf(make_uint4(hp[0] | (hp[1] << 16), hp[2] | (hp[3] << 16),
                                                hp[4] | (hp[5] << 16), hp[6] | (hp[7] << 16)));
            const v8bf opw = as_v8bf(make_uint4(hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16),
                                                hw[4] | (hw[5] << 16), hw[6] | (hw[7] << 16)));
            for (int ch = 0; ch < nchunks; ++ch) {
                for (int tt = 0; tt < kChunkTiles; ++tt) {
                    const int e = (ch * kChunkTiles + tt) * kTile + col;
                    const v4f pn = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(sbq[e]), opp, zero4, 0, 0, 0);
                    const v4f nn = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(sbq2[e]), opw, zero4, 0, 0, 0);
                    fold_tile(pn, nn, best);
                }
                track_chunk(ch, best, snap, chunk_of);
            }
        } else {
            // fp32 operands: elements kb and kb+4 of the group side, read
            // again rather than selected from registers.
            float bw0 = 1.0f, bw1 = 1.0f, bx0 = 0.0f, bx1 = 0.0f;
            if (!skip) {
                bx0 = xb.one(g * 8 + kb);
                bx1 = xb.one(g * 8 + kb + 4);
                if (wblk) { bw0 = wblk[g * 8 + kb]; bw1 = wblk[g * 8 + kb + 4]; }
            }
            float bp0 = bw0 * bx0, bp1 = bw1 * bx1;
            if ((neg >> kb) & 1) bp0 = -bp0;
            if ((neg >> (kb + 4)) & 1) bp1 = -bp1;
            bp0 = -2.0f * (bp0 * inv_d);
            bp1 = -2.0f * (bp1 * inv_d);
            for (int ch = 0; ch < nchunks; ++ch) {
                for (int tt = 0; tt < kChunkTiles; ++tt) {
                    const int e = (ch * kChunkTiles + tt) * kTile + col;
                    const float2 aq = sq[4 * e + kb];
                    const float2 aq2 = sq2[4 * e + kb];
                    v4f pn = __builtin_amdgcn_mfma_f32_16x16x4f32(aq.x, bp0, zero4, 0, 0, 0);
                    pn = __builtin_amdgcn_mfma_f32_16x16x4f32(aq.y, bp1, pn, 0, 0, 0);
                    v4f nn = __builtin_amdgcn_mfma_f32_16x16x4f32(aq2.x, bw0, zero4, 0, 0, 0);
                    nn = __builtin_amdgcn_mfma_f32_16x16x4f32(aq2.y, bw1, nn, 0, 0, 0);
                    fold_tile(pn, nn, best);
                }
                track_chunk(ch, best, snap, chunk_of);
            }
        }

        // The rescans need the signed weighted values again; they are
        // rebuilt from memory rather than held through the sweep.
        __asm__ volatile("" ::: "memory");
        load_group(xb, wblk, g, skip, x, w);
        float wxs[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float wx = w[j] * x[j];
            wxs[j] = ((neg >> j) & 1) ? -wx : wx;
        }

        // Scale-group cost of every local scale: the least minimum of each
        // group's four lanes, summed over the two groups, times 2k+1.
        float cost[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            float v = best[k];
            v = fminf(v, __shfl_xor(v, 16));
            v = fminf(v, __shfl_xor(v, 32));
            cost[k] = (float)(2 * k + 1) * (v + __shfl_xor(v, 1));
        }

        // Entry of local scale k for this lane's group: rescan the lane's part
        // of its winning chunk, then keep the lane of least matrix-core minimum.
        auto pick = [&](int k) -> int {
            float lm = best[0];
#pragma unroll
            for (int c = 1; c < 16; ++c)
                if (k == c) lm = best[c];
            const int tchunk = (int)((chunk_of[k >> 3] >> (4 * (k & 7))) & 0xfu);
            // The lane of the column whose matrix-core minimum is least holds
            // the entry.  Unless two lanes of some column hold equal minima,
            // the four lanes split that lane's entries of its chunk and keep
            // the least key, lowest entry on equal keys; with equal minima
            // every lane rescans its own entries and the lane of least
            // minimum, then lowest entry, wins.
            constexpr int kPer = kChunkTiles;          // 4*kChunkTiles entries over 4 lanes
            float cm = fminf(lm, __shfl_xor(lm, 16));
            cm = fminf(cm, __shfl_xor(cm, 32));
            const uint64_t holders = (__ballot(lm == cm) >> col) & 0x0001000100010001ull;
            const bool tie = __ballot(__popcll(holders) > 1) != 0;      // wave-uniform
            int idx;
            float key;
            if (!tie) {
                const int kbs = __builtin_ctzll(holders) >> 4;
                const int tch = __shfl(tchunk, col + 16 * kbs);
                idx = rescan<kChunkTiles>(sgrid, tch, kbs, kb * kPer, kPer, k, wxs, w, inv_d, &key);
#pragma unroll
                for (int o = 16; o <= 32; o <<= 1) {
                    const float ok = __shfl_xor(key, o);
                    const int oi = __shfl_xor(idx, o);
                    if (ok < key || (ok == key && oi < idx)) { key = ok; idx = oi; }
                }
            } else {
                idx = rescan<kChunkTiles>(sgrid, tchunk, kb, 0, 4 * kChunkTiles, k, wxs, w, inv_d,
                                          &key);
#pragma unroll
                for (int o = 16; o <= 32; o <<= 1) {
                    const float om = __shfl_xor(lm, o);
                    const int oi = __shfl_xor(idx, o);
                    if (om < lm || (om == lm && oi < idx)) { lm = om; idx = oi; }
                }
            }
            return idx < n ? idx : n - 1;
        };

        if (kMode == kModeEvery) {
            // Every local scale k for every scale group: the payload forced to k.
            for (int k = 0; k < 16; ++k) {
                const int idx = pick(k);
                if (!skip && kb == 0) {
                    uint8_t* ob = sout + (k * kBlocksPerWG + slot) * kBlockBytes;
                    const uint32_t code = (uint32_t)idx | ((uint32_t)(neg & 0x7f) << 9);
                    ob[2 + 2 * g] = (uint8_t)(code & 0xff);
                    ob[3 + 2 * g] = (uint8_t)(code >> 8);
                    if ((g & 3) == 0) ob[66 + (m >> 1)] = (uint8_t)(k | (k << 4));
                    if (g == 0) {
                        ob[0] = (uint8_t)(dh & 0xff);
                        ob[1] = (uint8_t)(dh >> 8);
                    }
                }
            }
        } else if (!kCandidates) {
            int kstar = 0;
            float cbv = cost[0];
#pragma unroll
            for (int k = 1; k < 16; ++k)
                if (cost[k] < cbv) { cbv = cost[k]; kstar = k; }
            int idx;
            if (forced >= 0) {                      // wave-uniform
                kstar = forced;
                idx = pick(kstar);
            } else {
                // The runner-up local scale.  The fp32 costs carry rounding
                // of the size of the sums they cancel, so when the runner-up
                // is within 2^-18 of the best's magnitude (32 to 64 ulps) both
                // are evaluated again in fp64 from the error's definition,
                // with their own entries; the lower error wins, the lower k on
                // equal errors.
                int k2 = kstar == 0 ? 1 : 0;
                float c2 = cost[k2];
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    if (k != kstar && cost[k] < c2) { c2 = cost[k]; k2 = k; }
                const bool near = !skip && c2 - cbv <= 0x1p-18f * fabsf(cbv);
                if (__ballot(near) == 0) {
                    idx = pick(kstar);
                } else {
                    const int i1 = pick(kstar);
                    const int i2 = pick(k2);
                    __asm__ volatile("" ::: "memory");
                    float xr[8], wr[8];
                    load_group(xb, wblk, g, skip, xr, wr);
                    const double dd = (double)d;
                    double e1 = group_error64(xr, wr, neg, sgrid + entry_off<kChunk>(i1),
                                              dd * (double)(2 * kstar + 1));
                    double e2 = group_error64(xr, wr, neg, sgrid + entry_off<kChunk>(i2),
                                              dd * (double)(2 * k2 + 1));
                    e1 += __shfl_xor(e1, 1);        // the other group of the scale group
                    e2 += __shfl_xor(e2, 1);
                    const bool take2 = near && (e2 < e1 || (e2 == e1 && k2 < kstar));
                    idx = take2 ? i2 : i1;
                    if (take2) kstar = k2;
                }
            }
            const int kodd = __shfl_xor(kstar, 2);
            const uint32_t code = (uint32_t)idx | ((uint32_t)(neg & 0x7f) << 9);
            if (!skip && kb == 0) {
                uint8_t* ob = sout + slot * kBlockBytes;
                ob[2 + 2 * g] = (uint8_t)(code & 0xff);
                ob[3 + 2 * g] = (uint8_t)(code >> 8);
                if ((g & 3) == 0) ob[66 + (m >> 1)] = (uint8_t)(kstar | (kodd << 4));
                if (g == 0) {
                    ob[0] = (uint8_t)(dh & 0xff);
                    ob[1] = (uint8_t)(dh >> 8);
                }
            }
            if (kMode == kModeFake && kb == 0) {
                // The decoded group, d*(2k+1)*sign*q with the payload's fields
                // (the 8th sign from even parity of the 7-bit mask; a zero
                // block decodes as the all-zero payload does; a rejected block
                // is written as zeros).
                const uint32_t cz = skip ? 0u : code;
                const int kz = skip ? 0 : kstar;
                const float sk = f16_bits_to_f32(skip ? 0u : dh) * (float)(2 * kz + 1);
                const uint32_t mask = cz >> 9;
                const uint32_t signs = mask | ((__popc(mask) & 1u) << 7);
                const float* q = sgrid + entry_off<kChunk>((int)(cz & 0x1ffu));
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v[j] = bad_block ? 0.0f : (((signs >> j) & 1u) ? -sk : sk) * q[j];
                float4* o = reinterpret_cast<float4*>(a.xhat + blk * kBlockElems + g * 8);
                o[0] = make_float4(v[0], v[1], v[2], v[3]);
                o[1] = make_float4(v[4], v[5], v[6], v[7]);
            }
        } else {
            // Top-C local scales by (cost, k); a zero scale makes every choice
            // decode to zero with entry 0 and no signs, so the order is k = 0, 1, ...
            const int C = a.top_c;
            float xo[8], wo[8];
            load_group(xb, wblk, g, bad_block, xo, wo);   // the original values
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
                int idx = pick(kr);
                int msk = neg & 0x7f;
                if (zero_scale) { idx = 0; msk = 0; }
                if (kb == 0) {
                    const int64_t base = (blk * 16 + m) * C + r;     // [block][m][r]
                    float ev[8];
                    if (bad_block) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) ev[j] = 0.0f;
                    } else if (grid_exact) {
                        // xhat exact in fp32: d*(2k+1) has at most 16
                        // significant bits and a bf16-exact q at most 8, so
                        // the product has at most 24; one rounding of xhat - x.
                        const float sk = d * (float)(2 * kr + 1);
                        const float* q = sgrid + entry_off<kChunk>(idx);
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float sg = (!zero_scale && ((neg >> j) & 1)) ? -sk : sk;
                            ev[j] = sg * q[j] - xo[j];
                        }
                    } else {
                        // xhat in fp64 (exact: d*(2k+1) has at most 16
                        // significant bits), one rounding of xhat - x to fp32.
                        const double sk = (double)d * (double)(2 * kr + 1);
                        const float* q = sgrid + entry_off<kChunk>(idx);
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const double sg = (!zero_scale && ((neg >> j) & 1)) ? -sk : sk;
                            ev[j] = (float)(sg * (double)q[j] - (double)xo[j]);
                        }
                    }
                    float4* ep = reinterpret_cast<float4*>(a.cand_err + base * 16 + h * 8);
                    ep[0] = make_float4(ev[0], ev[1], ev[2], ev[3]);
                    ep[1] = make_float4(ev[4], ev[5], ev[6], ev[7]);
                    if (h == 0) a.cand_choice[base] = kr;
                    if (a.cand_codes)
                        a.cand_codes[base * 2 + h] = bad_block ? (uint16_t)0 : (uint16_t)(idx | (msk << 9));
                }
            }
        }
    }
    if (!kCandidates && a.out) {
        // Copy the staged payloads out and clear what was copied (each word
        // by the thread that copied it) for the next set.
        __syncthreads();
        const int64_t first = set * kBlocksPerWG;
        const int64_t left = a.g.nblocks - first;
        const int nb = left < kBlocksPerWG ? (int)left : kBlocksPerWG;
        for (int k = 0; k < kPayloads; ++k) {
            uint16_t* o16 = reinterpret_cast<uint16_t*>(a.out + (k * a.g.nblocks + first) * kBlockBytes);
            uint16_t* s16 = sout16 + k * kBlocksPerWG * (kBlockBytes / 2);
            // An opaque copy of the thread index: the offsets derived from it are
            // recomputed here rather than held (and spilled) across the sets.
            int t0 = tid;
            __asm__ volatile("" : "+v"(t0));
            for (int i = t0; i < nb * (kBlockBytes / 2); i += kThreads) {
                o16[i] = s16[i];
                s16[i] = 0;
            }
        }
    }
    }
}

// ---------------------------------------------------------------------------
// Payload encode in 32 x 32 matrix tiles: a wave owns a whole block.
//
// v_mfma_f32_32x32x16_bf16 takes the 32 groups of the block as the 32 columns
// (lane l: column l%32) and 32 grid entries as the rows; the lane holds 16 of
// the rows (8*(v/4) + 4*(l/32) + v%4, v = 0..15), so each group is covered by
// two lanes instead of four, and the per-group work outside the sweep (signs,
// split, costs, choice, packing) is repeated twice instead of four times.  K
// is 16 per product: the three bf16 parts of the group side go in two
// products per output (parts 0 and 1 in the lanes' two K halves, then part 2
// and zeros).  The payload is written straight from the lanes (coalesced
// 16-bit codes), so waves never wait for each other after the grid staging.
// ---------------------------------------------------------------------------
constexpr int kWTile = 32;                 // entries per wide tile
constexpr int kWChunkTiles = 2;            // wide tiles per tracking chunk
constexpr int kWChunk = kWTile * kWChunkTiles;

// The 16 keys (2k+1)*N + P' of the lane's 16 entries folded into the minima
// (a tree of three-input minima: 8 per local scale).
__device__ __forceinline__ void fold_wide(const v16f& pn, const v16f& nn, float (&best)[16])
{
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const float mk = (float)(2 * k + 1);
        float key[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) key[v] = __builtin_fmaf(nn[v], mk, pn[v]);
        const float a0 = fminf(fminf(key[0], key[1]), key[2]);
        const float a1 = fminf(fminf(key[3], key[4]), key[5]);
        const float a2 = fminf(fminf(key[6], key[7]), key[8]);
        const float a3 = fminf(fminf(key[9], key[10]), key[11]);
        const float a4 = fminf(fminf(key[12], key[13]), key[14]);
        const float a5 = fminf(fminf(key[15], best[k]), a0);
        best[k] = fminf(fminf(fminf(fminf(a1, a2), a3), a4), a5);
    }
}

// After chunk ch: record ch for every minimum it lowered, against the
// snapshot of the minima kept in LDS (four float4 per lane).
__device__ __forceinline__ void track_chunk_lds(int ch, const float (&best)[16], float4* snap,
                                                uint32_t (&chunk_of)[2])
{
    const uint32_t chrep = (uint32_t)ch * 0x11111111u;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const float4 o = snap[q4 * kThreads];
        const float old[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = 4 * q4 + i;
            const uint32_t msk = best[k] < old[i] ? (0xfu << (4 * (k & 7))) : 0u;
            chunk_of[k >> 3] = (chunk_of[k >> 3] & ~msk) | (chrep & msk);
        }
        snap[q4 * kThreads] = make_float4(best[4 * q4], best[4 * q4 + 1], best[4 * q4 + 2], best[4 * q4 + 3]);
    }
}

// Entry of lane row v (0..15) of wide tile t for the lane half hl.
__device__ __forceinline__ int wide_entry(int t, int hl, int v)
{
    return kWTile * t + 8 * (v >> 2) + 4 * hl + (v & 3);
}

// VALU rescan for local scale k over rows v0 .. v0+nv-1 of half hs in both
// tiles of chunk `chunk`: the lowest entry with the least key.
__device__ __forceinline__ int rescan_wide(const float* __restrict__ sg, int chunk, int hs, int v0,
                                           int nv, int k, const float (&wxs)[8],
                                           const float (&w)[8], float inv_d, float* key_out)
{
    const float mk = (float)(2 * k + 1);
    int idx = -1;
    float vbest = 0.0f;
    for (int tt = 0; tt < kWChunkTiles; ++tt) {
        for (int v = v0; v < v0 + nv; ++v) {
            const int e = wide_entry(chunk * kWChunkTiles + tt, hs, v);
            const float2* p = reinterpret_cast<const float2*>(sg + entry_off<kWChunk>(e));
            float q[8], q2[8];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float2 u = p[t], u2 = p[4 + t];
                q[2 * t] = u.x; q[2 * t + 1] = u.y;
                q2[2 * t] = u2.x; q2[2 * t + 1] = u2.y;
            }
            float P = 0.0f, N = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                P = __builtin_fmaf(wxs[j], q[j], P);
                N = __builtin_fmaf(w[j], q2[j], N);
            }
            const float key = __builtin_fmaf(N, mk, (-2.0f * P) * inv_d);
            if (idx < 0 || key < vbest || (key == vbest && e < idx)) { vbest = key; idx = e; }
        }
    }
    *key_out = vbest;
    return idx;
}

template <int kDT>
__global__ __launch_bounds__(kThreads) void iq2xs_payload_wide_kernel(Iq2xsArgs a)
{
    __shared__ float sgrid[kMaxGrid * kEntryStride + 2 * (kMaxGrid / 32)];  // q[0..7], q^2[0..7]
    __shared__ uint4 sbq[kMaxGrid];                     // entry e: q[0..7] as bf16
    __shared__ uint4 sbq2[kMaxGrid];                    // entry e: q^2[0..7] as bf16
    __shared__ int sgrid_bad, sgrid_inexact;
    __shared__ float4 ssnap[4 * kThreads];              // per lane: the minima at the last chunk end
    __shared__ uint16_t sout16[kWavesPerWG * kBlockBytes / 2];    // the set's payloads

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: block pointers in SGPRs
    const int n = a.grid_size;
    const int nchunks = (n + kWChunk - 1) / kWChunk;
    const int npad = nchunks * kWChunk;

    if (tid == 0) { sgrid_bad = 0; sgrid_inexact = 0; }
    for (int i = tid; i < kWavesPerWG * kBlockBytes / 2; i += kThreads) sout16[i] = 0;
    __syncthreads();
    {
        int bad = 0, inexact = 0;
        for (int i = tid; i < npad * 4; i += kThreads) {
            const int e = i >> 2, t = i & 3;
            const int src = e < n ? e : n - 1;
            const float a0 = a.grid[8 * src + 2 * t], a1 = a.grid[8 * src + 2 * t + 1];
            bad |= !(a0 >= 0.0f && finite_f32(a0) && a1 >= 0.0f && finite_f32(a1));
            float2* ge = reinterpret_cast<float2*>(sgrid + entry_off<kWChunk>(e));
            ge[t] = make_float2(a0, a1);
            ge[4 + t] = make_float2(a0 * a0, a1 * a1);
            inexact |= !(bf16_exact_with_square(a0) && bf16_exact_with_square(a1));
            reinterpret_cast<uint32_t*>(sbq)[i] = bf16_bits(a0) | (bf16_bits(a1) << 16);
            reinterpret_cast<uint32_t*>(sbq2)[i] = bf16_bits(a0 * a0) | (bf16_bits(a1 * a1) << 16);
        }
        if (bad) sgrid_bad = 1;
        if (inexact) sgrid_inexact = 1;
    }
    __syncthreads();
    const bool grid_bad = sgrid_bad != 0;
    const bool grid_exact = sgrid_inexact == 0;     // workgroup-uniform
    if (grid_bad && tid == 0) report(a.status, IQ_ERR_GRID);

    // Persistent workgroups: the grid is staged once, then each workgroup
    // takes every gridDim.x-th set of 16 blocks, a block per wave; the set's
    // payloads are staged in LDS and stored together (whole cache lines).
    const int64_t nsets = (a.g.nblocks + kWavesPerWG - 1) / kWavesPerWG;
    for (int64_t set = blockIdx.x; set < nsets; set += gridDim.x) {
    if (set != blockIdx.x) __syncthreads();     // the previous set's payloads are out
    const int64_t blk = set * kWavesPerWG + wave;
    if (blk < a.g.nblocks) {                    // wave-uniform
        // The lane's indices, formed in every block from an opaque copy of
        // the lane number: offsets derived from them are recomputed here
        // rather than held (and spilled) across the blocks.
        int ln = lane;
        __asm__ volatile("" : "+v"(ln));
        const int g = ln & 31;              // group in block = matrix column
        const int hl = ln >> 5;             // K half of the operands / row half of the result
        const int m = g >> 1;               // scale group
        const int64_t bt = blk / a.g.blocks_per_batch;
        const int64_t cb = blk % a.g.blocks_per_row;
        const WeightBlock<kDT> xb(a.w, blk);
        const float* wblk = a.imp ? a.imp + bt * a.g.cols + cb * kBlockElems : nullptr;

        int err = 0;
        float amax = 0.0f;
        {
            const float4 xv = xb.quad(lane);
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
        if (err) report(a.status, err);
        const bool block_bad = __ballot(err != 0) != 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));

        uint32_t dh;
        if (a.scales) {
            dh = (uint32_t)a.scales[blk];
        } else {
            const float t = amax / 155.0f;
            const float u = t * 0.61f;
            dh = f32_to_f16_bits(u);
        }
        const bool scale_bad = ((dh & 0x7c00u) == 0x7c00u) || ((dh & 0x8000u) && (dh & 0x7fffu));
        dh &= 0x7fffu;
        if (scale_bad && !block_bad && lane == 0) report(a.status, IQ_ERR_SCALE_RANGE);
        dh = __builtin_amdgcn_readfirstlane(dh);           // the same in every lane
        const float d = scale_bad ? 0.0f : f16_bits_to_f32(dh);

        bool choice_bad = false;
        if (a.choices) {
            int ln = lane;                  // opaque: the address is formed here, not hoisted
            __asm__ volatile("" : "+v"(ln));
            const int cv = ln < 16 ? a.choices[blk * 16 + ln] : 0;
            const bool bad = cv < 0 || cv > 15;
            if (bad) report(a.status, IQ_ERR_ARG);
            choice_bad = __ballot(bad) != 0;
        }
        const bool bad_block = grid_bad || block_bad || scale_bad || choice_bad;
        const bool zero_scale = dh == 0u;
        const bool skip = bad_block || zero_scale;

        float x[8], w[8];
        load_group(xb, wblk, g, skip, x, w);
        const int neg = group_signs(x, w);
        const float inv_d = skip ? 1.0f : 1.0f / d;

        float best[16];
        uint32_t chunk_of[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < 16; ++k) best[k] = __builtin_inff();
        float4* snap = ssnap + tid;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) snap[q4 * kThreads] = make_float4(best[0], best[0], best[0], best[0]);
        const v16f zero16 = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f,
                             0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        if (grid_exact) {
            // The lane's K half: part hl of the exact three-way bf16 split of
            // -2*(w*sign*x)/d and of w (first product), part 2 or zeros
            // (second product).
            uint32_t hp1[8], hp2[8], hw1[8], hw2[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float v = w[j] * x[j];
                if ((neg >> j) & 1) v = -v;
                v = -2.0f * (v * inv_d);
                hp1[j] = split_part(v, hl);
                hp2[j] = hl == 0 ? split_part(v, 2) : 0u;
                hw1[j] = split_part(w[j], hl);
                hw2[j] = hl == 0 ? split_part(w[j], 2) : 0u;
            }
            const v8bf opp1 = as_v8bf(make_uint4(hp1[0] | (hp1[1] << 16), hp1[2] | (hp1[3] << 16),
                                                 hp1[4] | (hp1[5] << 16), hp1[6] | (hp1[7] << 16)));
            const v8bf opp2 = as_v8bf(make_uint4(hp2[0] | (hp2[1] << 16), hp2[2] | (hp2[3] << 16),
                                                 hp2[4] | (hp2[5] << 16), hp2[6] | (hp2[7] << 16)));
            const v8bf opw1 = as_v8bf(make_uint4(hw1[0] | (hw1[1] << 16), hw1[2] | (hw1[3] << 16),
                                                 hw1[4] | (hw1[5] << 16), hw1[6] | (hw1[7] << 16)));
            const v8bf opw2 = as_v8bf(make_uint4(hw2[0] | (hw2[1] << 16), hw2[2] | (hw2[3] << 16),
                                                 hw2[4] | (hw2[5] << 16), hw2[6] | (hw2[7] << 16)));
            for (int ch = 0; ch < nchunks; ++ch) {
                for (int tt = 0; tt < kWChunkTiles; ++tt) {
                    const int e = (ch * kWChunkTiles + tt) * kWTile + g;
                    const v8bf aq = as_v8bf(sbq[e]), aq2 = as_v8bf(sbq2[e]);
                    const v16f pn = mfma32(aq, opp2, mfma32(aq, opp1, zero16));
                    const v16f nn = mfma32(aq2, opw2, mfma32(aq2, opw1, zero16));
                    fold_wide(pn, nn, best);
                }
                track_chunk_lds(ch, best, snap, chunk_of);
            }
        } else {
            // fp32 operands (v_mfma_f32_32x32x2_f32, K = 2): product s takes
            // elements 2s + hl of the group and of the entries.
            float bp[4], bw[4];
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int j = 2 * s2 + hl;
                float v = w[j] * x[j];
                if ((neg >> j) & 1) v = -v;
                bp[s2] = -2.0f * (v * inv_d);
                bw[s2] = w[j];
            }
            for (int ch = 0; ch < nchunks; ++ch) {
                for (int tt = 0; tt < kWChunkTiles; ++tt) {
                    const int e = (ch * kWChunkTiles + tt) * kWTile + g;
                    const float* q = sgrid + entry_off<kWChunk>(e);
                    v16f pn = zero16, nn = zero16;
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) {
                        pn = __builtin_amdgcn_mfma_f32_32x32x2f32(q[2 * s2 + hl], bp[s2], pn, 0, 0, 0);
                        nn = __builtin_amdgcn_mfma_f32_32x32x2f32(q[8 + 2 * s2 + hl], bw[s2], nn, 0, 0, 0);
                    }
                    fold_wide(pn, nn, best);
                }
                track_chunk_lds(ch, best, snap, chunk_of);
            }
        }

        // The values, the signs and the forced choice again, rebuilt from
        // memory rather than held through the sweep.
        __asm__ volatile("" ::: "memory");
        load_group(xb, wblk, g, skip, x, w);
        const int neg2 = group_signs(x, w);
        const int forced = (a.choices && !choice_bad) ? a.choices[blk * 16 + m] : -1;
        float wxs[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float wx = w[j] * x[j];
            wxs[j] = ((neg2 >> j) & 1) ? -wx : wx;
        }

        // Scale-group costs: the lesser minimum of each group's two lanes,
        // summed over the two groups, times 2k+1.
        float cost[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            float v = fminf(best[k], __shfl_xor(best[k], 32));
            cost[k] = (float)(2 * k + 1) * (v + quad_xchg<kQuadXor1>(v));
        }

        // Entry of local scale k for this lane's group: the lane of the
        // column whose minimum is least holds it; both lanes rescan half of
        // its chunk's entries (lowest entry of least key).  With equal minima
        // in the two lanes of any column, every lane rescans its own entries
        // and the lane of least minimum, then lowest entry, wins.
        auto pick = [&](int k) -> int {
            float lm = best[0];
#pragma unroll
            for (int c = 1; c < 16; ++c)
                if (k == c) lm = best[c];
            const int tchunk = (int)((chunk_of[k >> 3] >> (4 * (k & 7))) & 0xfu);
            const float om = __shfl_xor(lm, 32);
            const bool tie = __ballot(om == lm) != 0;                // wave-uniform
            int idx;
            float key;
            if (!tie) {
                const int hs = (om < lm) ? (hl ^ 1) : hl;             // holder half
                const int tch = __shfl(tchunk, g + 32 * hs);
                idx = rescan_wide(sgrid, tch, hs, 8 * hl, 8, k, wxs, w, inv_d, &key);
                const float ok = __shfl_xor(key, 32);
                const int oi = __shfl_xor(idx, 32);
                if (ok < key || (ok == key && oi < idx)) { key = ok; idx = oi; }
            } else {
                idx = rescan_wide(sgrid, tchunk, hl, 0, 16, k, wxs, w, inv_d, &key);
                const int oi = __shfl_xor(idx, 32);
                if (om < lm || (om == lm && oi < idx)) idx = oi;
            }
            return idx < n ? idx : n - 1;
        };

        int kstar = 0;
        float cbv = cost[0];
#pragma unroll
        for (int k = 1; k < 16; ++k)
            if (cost[k] < cbv) { cbv = cost[k]; kstar = k; }
        int idx;
        if (forced >= 0) {                      // wave-uniform
            kstar = forced;
            idx = pick(kstar);
        } else {
            int k2 = kstar == 0 ? 1 : 0;
            float c2 = cost[k2];
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if (k != kstar && cost[k] < c2) { c2 = cost[k]; k2 = k; }
            const bool near = !skip && c2 - cbv <= 0x1p-18f * fabsf(cbv);
            if (__ballot(near) == 0) {
                idx = pick(kstar);
            } else {
                const int i1 = pick(kstar);
                const int i2 = pick(k2);
                __asm__ volatile("" ::: "memory");
                float xr[8], wr[8];
                load_group(xb, wblk, g, skip, xr, wr);
                const double dd = (double)d;
                double e1 = group_error64(xr, wr, neg2, sgrid + entry_off<kWChunk>(i1),
                                          dd * (double)(2 * kstar + 1));
                double e2 = group_error64(xr, wr, neg2, sgrid + entry_off<kWChunk>(i2),
                                          dd * (double)(2 * k2 + 1));
                e1 += quad_xchg<kQuadXor1>(e1);  // the other group of the scale group
                e2 += quad_xchg<kQuadXor1>(e2);
                const bool take2 = near && (e2 < e1 || (e2 == e1 && k2 < kstar));
                idx = take2 ? i2 : i1;
                if (take2) kstar = k2;
            }
        }
        const int kodd = quad_xchg<kQuadXor2>(kstar);
        const uint32_t code = (uint32_t)idx | ((uint32_t)(neg2 & 0x7f) << 9);
        if (hl == 0 && !skip) {
            // d, the 32 codes and the 16 scale nibbles into the wave's staged
            // block (a rejected or zero-scale block stays all zeros).
            uint8_t* ob = reinterpret_cast<uint8_t*>(sout16) + wave * kBlockBytes;
            ob[2 + 2 * g] = (uint8_t)(code & 0xff);
            ob[3 + 2 * g] = (uint8_t)(code >> 8);
            if ((g & 3) == 0) ob[66 + (g >> 2)] = (uint8_t)(kstar | (kodd << 4));
            if (g == 0) {
                ob[0] = (uint8_t)(dh & 0xff);
                ob[1] = (uint8_t)(dh >> 8);
            }
        }
    }
    if (a.out) {
        // Copy the set's payloads out and clear what was copied (each word
        // by the thread that copied it) for the next set.
        __syncthreads();
        const int64_t first = set * kWavesPerWG;
        const int64_t left = a.g.nblocks - first;
        const int nb = left < kWavesPerWG ? (int)left : kWavesPerWG;
        uint16_t* o16 = reinterpret_cast<uint16_t*>(a.out + first * kBlockBytes);
        int t0 = tid;
        __asm__ volatile("" : "+v"(t0));
        for (int i = t0; i < nb * (kBlockBytes / 2); i += kThreads) {
            o16[i] = sout16[i];
            sout16[i] = 0;
        }
    }
    }
}

// One workgroup per compute unit (the LDS holds one), or one per set of 16
// blocks when there are fewer sets.
unsigned persistent_wgs(const BlockGeom& g)
{
    const int64_t sets = (g.nblocks + kBlocksPerWG - 1) / kBlocksPerWG;
    return (unsigned)(sets < g.cus ? sets : g.cus);
}

template <int kDT>
hipError_t launch_mode(const Iq2xsArgs& a, int mode, hipStream_t stream)
{
    const unsigned wgs = persistent_wgs(a.g);
    if (mode == kModeEvery)
        hipLaunchKernelGGL((iq2xs_kernel<kModeEvery, kDT>), dim3(wgs), dim3(kThreads), 0, stream, a);
    else if (mode == kModeFake)
        hipLaunchKernelGGL((iq2xs_kernel<kModeFake, kDT>), dim3(wgs), dim3(kThreads), 0, stream, a);
    else if (mode == kModeCandidates)
        hipLaunchKernelGGL((iq2xs_kernel<kModeCandidates, kDT>), dim3(wgs), dim3(kThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((iq2xs_payload_wide_kernel<kDT>), dim3(wgs), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_dtype(const Iq2xsArgs& a, int wdtype, int mode, hipStream_t stream)
{
    switch (wdtype) {
    case IQ_DTYPE_BF16: return launch_mode<IQ_DTYPE_BF16>(a, mode, stream);
    case IQ_DTYPE_F16: return launch_mode<IQ_DTYPE_F16>(a, mode, stream);
    case IQ_DTYPE_F64: return launch_mode<IQ_DTYPE_F64>(a, mode, stream);
    default: return launch_mode<IQ_DTYPE_F32>(a, mode, stream);
    }
}

}  // namespace

hipError_t launch_iq2xs_encode(int wdtype, const void* w, const float* imp, const float* grid,
                               int grid_size, const uint16_t* scales, const int32_t* choices,
                               uint8_t* out, float* xhat, int mode, int32_t* status,
                               const BlockGeom& g, hipStream_t stream)
{
    Iq2xsArgs a{w, imp, grid, scales, choices, out, xhat, nullptr, nullptr, nullptr, status, g,
                grid_size, 0};
    return launch_dtype(a, wdtype, mode, stream);
}

hipError_t launch_iq2xs_candidates(int wdtype, const void* w, const float* imp, const float* grid,
                                   int grid_size, int top_c, float* cand_err, int32_t* cand_choice,
                                   uint16_t* cand_codes, int32_t* status, const BlockGeom& g,
                                   hipStream_t stream)
{
    Iq2xsArgs a{w, imp, grid, nullptr, nullptr, nullptr, nullptr, cand_err, cand_choice,
                cand_codes, status, g, grid_size, top_c};
    return launch_dtype(a, wdtype, kModeCandidates, stream);
}

}  // namespace iqk
