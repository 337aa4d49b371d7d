// iq2xs_encode.hip -- importance-weighted codebook search for IQ2_XS on
// gfx950, with the epilogues of every output: the packed payload, the payload
// under every choice, the fake quant, and the top-C candidates that feed the
// local-Hessian choice search.
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
// N for a tile of entries x groups are two [entries x 8] x [8 x groups]
// products on the matrix cores.  When every grid value and its square are
// exact in bf16 (the odd-integer grids {1,3,5} among them), the group side is
// split in three bf16 parts whose sum is the fp32 value, so the bf16 products
// are exact; any other magnitude grid is used as given with fp32 operands
// (four times the matrix-core time).  Dividing by d, the key of local scale k
// is (2k+1)*N - 2P/d: one FMA with a literal multiplier; the choice cost of a
// scale group is (2k+1) times the sum of its two groups' minima.
//
// One kernel, iq2xs_wide_kernel, runs every output in 32 x 32 matrix tiles,
// v_mfma_f32_32x32x16_bf16, with a wave per block: matrix column = group, two
// lanes per column, each holding 16 entries of every 32-entry tile.
// Persistent 1024-thread workgroups (one per CU) stage the grid once in LDS
// (q and q^2 as bf16 operands, and a padded fp32 copy for the rescans).
// Value-only minima (v_min3); each lane records the chunk that last lowered
// each minimum; the lane of each column whose matrix-core minimum is least is
// found, and the two lanes of the column split its entries of that chunk and
// rescan them on the VALU (lowest entry of least key).
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace iqk {
namespace {


constexpr int kWavesPerWG = 16;
constexpr int kThreads = kWave * kWavesPerWG;        // 1024
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
// padded to 18 floats (at 16, entries 4 apart would share their LDS banks).
constexpr int kEntryStride = 18;
// Tracking chunks are 32 or 64 entries, a multiple of the 64 LDS banks apart
// at that stride, so lanes rescanning different chunks would all hit the same
// banks; every chunk therefore starts 2 floats later than the stride alone
// puts it.
template <int kChunk>
__device__ __forceinline__ int entry_off(int e) { return kEntryStride * e + 2 * (e / kChunk); }

// ---------------------------------------------------------------------------
// The search in 32 x 32 matrix tiles: a wave owns a whole block.
//
// v_mfma_f32_32x32x16_bf16 takes the 32 groups of the block as the 32 columns
// (lane l: column l%32) and 32 grid entries as the rows; the lane holds 16 of
// the rows (8*(v/4) + 4*(l/32) + v%4, v = 0..15), so each group is covered by
// the two lanes of its column, which share the per-group work outside the
// sweep (signs, split, costs, choice, packing).  K is 16 per product: the
// three bf16 parts of the group side go in two products per output (parts 0
// and 1 in the lanes' two K halves, then part 2 and zeros).  A set's payloads
// are staged in LDS and stored together after a workgroup barrier (whole
// cache lines); the candidates are written straight from the lanes.
// ---------------------------------------------------------------------------
constexpr int kWTile = 32;                 // entries per wide tile
constexpr int kWChunkTiles = 2;            // wide tiles per tracking chunk

// The 16 keys (2k+1)*N + P' of the lane's 16 entries folded into the minima.
// kChain false: a tree of three-input minima, 8 per local scale.  kChain
// true: each minimum a chain of three-input minima over pairs of keys, the
// chains of two local scales alternating, so that each wave's instruction
// stream is two key FMAs and one minimum throughout (the dual issue pairs an
// FMA of one wave with a minimum of another, never two minima).  Which is
// faster depends on the epilogue the compiler schedules around the sweep:
// measured, the chains help the fake quant (5 %) and not the other modes.
template <bool kChain>
__device__ __forceinline__ void fold_wide(const v16f& pn, const v16f& nn, float (&best)[16])
{
    if constexpr (kChain) {
#pragma unroll
        for (int k = 0; k < 16; k += 2) {
            const float ma = (float)(2 * k + 1), mb = (float)(2 * k + 3);
            float ba = best[k], bb = best[k + 1];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float a0 = __builtin_fmaf(nn[r], ma, pn[r]);
                const float a1 = __builtin_fmaf(nn[r + 1], ma, pn[r + 1]);
                ba = fminf(fminf(ba, a0), a1);
                __builtin_amdgcn_sched_barrier(0);
                const float b0 = __builtin_fmaf(nn[r], mb, pn[r]);
                const float b1 = __builtin_fmaf(nn[r + 1], mb, pn[r + 1]);
                bb = fminf(fminf(bb, b0), b1);
                __builtin_amdgcn_sched_barrier(0);
            }
            best[k] = ba;
            best[k + 1] = bb;
        }
    } else {
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

// VALU rescan for local scale k over rows v0 .. v0+kNV-1 (v0 a multiple of 4)
// of half hs in the kCT tiles of chunk `chunk`: the lowest entry with the
// least key.  The lane visits its entries in increasing order, so a strict
// comparison keeps the lowest of equal keys; the entry offsets inside the
// chunk are constants of the unrolled loop.
template <int kCT, int kNV>
__device__ __forceinline__ int rescan_wide(const float* __restrict__ sg, int chunk, int hs, int v0,
                                           int k, const float (&wxs)[8], const float (&w)[8],
                                           float inv_d, float* key_out)
{
    const float mk = (float)(2 * k + 1);
    // entry e0 + de, de = 32*tile + 8*(i/4) + i%4 for row v0 + i
    const int e0 = kWTile * kCT * chunk + 4 * hs + 8 * (v0 >> 2);
    const float* base = sg + kEntryStride * e0 + 2 * chunk;      // entry_off<32*kCT>(e0)
    int idx = e0;
    float vbest = __builtin_inff();
#pragma unroll
    for (int tt = 0; tt < kCT; ++tt) {
#pragma unroll
        for (int i = 0; i < kNV; ++i) {
            const int de = kWTile * tt + 8 * (i >> 2) + (i & 3);
            const float2* p = reinterpret_cast<const float2*>(base + kEntryStride * de);
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
            const bool better = key < vbest;
            vbest = better ? key : vbest;
            idx = better ? e0 + de : idx;
        }
    }
    *key_out = vbest;
    return idx;
}

// The same rescan with the same keys, for a pick whose holder lane is known:
// it reads only q from the LDS (q^2 formed in fp32 is the table's value
// exactly), and it requests the four entries of a row quad before it forms
// their keys, so a pick waits for the LDS kNV/4 times rather than kNV times.
template <int kCT, int kNV>
__device__ __forceinline__ int rescan_quads(const float* __restrict__ sg, int chunk, int hs, int v0,
                                            int k, const float (&wxs)[8], const float (&w)[8],
                                            float inv_d, float* key_out)
{
    const float mk = (float)(2 * k + 1);
    const int e0 = kWTile * kCT * chunk + 4 * hs + 8 * (v0 >> 2);
    const float* base = sg + kEntryStride * e0 + 2 * chunk;      // entry_off<32*kCT>(e0)
    int idx = e0;
    float vbest = __builtin_inff();
#pragma unroll
    for (int tt = 0; tt < kCT; ++tt) {
#pragma unroll
        for (int r4 = 0; r4 < kNV / 4; ++r4) {
            float q[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int de = kWTile * tt + 8 * r4 + i;
                const float2* p = reinterpret_cast<const float2*>(base + kEntryStride * de);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float2 u = p[t];
                    q[i][2 * t] = u.x;
                    q[i][2 * t + 1] = u.y;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int de = kWTile * tt + 8 * r4 + i;
                float P = 0.0f, N = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    P = __builtin_fmaf(wxs[j], q[i][j], P);
                    N = __builtin_fmaf(w[j], q[i][j] * q[i][j], N);
                }
                const float key = __builtin_fmaf(N, mk, (-2.0f * P) * inv_d);
                const bool better = key < vbest;
                vbest = better ? key : vbest;
                idx = better ? e0 + de : idx;
            }
        }
    }
    *key_out = vbest;
    return idx;
}

// kMode: kModePayload, kModeEvery, kModeFake or kModeCandidates; kDT: the
// weight's iq_dtype_t.
template <int kMode, int kDT>
__global__ __launch_bounds__(kThreads) void iq2xs_wide_kernel(Iq2xsArgs a)
{
    constexpr bool kCand = kMode == kModeCandidates;
    // Tiles per tracking chunk: 2 (64 entries) for one pick per group; the
    // candidates pick top_c local scales per group, each rescanning one
    // lane-half of a chunk, so their chunks are one tile (32 entries): twice
    // the tracking in the sweep, half the rescan per pick.
    constexpr bool kEvery = kMode == kModeEvery;
    constexpr int kNP = kEvery ? 16 : 1;           // payloads per block
    constexpr int kCT = (kCand || kEvery) ? 1 : kWChunkTiles;
    constexpr int kCh = kWTile * kCT;
    __shared__ float sgrid[kMaxGrid * kEntryStride + 2 * (kMaxGrid / 32)];  // q[0..7], q^2[0..7]
    __shared__ uint4 sbq[kMaxGrid];                     // entry e: q[0..7] as bf16
    __shared__ uint4 sbq2[kMaxGrid];                    // entry e: q^2[0..7] as bf16
    __shared__ int sgrid_bad, sgrid_inexact;
    __shared__ float4 ssnap[4 * kThreads];              // per lane: the minima at the last chunk end
    __shared__ uint16_t sout16[kCand ? 1 : kNP * kWavesPerWG * kBlockBytes / 2];    // the set's payloads
    // candidates: per wave and scale group, the 16 local scales and their
    // costs in (cost, k) order
    __shared__ float srank_cost[kCand ? kWavesPerWG * 16 * 16 : 1];
    __shared__ uint8_t srank_k[kCand ? kWavesPerWG * 16 * 16 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: block pointers in SGPRs
    const int n = a.grid_size;
    const int nchunks = (n + kCh - 1) / kCh;
    const int npad = nchunks * kCh;

    if (tid == 0) { sgrid_bad = 0; sgrid_inexact = 0; }
    if (!kCand)
        for (int i = tid; i < kNP * kWavesPerWG * kBlockBytes / 2; i += kThreads) sout16[i] = 0;
    __syncthreads();
    {
        int bad = 0, inexact = 0;
        for (int i = tid; i < npad * 4; i += kThreads) {
            const int e = i >> 2, t = i & 3;
            const int src = e < n ? e : n - 1;
            const float a0 = a.grid[8 * src + 2 * t], a1 = a.grid[8 * src + 2 * t + 1];
            bad |= !(a0 >= 0.0f && finite_f32(a0) && a1 >= 0.0f && finite_f32(a1));
            float2* ge = reinterpret_cast<float2*>(sgrid + entry_off<kCh>(e));
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
    // The candidates are written straight from the lanes.
    const int64_t nsets = (a.g.nblocks + kWavesPerWG - 1) / kWavesPerWG;
    for (int64_t set = blockIdx.x; set < nsets; set += gridDim.x) {
    if (set != blockIdx.x) __syncthreads();     // the previous set's payloads are out
    // every wave of the workgroup has a block of this set (workgroup-uniform)
    const bool set_full = (set + 1) * kWavesPerWG <= a.g.nblocks;
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
        if (!kCand && a.scales) {
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
        if (!kCand && !kEvery && a.choices) {
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
                for (int tt = 0; tt < kCT; ++tt) {
                    const int e = (ch * kCT + tt) * kWTile + g;
                    const v8bf aq = as_v8bf(sbq[e]), aq2 = as_v8bf(sbq2[e]);
                    const v16f pn = mfma32(aq, opp2, mfma32(aq, opp1, zero16));
                    const v16f nn = mfma32(aq2, opw2, mfma32(aq2, opw1, zero16));
                    fold_wide<kMode == kModeFake>(pn, nn, best);
                }
                track_chunk_lds(ch, best, snap, chunk_of);
                if (!kEvery && set_full) __syncthreads();   // the waves of a full set sweep in step
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
                for (int tt = 0; tt < kCT; ++tt) {
                    const int e = (ch * kCT + tt) * kWTile + g;
                    const float* q = sgrid + entry_off<kCh>(e);
                    v16f pn = zero16, nn = zero16;
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) {
                        pn = __builtin_amdgcn_mfma_f32_32x32x2f32(q[2 * s2 + hl], bp[s2], pn, 0, 0, 0);
                        nn = __builtin_amdgcn_mfma_f32_32x32x2f32(q[8 + 2 * s2 + hl], bw[s2], nn, 0, 0, 0);
                    }
                    fold_wide<kMode == kModeFake>(pn, nn, best);
                }
                track_chunk_lds(ch, best, snap, chunk_of);
                if (!kEvery && set_full) __syncthreads();   // the waves of a full set sweep in step
            }
        }

        // The values, the signs and the forced choice again, rebuilt from
        // memory rather than held through the sweep.
        __asm__ volatile("" ::: "memory");
        load_group(xb, wblk, g, skip, x, w);
        const int neg2 = group_signs(x, w);
        const int forced = (!kCand && !kEvery && a.choices && !choice_bad) ? a.choices[blk * 16 + m] : -1;
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
        // The snapshot in LDS holds the lane's final minima (the last chunk
        // wrote it), so best[] need not stay live through the epilogue.
        auto pick = [&](int k) -> int {
            const float lm = reinterpret_cast<const float*>(snap + (k >> 2) * kThreads)[k & 3];
            const int tchunk = (int)((chunk_of[k >> 3] >> (4 * (k & 7))) & 0xfu);
            const float om = __shfl_xor(lm, 32);
            const bool tie = __ballot(om == lm) != 0;                // wave-uniform
            int idx;
            float key;
            if (!tie) {
                const int hs = (om < lm) ? (hl ^ 1) : hl;             // holder half
                const int tch = __shfl(tchunk, g + 32 * hs);
                idx = rescan_quads<kCT, 8>(sgrid, tch, hs, 8 * hl, k, wxs, w, inv_d, &key);
                const float ok = __shfl_xor(key, 32);
                const int oi = __shfl_xor(idx, 32);
                if (ok < key || (ok == key && oi < idx)) { key = ok; idx = oi; }
            } else {
                idx = rescan_wide<kCT, 16>(sgrid, tchunk, hl, 0, k, wxs, w, inv_d, &key);
                const int oi = __shfl_xor(idx, 32);
                if (om < lm || (om == lm && oi < idx)) idx = oi;
            }
            return idx < n ? idx : n - 1;
        };

        if constexpr (kEvery) {
            // Every choice: payload k has every scale group at local scale k,
            // a pick per group and k (a rejected or zero-scale block stays all
            // zeros in every payload).
#pragma unroll 1
            for (int k = 0; k < 16; ++k) {
                const int idx = pick(k);
                const uint32_t code = (uint32_t)idx | ((uint32_t)(neg2 & 0x7f) << 9);
                if (hl == 0 && !skip) {
                    uint8_t* ob = reinterpret_cast<uint8_t*>(sout16) + (k * kWavesPerWG + wave) * kBlockBytes;
                    ob[2 + 2 * g] = (uint8_t)(code & 0xff);
                    ob[3 + 2 * g] = (uint8_t)(code >> 8);
                    if ((g & 3) == 0) ob[66 + (g >> 2)] = (uint8_t)(k | (k << 4));
                    if (g == 0) {
                        ob[0] = (uint8_t)(dh & 0xff);
                        ob[1] = (uint8_t)(dh >> 8);
                    }
                }
            }
        } else if constexpr (!kCand) {
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
                double e1 = group_error64(xr, wr, neg2, sgrid + entry_off<kCh>(i1),
                                          dd * (double)(2 * kstar + 1));
                double e2 = group_error64(xr, wr, neg2, sgrid + entry_off<kCh>(i2),
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
        if (kMode == kModeFake) {
            // The decoded group, d*(2k+1)*sign*q with the payload's fields
            // (the 8th sign from even parity of the 7-bit mask; a zero block
            // decodes as the all-zero payload does; a rejected block is
            // written as zeros), with the decode kernel's fp32 expression.
            // The two lanes of the column write four values each: one
            // 1 KiB store per wave.
            const uint32_t cz = skip ? 0u : code;
            const int kz = skip ? 0 : kstar;
            const float sk = f16_bits_to_f32(skip ? 0u : dh) * (float)(2 * kz + 1);
            const uint32_t mask = cz >> 9;
            const uint32_t signs = (mask | ((__popc(mask) & 1u) << 7)) >> (4 * hl);
            const float* q = sgrid + entry_off<kCh>((int)(cz & 0x1ffu)) + 4 * hl;
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = bad_block ? 0.0f : (((signs >> j) & 1u) ? -sk : sk) * q[j];
            reinterpret_cast<float4*>(a.xhat + blk * kBlockElems + g * 8)[hl] =
                make_float4(v[0], v[1], v[2], v[3]);
        }
        } else {
            // Top-C local scales by (cost, k); a zero scale makes every choice
            // decode to zero with entry 0 and no signs, so the order is k = 0,
            // 1, ...  Each pick rescans one lane-half of a 32-entry chunk.
            const int C = a.top_c;
            const int h = g & 1;                // group in the scale group
            // The scale group's fp64 error under local scale k with this
            // lane's entry (and the other group's, one column away).
            auto cost64 = [&](int k, int e) -> double {
                __asm__ volatile("" ::: "memory");
                float xr[8], wr[8];
                load_group(xb, wblk, g, skip, xr, wr);
                const double v = group_error64(xr, wr, neg2, sgrid + entry_off<kCh>(e),
                                               (double)d * (double)(2 * k + 1));
                return v + quad_xchg<kQuadXor1>(v);
            };
            float xo[8], wo[8];
            load_group(xb, wblk, g, bad_block, xo, wo);   // the original values

            // The order of the 16 local scales by (cost, k), formed once: the
            // four lanes of a scale group hold the same 16 costs, and the lane
            // of slot s4 ranks k = 4*s4 .. 4*s4+3 by counting the costs below
            // each, then files k and its cost under its rank in the LDS, where
            // every lane of the group reads the order.  Equal costs (or a NaN)
            // leave the ranks short of a permutation; a wave with such a scale
            // group takes the selection below in every round instead.  A
            // zero or rejected block keeps the order 0, 1, ...
            const int s4 = h | (hl << 1);
            float* rc = srank_cost + (wave * 16 + m) * 16;
            uint8_t* rk8 = srank_k + (wave * 16 + m) * 16;
            int rmask = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float mi = s4 == 0 ? cost[i] : s4 == 1 ? cost[4 + i] : s4 == 2 ? cost[8 + i] : cost[12 + i];
                int rank = 0;
#pragma unroll
                for (int k = 0; k < 16; ++k) rank += cost[k] < mi ? 1 : 0;
                if (skip) rank = 4 * s4 + i;
                rmask |= 1 << rank;
                rc[rank] = mi;
                rk8[rank] = (uint8_t)(4 * s4 + i);
            }
            rmask |= __shfl_xor(rmask, 1);
            rmask |= __shfl_xor(rmask, 32);
            bool ordered = __ballot(rmask != 0xffff) == 0;   // wave-uniform
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

            int used = 0;
            for (int r = 0; r < C; ++r) {
                int kr = -1;
                float cr = 0.0f;
                bool near = false;
                if (ordered) {                                  // wave-uniform
                    kr = rk8[r];
                    cr = rc[r];
                    if (r + 1 < 16 && !skip) near = rc[r + 1] - cr <= 0x1p-18f * fabsf(cr);
                }
                int idx;
                if (ordered && __ballot(near) == 0) {           // wave-uniform
                    idx = pick(kr);
                } else {
                    const int kord = kr;
                    kr = -1;
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        const bool free_k = !((used >> k) & 1);
                        const bool better = zero_scale ? (kr < 0) : (kr < 0 || cost[k] < cr);
                        if (free_k && better) { kr = k; cr = cost[k]; }
                    }
                    // Unused local scales whose fp32 cost is within 2^-18 of
                    // the least's magnitude are ranked again by their fp64
                    // errors (with their own entries), the lower k on equal
                    // errors, as the payload's runner-up is.
                    uint32_t nearm = 0u;
                    if (!skip) {
#pragma unroll
                        for (int k = 0; k < 16; ++k)
                            if (!((used >> k) & 1) && k != kr && cost[k] - cr <= 0x1p-18f * fabsf(cr))
                                nearm |= 1u << k;
                    }
                    if (__ballot(nearm != 0u) != 0) {           // wave-uniform
                        idx = pick(kr);
                        double b64 = cost64(kr, idx);
                        for (int k = 0; k < 16; ++k) {
                            if (__ballot((nearm >> k) & 1u) == 0) continue;   // wave-uniform
                            const int ik = pick(k);
                            const double e = cost64(k, ik);
                            if (((nearm >> k) & 1u) && (e < b64 || (e == b64 && k < kr))) {
                                b64 = e;
                                kr = k;
                                idx = ik;
                            }
                        }
                    } else {
                        idx = pick(kr);
                    }
                    // a pick out of the filed order ends its use
                    if (ordered && __ballot(kr != kord) != 0) ordered = false;
                }
                used |= 1 << kr;
                int msk = neg2 & 0x7f;
                if (zero_scale) { idx = 0; msk = 0; }
                {
                    // The two lanes of the column write four errors each
                    // (elements 4*hl .. 4*hl+3 of the group).
                    const int64_t base = (blk * 16 + m) * C + r;     // [block][m][r]
                    const int j0 = 4 * hl;
                    float xq[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) xq[jj] = hl ? xo[4 + jj] : xo[jj];
                    float ev[4];
                    if (bad_block) {
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) ev[jj] = 0.0f;
                    } else if (grid_exact) {
                        // xhat exact in fp32: d*(2k+1) has at most 16
                        // significant bits and a bf16-exact q at most 8, so
                        // the product has at most 24; one rounding of xhat - x.
                        const float sk = d * (float)(2 * kr + 1);
                        const float* q = sgrid + entry_off<kCh>(idx) + j0;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const float sg = (!zero_scale && ((neg2 >> (j0 + jj)) & 1)) ? -sk : sk;
                            ev[jj] = sg * q[jj] - xq[jj];
                        }
                    } else {
                        // xhat in fp64 (exact: d*(2k+1) has at most 16
                        // significant bits), one rounding of xhat - x to fp32.
                        const double sk = (double)d * (double)(2 * kr + 1);
                        const float* q = sgrid + entry_off<kCh>(idx) + j0;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const double sg = (!zero_scale && ((neg2 >> (j0 + jj)) & 1)) ? -sk : sk;
                            ev[jj] = (float)(sg * (double)q[jj] - (double)xq[jj]);
                        }
                    }
                    reinterpret_cast<float4*>(a.cand_err + base * 16 + h * 8)[hl] =
                        make_float4(ev[0], ev[1], ev[2], ev[3]);
                    if (hl == 0 && h == 0) a.cand_choice[base] = kr;
                    if (hl == 0 && a.cand_codes)
                        a.cand_codes[base * 2 + h] = bad_block ? (uint16_t)0 : (uint16_t)(idx | (msk << 9));
                }
            }
        }
    }
    if (!kCand && a.out) {
        // Copy the set's payloads out (every choice: payload k of the set to
        // out[k]) and clear what was copied (each word by the thread that
        // copied it) for the next set.
        __syncthreads();
        const int64_t first = set * kWavesPerWG;
        const int64_t left = a.g.nblocks - first;
        const int nb = left < kWavesPerWG ? (int)left : kWavesPerWG;
        for (int k = 0; k < kNP; ++k) {
            uint16_t* o16 = reinterpret_cast<uint16_t*>(a.out + (k * a.g.nblocks + first) * kBlockBytes);
            uint16_t* s16 = sout16 + k * kWavesPerWG * (kBlockBytes / 2);
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

// One workgroup per compute unit (the LDS holds one), or one per set of 16
// blocks when there are fewer sets.
unsigned persistent_wgs(const BlockGeom& g)
{
    const int64_t sets = (g.nblocks + kWavesPerWG - 1) / kWavesPerWG;
    return (unsigned)(sets < g.cus ? sets : g.cus);
}

template <int kDT>
hipError_t launch_mode(const Iq2xsArgs& a, int mode, hipStream_t stream)
{
    const unsigned wgs = persistent_wgs(a.g);
    if (mode == kModeEvery)
        hipLaunchKernelGGL((iq2xs_wide_kernel<kModeEvery, kDT>), dim3(wgs), dim3(kThreads), 0,
                           stream, a);
    else if (mode == kModeFake)
        hipLaunchKernelGGL((iq2xs_wide_kernel<kModeFake, kDT>), dim3(wgs), dim3(kThreads), 0,
                           stream, a);
    else if (mode == kModeCandidates)
        hipLaunchKernelGGL((iq2xs_wide_kernel<kModeCandidates, kDT>), dim3(wgs), dim3(kThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((iq2xs_wide_kernel<kModePayload, kDT>), dim3(wgs), dim3(kThreads), 0,
                           stream, a);
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
