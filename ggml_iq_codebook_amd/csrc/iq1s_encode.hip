// iq1s_encode.hip -- importance-weighted exhaustive codebook search for IQ1_S
// and IQ1_M on gfx950, with the weighted dot products on the matrix cores.
//
// The format (NVIDIA Model-Optimizer, "Add IQ tests and release notes" #2450,
// code review; "Weight the IQ1 encoders by the square root of GPTQ's Hessian
// diagonal" #2723): a 256-value block has an fp16 scale d predicted as
// (amax/16.875)*0.61; each group of 8 values is s*(q + delta) with q one of up
// to 2048 ternary grid entries; the 4 groups of a 32-value sub-block share the
// local scale s = d*(2k+1), k = 0..7, and delta = +-1/8.  The codes minimise
// sum w*(x - s*(q+delta))^2, lowest index winning ties.  IQ1_M (the IQ1_S
// grid, 56-byte blocks) has a local scale per 16 values, a free shift per
// group and a peak-to-RMS anchor for d.
//
// For a group and a grid entry the error is, up to a constant,
//   s^2 * U(delta) - 2 s * V(delta),  U(delta) = sum w*(q+delta)^2,
//   V(delta) = sum wx*(q+delta).
// The entry side ((q+delta)^2 and q) is exact in bf16 (values like 81/64
// need 7 mantissa bits) and the group side is split into three bf16 parts
// whose sum is exactly the fp32 value, so the matrix-core products are exact
// and only the fp32 accumulation rounds.  The rest of -2V(delta),
// -2*delta*sum(wx), is the same for every entry of a group and shift, so it
// does not move the sweep's minima between entries: it is added to them once
// after the sweep.  Everything is divided by the block scale d (the V side
// carries 1/d), so the sweep key of local scale s_k = d*(2k+1) is
// (2k+1)*U - 2*sum(wx*q)/d: one FMA with a literal multiplier (v_fmamk_f32,
// two register operands, which pairs well with v_min3 in the dual-issue
// VALU); the choice cost of a sub-block is (2k+1) times the sum of its
// groups' minima (the common factor d^2 dropped).  The VALU keeps value-only
// minima (v_min3).
//
// One kernel, iq1s_payload_wide_kernel (32 x 32 tiles, a wave per block,
// described below), gives every output of both formats: the payload, the
// payload under every choice, the fake quant and the top-C candidates.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace iqk {
namespace {

constexpr int kWavesPerWG = 16;
constexpr int kThreads = kWave * kWavesPerWG;        // 1024
constexpr int kMaxGrid = 2048;
constexpr int kBlockBytes = 50;
constexpr int kBlockBytesM = 56;

struct Iq1sArgs {
    const void* w;           // weights in the storage type the kernel is built for
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

// The 8 values and importance weights of group g of a block (zeros and ones
// for a rejected block, so the sweep stays finite).
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

// A lane's group values and weights, read again from global memory after the
// sweep rather than held through it.
template <class XB>
struct GlobalGroup {
    XB xb;
    const float* wblk;
    int g;
    __device__ __forceinline__ void load(bool zero, float (&x)[8], float (&w)[8]) const
    {
        load_group(xb, wblk, g, zero, x, w);
    }
};

// ---------------------------------------------------------------------------
// The search in 32 x 32 matrix tiles: a wave owns a whole block.
//
// v_mfma_f32_32x32x16_bf16 takes the block's 32 groups as the columns and 32
// grid entries as the rows (the lane holds 16 of them: rows 8*(i/4) + 4*half
// + i%4), so each group is covered by the two lanes of its column.  A
// 1024-thread workgroup runs 16 waves, a block each; the workgroups are
// persistent (one per CU, 4 waves per SIMD) and stage the grid once in LDS.
// Two operand tables, (q+1/8)^2 and q, as bf16; per tile,
// V = -2*sum(wx*q)/d and U(+1/8) from two products each (the group side's
// three exact bf16 parts in the two K halves of the first product and the
// first K half of the second), the 8 keys of shift +1/8 folded, then
// U(-1/8) = U(+1/8) + sum(q*(-w/2)) by two more products on the same
// accumulator, and the 8 keys of shift -1/8.
// ---------------------------------------------------------------------------
constexpr int kW1Tile = 32;
constexpr int kW1ChunkTiles = 4;                       // 128-entry chunks (16 for 2048 entries)

// The 8 keys (2k+1)*U + V of the lane's 16 entries for k = 0..7 folded into
// best[kBase + k].  Each minimum is a chain of three-input minima over pairs
// of keys, and the chains of two local scales alternate, so each wave's
// instruction stream is two key FMAs and one minimum throughout: the dual
// issue pairs an FMA of one wave with a minimum of another, never two minima,
// and a stream with the minima spread evenly leaves two waves waiting on
// minima at the same time less often than one with them in runs.
template <int kBase>
__device__ __forceinline__ void fold_wide8(const v16f& u, const v16f& v, float (&best)[16])
{
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
        const float ma = (float)(2 * k + 1), mb = (float)(2 * k + 3);
        float ba = best[kBase + k], bb = best[kBase + k + 1];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float a0 = __builtin_fmaf(u[r], ma, v[r]);
            const float a1 = __builtin_fmaf(u[r + 1], ma, v[r + 1]);
            ba = fminf(fminf(ba, a0), a1);
            __builtin_amdgcn_sched_barrier(0);
            const float b0 = __builtin_fmaf(u[r], mb, v[r]);
            const float b1 = __builtin_fmaf(u[r + 1], mb, v[r + 1]);
            bb = fminf(fminf(bb, b0), b1);
            __builtin_amdgcn_sched_barrier(0);
        }
        best[kBase + k] = ba;
        best[kBase + k + 1] = bb;
    }
}

// VALU rescan for choice cs = k + 8*deltabit over rows v0 .. v0+kNV-1 (v0 a
// multiple of 4) of half hs in the tiles of chunk `chunk`: the lowest entry
// with the least key (2k+1)*U - 2V/d, recomputed in fp32 from the group's
// values and weights.  The lane visits its entries in increasing order, so a
// strict comparison keeps the lowest of equal keys; the entry offsets inside
// a tile are constants of the unrolled row loop.
template <int kNV, int kCT, class GS>
__device__ __forceinline__ int rescan_w1(const uint4* __restrict__ sq, int chunk, int hs, int v0,
                                         int cs, const GS& src, bool zero_block, float w64,
                                         float b4, float inv_d, float* key_out)
{
    float x[8], w[8];
    __asm__ volatile("" ::: "memory");
    src.load(zero_block, x, w);
    float wx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) wx[j] = w[j] * x[j];
    const float mk = (float)(2 * (cs & 7) + 1);
    const float dl = (cs >> 3) ? -0.25f : 0.25f;      // 2*delta
    const float bd = (cs >> 3) ? b4 : -b4;
    // entry e0 + de, de = 32*tile + 8*(i/4) + i%4 for row v0 + i; the table
    // holds entry e at e + e/(32*kCT) (one spare slot per chunk of kCT tiles)
    const int e0 = kW1Tile * kCT * chunk + 4 * hs + 8 * (v0 >> 2);
    const uint4* base = sq + e0 + chunk;
    int idx = e0;
    float vbest = __builtin_inff();
#pragma unroll 1
    for (int tt = 0; tt < kCT; ++tt) {
#pragma unroll
        for (int i = 0; i < kNV; ++i) {
            const int de = 8 * (i >> 2) + (i & 3);
            const uint4 u = base[kW1Tile * tt + de];
            const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
            float A = 0.0f, M = 0.0f, N = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float q = (j & 1) ? __uint_as_float(uu[j >> 1] & 0xffff0000u)
                                        : __uint_as_float(uu[j >> 1] << 16);
                A = __builtin_fmaf(wx[j], q, A);
                M = __builtin_fmaf(w[j], q, M);
                N = __builtin_fmaf(w[j], fabsf(q), N);
            }
            const float U = __builtin_fmaf(M, dl, N + w64);
            const float key = __builtin_fmaf(U, mk, __builtin_fmaf(A, -2.0f, bd) * inv_d);
            const bool better = key < vbest;
            vbest = better ? key : vbest;
            idx = better ? e0 + kW1Tile * tt + de : idx;
        }
    }
    *key_out = vbest;
    return idx;
}

// Weighted squared error of a group against d*(2k+1)*(q + delta) for entry e
// and choice cs = k + 8*shift, in fp64 from its definition: the sum of
// w*(x - s*(q + delta))^2, delta = +1/8 for shift 0 and -1/8 for shift 1 (the
// table holds entry e at e + e/kCh).
template <int kCh, class GS>
__device__ __forceinline__ double group_error64_w1(const GS& src, bool zero, const uint4* sq, int e,
                                                   int cs, float d)
{
    float x[8], w[8];
    src.load(zero, x, w);
    const uint4 u = sq[e + e / kCh];
    const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
    const double sc = (double)d * (double)(2 * (cs & 7) + 1);
    const double delta = (cs >> 3) ? -0.125 : 0.125;
    double err = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const double q = (double)bf16_to_f32((uu[j >> 1] >> (16 * (j & 1))) & 0xffffu);
        const double r = (double)x[j] - sc * (q + delta);
        err += (double)w[j] * r * r;
    }
    return err;
}

// kFmt: IQ_FMT_IQ1_S or IQ_FMT_IQ1_M; kMode: kModePayload, kModeEvery,
// kModeFake (IQ1_S) or kModeCandidates; kDT: the weight's iq_dtype_t.
template <int kFmt, int kMode, int kDT>
__global__ __launch_bounds__(kThreads) void iq1s_payload_wide_kernel(Iq1sArgs a)
{
    // IQ1_M: 56-byte blocks, a local scale per two groups (16 choice groups
    // of 8 choices), the shift free per group.
    constexpr bool kM = kFmt == IQ_FMT_IQ1_M;
    constexpr int kBB = kM ? kBlockBytesM : kBlockBytes;
    constexpr int kCG = kM ? 16 : 8;         // choice groups per block
    constexpr int kNC = kM ? 8 : 16;         // choices per choice group
    // Tracking chunks of kCT tiles; more than 16 chunks take 8-bit indices.
    // The candidates and every choice pick several choices per group, each a
    // rescan of its chunk, so their chunks are 2 tiles (32 of them for 2048
    // entries; candidates 14 % faster at top_c 8 than with 4 tiles).  One
    // pick per group keeps 4 tiles (2 tiles cost the payload 2 %: the
    // tracking runs twice as often).
    constexpr bool kCand = kMode == kModeCandidates;
    constexpr bool kEvery = kMode == kModeEvery;
    constexpr bool kMany = kCand || kEvery;
    constexpr int kNP = kEvery ? kNC : 1;             // payloads per block
    constexpr int kCT = kMany ? 2 : kW1ChunkTiles;   // tiles per chunk
    constexpr int kCh = kW1Tile * kCT;                // entries per chunk
    constexpr int kSlots = kMaxGrid + kMaxGrid / kCh;
    constexpr int kCB = kMaxGrid / kCh > 16 ? 8 : 4;  // bits of a chunk index
    constexpr int kFPW = 32 / kCB;                    // chunk indices per word
    constexpr int kCW = 16 / kFPW;                    // words of chunk indices
    __shared__ uint4 wsp[kSlots];                      // (q[0..7] + 1/8)^2 as bf16
    __shared__ uint4 wsq[kSlots];                      // q[0..7] as bf16
    __shared__ uint16_t sout16[kCand ? 1 : kNP * kWavesPerWG * kBB / 2];   // the set's payloads
    // candidates and every choice: each lane's 16 minima after the sweep;
    // candidates: per wave and choice unit the choices and their costs in
    // (cost, choice) order
    __shared__ float4 sbest[kMany ? 4 * kThreads : 1];   // [c/4][thread]
    __shared__ float srank_cost[kCand ? kWavesPerWG * 128 : 1];
    __shared__ uint8_t srank_c[kCand ? kWavesPerWG * 128 : 1];
    __shared__ int sgrid_bad;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: block pointers in SGPRs
    const int n = a.grid_size;
    const int nchunks = (n + kCh - 1) / kCh;
    const int npad = nchunks * kCh;

    if (tid == 0) sgrid_bad = 0;
    if (!kCand)
        for (int i = tid; i < kNP * kWavesPerWG * kBB / 2; i += kThreads) sout16[i] = 0;
    __syncthreads();
    {
        const float4* gsrc = reinterpret_cast<const float4*>(a.grid);
        int bad = 0;
        for (int e = tid; e < npad; e += kThreads) {
            const int src = e < n ? e : n - 1;
            const float4 v0 = gsrc[2 * src], v1 = gsrc[2 * src + 1];
            const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            uint32_t h[8], hp[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                bad |= !(v[t] == 0.0f || v[t] == 1.0f || v[t] == -1.0f);
                h[t] = bf16_bits(v[t]);
                const float pp = v[t] + 0.125f;
                hp[t] = bf16_bits(pp * pp);        // exact: 81/64, 1/64, 49/64
            }
            const int at = e + e / kCh;
            wsq[at] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                 h[4] | (h[5] << 16), h[6] | (h[7] << 16));
            wsp[at] = make_uint4(hp[0] | (hp[1] << 16), hp[2] | (hp[3] << 16),
                                 hp[4] | (hp[5] << 16), hp[6] | (hp[7] << 16));
        }
        if (bad) sgrid_bad = 1;
    }
    __syncthreads();
    const bool grid_bad = sgrid_bad != 0;
    if (grid_bad && tid == 0) report(a.status, IQ_ERR_GRID);

    const int64_t nsets = (a.g.nblocks + kWavesPerWG - 1) / kWavesPerWG;
    for (int64_t set = blockIdx.x; set < nsets; set += gridDim.x) {
    if (set != blockIdx.x) __syncthreads();     // the previous set's payloads are out
    // every wave of the workgroup has a block of this set (workgroup-uniform)
    const bool set_full = (set + 1) * kWavesPerWG <= a.g.nblocks;
    const int64_t blk = set * kWavesPerWG + wave;
    if (blk < a.g.nblocks) {                    // wave-uniform
        int ln = lane;                          // opaque: lane offsets are formed per block
        __asm__ volatile("" : "+v"(ln));
        const int g = ln & 31;                  // group = matrix column
        const int hl = ln >> 5;                 // K half / row half
        const int64_t bt = blk / a.g.blocks_per_batch;
        const int64_t cb = blk % a.g.blocks_per_row;
        const WeightBlock<kDT> xb(a.w, blk);
        const float* wblk = a.imp ? a.imp + bt * a.g.cols + cb * kBlockElems : nullptr;
        const GlobalGroup<WeightBlock<kDT>> src{xb, wblk, g};

        int err = 0;
        float amax = 0.0f, ssq = 0.0f;
        {
            const float4 xv = xb.quad(lane);
            const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (!finite_f32(xs[t])) err = IQ_ERR_NONFINITE;
                amax = fmaxf(amax, fabsf(xs[t]));
            }
            if (kM) ssq = ((xs[0] * xs[0] + xs[1] * xs[1]) + xs[2] * xs[2]) + xs[3] * xs[3];
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
        for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl(amax, ln ^ o));
        if (kM) {
            // the sum of squares in the fixed order the IQ1_M predictor uses:
            // per lane left to right, then pairwise at distances 1, 2, ..., 32
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) ssq = ssq + __shfl(ssq, ln ^ o);
        }

        uint32_t dh;
        if (a.scales) {
            dh = (uint32_t)a.scales[blk];
        } else if (kM) {
            // anchor clamp(0.58 + 0.035 * amax / rms, 0.65, 0.95); d = 0 for
            // an all-zero block
            dh = 0u;
            if (amax > 0.0f) {
                const float rms = __builtin_sqrtf(ssq / 256.0f);
                const float ratio = amax / rms;
                const float tk = 0.035f * ratio;
                const float an = fminf(fmaxf(0.58f + tk, 0.65f), 0.95f);
                const float t = amax / 16.875f;
                const float u = t * an;
                dh = f32_to_f16_bits(u);
            }
        } else {
            const float t = amax / 16.875f;
            const float u = t * 0.61f;
            dh = f32_to_f16_bits(u);
        }
        dh = __builtin_amdgcn_readfirstlane(dh);            // the same in every lane
        const bool scale_bad = ((dh & 0x7c00u) == 0x7c00u) || ((dh & 0x8000u) && (dh & 0x7fffu));
        dh &= 0x7fffu;
        if (scale_bad && !block_bad && lane == 0) report(a.status, IQ_ERR_SCALE_RANGE);
        const float d = scale_bad ? 0.0f : f16_bits_to_f32(dh);

        bool choice_bad = false;
        if (!kMany && a.choices) {
            int lc = lane;                      // opaque: the address is formed here, not hoisted
            __asm__ volatile("" : "+v"(lc));
            const int cv = lc < kCG ? a.choices[blk * kCG + lc] : 0;
            const bool bad = cv < 0 || cv >= kNC;
            if (bad) report(a.status, IQ_ERR_ARG);
            choice_bad = __ballot(bad) != 0;
        }
        const bool zero_block = grid_bad || block_bad || scale_bad || dh == 0u || choice_bad;

        // The lane's group: its K half of the three-way bf16 split of
        // -2*w*x/d, of w, and of -w/2.
        float x[8], w[8];
        src.load(zero_block, x, w);
        const float inv_d = zero_block ? 1.0f : 1.0f / d;
        uint32_t n1[8], n2[8], w1[8], w2[8], h1[8], h2[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float wxj = w[j] * x[j];
            const float vn = -2.0f * (wxj * inv_d);
            const float vh = -0.5f * w[j];
            n1[j] = split_part(vn, hl);
            n2[j] = hl == 0 ? split_part(vn, 2) : 0u;
            w1[j] = split_part(w[j], hl);
            w2[j] = hl == 0 ? split_part(w[j], 2) : 0u;
            h1[j] = split_part(vh, hl);
            h2[j] = hl == 0 ? split_part(vh, 2) : 0u;
        }
        auto pack = [](const uint32_t (&b)[8]) {
            return as_v8bf(make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16),
                                      b[6] | (b[7] << 16)));
        };
        const v8bf on1 = pack(n1), on2 = pack(n2), ow1 = pack(w1), ow2 = pack(w2);
        const v8bf oh1 = pack(h1), oh2 = pack(h2);

        // chunk_of: kCB-bit chunk index of choice c in bits kCB*(c%kFPW) of
        // word c/kFPW.
        float best[16], snap[16];
        uint32_t chunk_of[kCW];
#pragma unroll
        for (int i = 0; i < kCW; ++i) chunk_of[i] = 0u;
#pragma unroll
        for (int c = 0; c < 16; ++c) { best[c] = __builtin_inff(); snap[c] = best[c]; }
        const v16f zero16 = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f,
                             0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        // The waves of a full set sweep in step, a barrier per chunk, so that
        // no wave is left to finish its block alone.  For the IQ1_S payload,
        // half the waves of each SIMD (waves w, w + 4, ... share a SIMD) pass
        // the barrier half a chunk later in their sweep than the other half,
        // so that their chunk-end work falls at different times (measured: 2 %
        // faster there, 2-3 % slower for the other outputs, which keep the
        // barrier after the chunk's tracking).
        constexpr bool kStagger = !kM && kMode == kModePayload;
        const int stag = ((wave >> 2) & 1) ? kCT / 2 - 1 : kCT - 1;
        for (int ch = 0; ch < nchunks; ++ch) {
            for (int tt = 0; tt < kCT; ++tt) {
                const int at = (ch * kCT + tt) * kW1Tile + g + ch;
                const v8bf ap = as_v8bf(wsp[at]), aq = as_v8bf(wsq[at]);
                const v16f vq = mfma32(aq, on2, mfma32(aq, on1, zero16));
                v16f uu = mfma32(ap, ow2, mfma32(ap, ow1, zero16));
                fold_wide8<0>(uu, vq, best);
                uu = mfma32(aq, oh2, mfma32(aq, oh1, uu));          // U(-1/8)
                fold_wide8<8>(uu, vq, best);
                if (kStagger && set_full && tt == stag) __syncthreads();
            }
            const uint32_t chrep = (uint32_t)ch * (kCB == 4 ? 0x11111111u : 0x01010101u);
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const uint32_t msk = best[c] < snap[c] ? (((1u << kCB) - 1u) << (kCB * (c % kFPW))) : 0u;
                chunk_of[c / kFPW] = (chunk_of[c / kFPW] & ~msk) | (chrep & msk);
                snap[c] = best[c];
            }
            if (!kStagger && set_full) __syncthreads();
        }

        // Candidates and every choice: the lane's minima go to LDS, where the
        // picks read them, so that they need not stay live through the
        // epilogue.
        if constexpr (kMany) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                sbest[q4 * kThreads + tid] = make_float4(best[4 * q4], best[4 * q4 + 1],
                                                         best[4 * q4 + 2], best[4 * q4 + 3]);
        }

        // Lane-derived values for the rest of the block, formed here from an
        // opaque lane id so that none is held (or spilled) through the sweep.
        int ln2 = lane;
        __asm__ volatile("" : "+v"(ln2) :: "memory");
        const int g2 = ln2 & 31;
        const int hl2 = ln2 >> 5;
        const int sub2 = g2 >> 2;
        const int lq2 = g2 & 3;
        const GlobalGroup<WeightBlock<kDT>> src2{xb, wblk, g2};
        float w64, b4;
        {
            float W = 0.0f, B = 0.0f;
            src2.load(zero_block, x, w);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float wxj = w[j] * x[j];
                W += w[j];
                B += wxj;
            }
            w64 = W * 0.015625f;
            b4 = B * 0.25f;
        }
        const float b4d = b4 * inv_d;               // -2*(-1/8)*B/d; +1/8 takes -b4d

        // Choice costs per sub-block: (2k+1) times the sum of its four groups'
        // least keys (each the lesser of the group's two lanes, plus the
        // -2*delta*sum(wx)/d the sweep left out).
        // IQ1_M: per group and local scale k, the lesser of its two shifts'
        // least keys (the lower shift on equal keys); per scale group, (2k+1)
        // times the sum over its two groups.
        int cstar = 0;
        float cbest = 0.0f;
        float cost[16];
        uint32_t shbits = 0u;        // IQ1_M: bit k = this group's shift under local scale k
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            float m = fminf(best[c], __shfl(best[c], ln2 ^ 32));
            m += c < 8 ? -b4d : b4d;
            if (kM) {
                cost[c] = m;
            } else {
                float v = m + quad_xchg<kQuadXor1>(m);
                v += quad_xchg<kQuadXor2>(v);
                cost[c] = (float)(2 * (c & 7) + 1) * v;
                if (c == 0 || cost[c] < cbest) { cbest = cost[c]; cstar = c; }
            }
        }
        if (kM) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const bool sh = cost[8 + k] < cost[k];
                shbits |= (uint32_t)sh << k;
                const float v = sh ? cost[8 + k] : cost[k];
                cost[k] = (float)(2 * k + 1) * (v + quad_xchg<kQuadXor1>(v));
                if (k == 0 || cost[k] < cbest) { cbest = cost[k]; cstar = k; }
            }
        }
        // Entry for choice cs: the lane of the column whose minimum is least
        // holds it; the two lanes split its entries of the chunk.  With equal
        // minima in the two lanes of any column, every lane rescans its own
        // entries and the lane of least minimum, then lowest entry, wins.
        auto pick = [&](int cs) -> int {
            float lm = best[0];
            if constexpr (kMany) {
                lm = reinterpret_cast<const float*>(sbest + (cs >> 2) * kThreads + tid)[cs & 3];
            } else {
#pragma unroll
                for (int c = 1; c < 16; ++c)
                    if (cs == c) lm = best[c];
            }
            const int tchunk = (int)((chunk_of[cs / kFPW] >> (kCB * (cs % kFPW))) & ((1u << kCB) - 1u));
            const float om = __shfl(lm, ln2 ^ 32);
            const bool tie = __ballot(om == lm) != 0;                // wave-uniform
            int idx;
            float key;
            if (!tie) {
                const int hs = (om < lm) ? (hl2 ^ 1) : hl2;             // holder half
                const int tch = __shfl(tchunk, g2 + 32 * hs);
                idx = rescan_w1<8, kCT>(wsq, tch, hs, 8 * hl2, cs, src2, zero_block, w64, b4, inv_d,
                                        &key);
                const float ok = __shfl(key, ln2 ^ 32);
                const int oi = __shfl(idx, ln2 ^ 32);
                if (ok < key || (ok == key && oi < idx)) { key = ok; idx = oi; }
            } else {
                idx = rescan_w1<16, kCT>(wsq, tchunk, hl2, 0, cs, src2, zero_block, w64, b4, inv_d,
                                         &key);
                const int oi = __shfl(idx, ln2 ^ 32);
                if (om < lm || (om == lm && oi < idx)) idx = oi;
            }
            return idx < n ? idx : n - 1;
        };

        // IQ1_M: the (k, shift) choice of this group under its scale group's k
        auto full = [&](int k) { return kM ? k + 8 * (int)((shbits >> k) & 1u) : k; };
        // This group's part of the block's payload ob under choice ch
        // ((k, shift) cs) and entry idx.  A zero block leaves ob zero.
        auto pack_payload = [&](uint8_t* ob, int ch, int cs, int idx) {
            if (kM) {
                // IQ1_M: low byte per group; one nibble per group (3 high
                // bits, shift bit); four scale words with the 3-bit local
                // scales of four scale groups and one nibble of d each.
                const int nib = ((idx >> 8) & 7) | ((cs >> 3) << 3);
                const int nib_odd = quad_xchg<kQuadXor1>(nib);
                int kk = (ch & 7) << (3 * ((g2 >> 1) & 3));
                kk |= quad_xchg<kQuadXor2>(kk);
                kk |= __shfl(kk, ln2 ^ 4);
                if (!zero_block && hl2 == 0) {
                    ob[g2] = (uint8_t)(idx & 0xff);
                    if ((g2 & 1) == 0) ob[32 + (g2 >> 1)] = (uint8_t)(nib | (nib_odd << 4));
                    if ((g2 & 7) == 0) {
                        const int wd = g2 >> 3;
                        const uint32_t v = (uint32_t)kk | (((dh >> (4 * wd)) & 0xfu) << 12);
                        ob[48 + 2 * wd] = (uint8_t)(v & 0xff);
                        ob[49 + 2 * wd] = (uint8_t)(v >> 8);
                    }
                }
            } else {
                // IQ1_S: low byte per group, qh word per sub-block, d per
                // block.
                int hi = ((idx >> 8) & 7) << (3 * lq2);
                hi |= quad_xchg<kQuadXor1>(hi);
                hi |= quad_xchg<kQuadXor2>(hi);
                if (!zero_block && hl2 == 0) {
                    ob[2 + g2] = (uint8_t)(idx & 0xff);
                    if (lq2 == 0) {
                        const uint32_t qh = (uint32_t)hi | ((uint32_t)cs << 12);
                        ob[34 + 2 * sub2] = (uint8_t)(qh & 0xff);
                        ob[35 + 2 * sub2] = (uint8_t)(qh >> 8);
                    }
                    if (g2 == 0) {
                        ob[0] = (uint8_t)(dh & 0xff);
                        ob[1] = (uint8_t)(dh >> 8);
                    }
                }
            }
        };

        if constexpr (kCand) {
            // Candidates: the unit's top_c choices by (cost, choice), formed
            // once.  Every lane of a choice unit (IQ1_S: 4 groups x 2 halves;
            // IQ1_M: 2 x 2) holds the same costs; the lane of slot u ranks
            // choices 2u and 2u+1 by counting the costs below each and files
            // each choice and its cost under its rank in the LDS.  Equal costs
            // (or a NaN) leave the ranks short of a permutation; a wave with
            // such a unit takes the selection below in every round instead.
            // With a zero scale every choice decodes to zero with entry 0, so
            // the order is 0, 1, ...
            const bool rejected = grid_bad || block_bad || scale_bad || choice_bad;
            const bool zero_scale = !rejected && dh == 0u;
            const int unit = kM ? (g2 >> 1) : sub2;
            const int part = kM ? (g2 & 1) : lq2;
            const int uslot = kM ? ((g2 & 1) | (hl2 << 1)) : (lq2 | (hl2 << 2));
            const int ubase = wave * 128 + unit * kNC;
            int rmask = 0;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int uc = 2 * uslot + i;
                float mine = cost[0];
#pragma unroll
                for (int c = 1; c < kNC; ++c)
                    if (uc == c) mine = cost[c];
                int rank = 0;
#pragma unroll
                for (int c = 0; c < kNC; ++c) rank += cost[c] < mine ? 1 : 0;
                if (zero_scale) rank = uc;
                srank_cost[ubase + rank] = mine;
                srank_c[ubase + rank] = (uint8_t)uc;
                rmask |= 1 << rank;
            }
            rmask |= quad_xchg<kQuadXor1>(rmask);
            if (!kM) rmask |= quad_xchg<kQuadXor2>(rmask);
            rmask |= __shfl(rmask, ln2 ^ 32);
            bool ordered = __ballot(rmask != (1 << kNC) - 1) == 0;     // wave-uniform
            const float* rc = srank_cost + ubase;
            const uint8_t* rk8 = srank_c + ubase;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

            // The unit's fp64 error under cs with this lane's entry: its four
            // groups (IQ1_S sub-block) or two (IQ1_M scale group).
            auto unit_err64 = [&](int cs, int idx) -> double {
                double e = group_error64_w1<kCh>(src2, zero_block, wsq, idx, cs, d);
                e += quad_xchg<kQuadXor1>(e);
                if (!kM) e += quad_xchg<kQuadXor2>(e);
                return e;
            };
            uint32_t used = 0u;
            for (int it = 0; it < a.top_c; ++it) {
                int cr = -1;
                float vr = 0.0f;
                bool nr = false;
                if (ordered) {                                  // wave-uniform
                    cr = rk8[it];
                    vr = rc[it];
                    if (it + 1 < kNC && !zero_block) nr = rc[it + 1] - vr <= 0x1p-18f * fabsf(vr);
                }
                if (!ordered || __ballot(nr) != 0) {            // wave-uniform
                    const int cord = cr;
                    cr = -1;
#pragma unroll
                    for (int c = 0; c < kNC; ++c) {
                        const bool better = zero_scale ? (cr < 0) : (cr < 0 || cost[c] < vr);
                        if (!((used >> c) & 1u) && better) { cr = c; vr = cost[c]; }
                    }
                    // Unused choices whose fp32 cost is within 2^-18 of the
                    // least's magnitude are ranked again by their fp64 errors
                    // (with their own entries), the lower choice on equal
                    // errors, as the payload's runner-up is.
                    uint32_t nearm = 0u;
                    if (!zero_block) {
#pragma unroll
                        for (int c = 0; c < kNC; ++c)
                            if (!((used >> c) & 1u) && c != cr && cost[c] - vr <= 0x1p-18f * fabsf(vr))
                                nearm |= 1u << c;
                    }
                    if (__ballot(nearm != 0u) != 0) {           // wave-uniform
                        double b64 = unit_err64(full(cr), pick(full(cr)));
                        for (int c = 0; c < kNC; ++c) {
                            if (__ballot((nearm >> c) & 1u) == 0) continue;   // wave-uniform
                            const double e = unit_err64(full(c), pick(full(c)));
                            if (((nearm >> c) & 1u) && (e < b64 || (e == b64 && c < cr))) {
                                b64 = e;
                                cr = c;
                            }
                        }
                    }
                    // a pick out of the filed order ends its use
                    if (ordered && __ballot(cr != cord) != 0) ordered = false;
                }
                used |= 1u << cr;
                const int cs = full(cr);
                int idx = pick(cs);
                if (zero_scale) idx = 0;
                // Each lane of a group writes 4 of its 8 errors xhat - x
                // (xhat exact in fp32, one rounding); the first half also its
                // code and, once per unit, the choice.
                const int64_t base = (blk * kCG + unit) * a.top_c + it;    // [block][unit][r]
                float xo[8], wo[8];
                src2.load(rejected, xo, wo);
                const float sk = f16_bits_to_f32(dh) * (float)(2 * (cs & 7) + 1);
                const float delta = (cs >> 3) ? -0.125f : 0.125f;
                const uint4 u = wsq[idx + idx / kCh];
                const uint32_t u0 = hl2 ? u.z : u.x, u1 = hl2 ? u.w : u.y;
                const uint32_t uu[4] = {u0 & 0xffffu, u0 >> 16, u1 & 0xffffu, u1 >> 16};
                float ev[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float xj = hl2 ? xo[4 + j] : xo[j];
                    ev[j] = rejected ? 0.0f : sk * (bf16_to_f32(uu[j]) + delta) - xj;
                }
                float4* ep = reinterpret_cast<float4*>(a.cand_err + base * (256 / kCG) + part * 8 + 4 * hl2);
                ep[0] = make_float4(ev[0], ev[1], ev[2], ev[3]);
                if (hl2 == 0) {
                    if (part == 0) a.cand_choice[base] = cr;
                    if (a.cand_codes) {
                        const int shc = (kM && !zero_scale) ? (cs >> 3) : 0;
                        const uint16_t code = kM ? (uint16_t)(idx | (shc << 11)) : (uint16_t)idx;
                        a.cand_codes[base * (kM ? 2 : 4) + part] = rejected ? (uint16_t)0 : code;
                    }
                }
            }
        } else if constexpr (kEvery) {
            // Every choice: payload c has every choice group forced to c, a
            // pick per group and choice.
#pragma unroll 1
            for (int c = 0; c < kNC; ++c) {
                const int cs = full(c);
                pack_payload(reinterpret_cast<uint8_t*>(sout16) + (c * kWavesPerWG + wave) * kBB, c, cs,
                             pick(cs));
            }
        } else {
            const int forced = (a.choices && !choice_bad) ? a.choices[blk * kCG + (kM ? (g2 >> 1) : sub2)] : -1;
            if (forced >= 0) cstar = forced;
            int c2 = 0;
            bool near = false;
            if (forced < 0) {                           // wave-uniform
                float v2 = 0.0f;
                c2 = -1;
#pragma unroll
                for (int c = 0; c < kNC; ++c)
                    if (c != cstar && (c2 < 0 || cost[c] < v2)) { c2 = c; v2 = cost[c]; }
                near = !zero_block && v2 - cbest <= 0x1p-18f * fabsf(cbest);
            }
            const bool refine = __ballot(near) != 0;  // wave-uniform

            int ch = cstar;
            int cs = full(cstar);
            int idx;
            if (!refine) {
                idx = pick(cs);
            } else {
                // The runner-up within 2^-18 of the best: both in fp64 from the
                // error's definition, summed over the sub-block; the lower error
                // wins, the lower choice on equal errors.
                const int cs2 = full(near ? c2 : cstar);
                const int i2 = pick(cs2);
                const int i1 = pick(cs);
                double e2 = group_error64_w1<kCh>(src2, zero_block, wsq, i2, cs2, d);
                double e1 = group_error64_w1<kCh>(src2, zero_block, wsq, i1, cs, d);
                e2 += quad_xchg<kQuadXor1>(e2);
                e1 += quad_xchg<kQuadXor1>(e1);
                if (!kM) {
                    e2 += quad_xchg<kQuadXor2>(e2);
                    e1 += quad_xchg<kQuadXor2>(e1);
                }
                idx = i1;
                if (near && (e2 < e1 || (e2 == e1 && c2 < cstar))) { ch = c2; cs = cs2; idx = i2; }
            }

            pack_payload(reinterpret_cast<uint8_t*>(sout16) + wave * kBB, ch, cs, idx);
            if (kMode == kModeFake && hl2 == 0) {
                // The decoded group, d*(2k+1)*(q + delta) with the payload's
                // fields, the expression the decode kernel uses (a zero block
                // decodes as the all-zero payload does; a rejected block is
                // written as zeros).
                const bool rejected = grid_bad || block_bad || scale_bad || choice_bad;
                const uint32_t dz = zero_block ? 0u : dh;
                const int ez = zero_block ? 0 : idx;
                const int cz = zero_block ? 0 : cs;
                const float sk = f16_bits_to_f32(dz) * (float)(2 * (cz & 7) + 1);
                const float delta = (cz >> 3) ? -0.125f : 0.125f;
                const uint4 u = wsq[ez + ez / kCh];
                const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float q = bf16_to_f32((uu[j >> 1] >> (16 * (j & 1))) & 0xffffu);
                    v[j] = rejected ? 0.0f : sk * (q + delta);
                }
                float4* o = reinterpret_cast<float4*>(a.xhat + blk * kBlockElems + g2 * 8);
                o[0] = make_float4(v[0], v[1], v[2], v[3]);
                o[1] = make_float4(v[4], v[5], v[6], v[7]);
            }
        }
    }
    if (!kCand && a.out) {
        // Copy the set's payloads out (every choice: payload c of the set to
        // out[c]) and clear what was copied (each word by the thread that
        // copied it) for the next set.
        __syncthreads();
        const int64_t first = set * kWavesPerWG;
        const int64_t left = a.g.nblocks - first;
        const int nb = left < kWavesPerWG ? (int)left : kWavesPerWG;
        for (int c = 0; c < kNP; ++c) {
            uint16_t* o16 = reinterpret_cast<uint16_t*>(a.out + (c * a.g.nblocks + first) * kBB);
            uint16_t* s16 = sout16 + c * kWavesPerWG * (kBB / 2);
            int t0 = tid;
            __asm__ volatile("" : "+v"(t0));
            for (int i = t0; i < nb * (kBB / 2); i += kThreads) {
                o16[i] = s16[i];
                s16[i] = 0;
            }
        }
    }
    }
}

template <int kFmt, int kDT>
hipError_t launch_fmt(const Iq1sArgs& a, int mode, hipStream_t stream)
{
    // One workgroup per compute unit (the LDS holds one), or one per set of
    // 16 blocks when there are fewer sets.
    const int64_t sets = (a.g.nblocks + kWavesPerWG - 1) / kWavesPerWG;
    const dim3 grid((unsigned)(sets < a.g.cus ? sets : a.g.cus));
    if (mode == kModeEvery) {
        hipLaunchKernelGGL((iq1s_payload_wide_kernel<kFmt, kModeEvery, kDT>), grid,
                           dim3(kThreads), 0, stream, a);
    } else if (mode == kModeFake) {
        hipLaunchKernelGGL((iq1s_payload_wide_kernel<kFmt, kModeFake, kDT>), grid, dim3(kThreads), 0,
                           stream, a);
    } else if (mode == kModeCandidates) {
        hipLaunchKernelGGL((iq1s_payload_wide_kernel<kFmt, kModeCandidates, kDT>), grid,
                           dim3(kThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL((iq1s_payload_wide_kernel<kFmt, kModePayload, kDT>), grid,
                           dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

template <int kFmt>
hipError_t launch_dtype(const Iq1sArgs& a, int wdtype, int mode, hipStream_t stream)
{
    switch (wdtype) {
    case IQ_DTYPE_BF16: return launch_fmt<kFmt, IQ_DTYPE_BF16>(a, mode, stream);
    case IQ_DTYPE_F16: return launch_fmt<kFmt, IQ_DTYPE_F16>(a, mode, stream);
    case IQ_DTYPE_F64: return launch_fmt<kFmt, IQ_DTYPE_F64>(a, mode, stream);
    default: return launch_fmt<kFmt, IQ_DTYPE_F32>(a, mode, stream);
    }
}

}  // namespace

hipError_t launch_iq1_encode(int fmt, int wdtype, const void* w, const float* imp,
                             const float* grid, int grid_size, const uint16_t* scales,
                             const int32_t* choices, uint8_t* out, float* xhat, int mode,
                             int32_t* status, const BlockGeom& g, hipStream_t stream)
{
    Iq1sArgs a{w, imp, grid, scales, choices, out, xhat, nullptr, nullptr, nullptr, status, g,
               grid_size, 0};
    return fmt == IQ_FMT_IQ1_M ? launch_dtype<IQ_FMT_IQ1_M>(a, wdtype, mode, stream)
                               : launch_dtype<IQ_FMT_IQ1_S>(a, wdtype, mode, stream);
}

hipError_t launch_iq1_candidates(int fmt, int wdtype, const void* w, const float* imp,
                                 const float* grid, int grid_size, int top_c, float* cand_err,
                                 int32_t* cand_choice, uint16_t* cand_codes, int32_t* status,
                                 const BlockGeom& g, hipStream_t stream)
{
    Iq1sArgs a{w, imp, grid, nullptr, nullptr, nullptr, nullptr, cand_err, cand_choice, cand_codes,
               status, g, grid_size, top_c};
    return fmt == IQ_FMT_IQ1_M ? launch_dtype<IQ_FMT_IQ1_M>(a, wdtype, kModeCandidates, stream)
                               : launch_dtype<IQ_FMT_IQ1_S>(a, wdtype, kModeCandidates, stream);
}

}  // namespace iqk
