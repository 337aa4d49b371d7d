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
// U(+1/8), U(-1/8) and -2*sum(wx*q) for 16 grid entries x 16 groups are
// three small products [16 entries x 8] x [8 x 16 groups], run as
// v_mfma_f32_16x16x32_bf16: the entry side (q+delta)^2 and q is exact in bf16
// (values like 81/64 need 7 mantissa bits), the group side (w and -2*w*x) is
// split into three bf16 parts whose sum is exactly the fp32 value, so the
// products are exact and only the fp32 accumulation rounds.  The rest of
// -2V(delta), -2*delta*sum(wx), is the same for every entry of a group and
// shift, so it does not move the sweep's minima between entries: it is added
// to them once after the sweep.  Everything is divided by the block scale d
// (the V side carries 1/d), so the sweep key of local scale s_k = d*(2k+1) is
// (2k+1)*U - 2*sum(wx*q)/d: one FMA with a literal multiplier
// (v_fmamk_f32, two register operands, which pairs well with v_min3 in the
// dual-issue VALU); the choice cost of a sub-block is (2k+1) times the sum of
// its groups' minima (the common factor d^2 dropped).  The VALU keeps
// value-only minima (v_min3 over two entries).
//
// Two kernels run this search.  iq1s_payload_wide_kernel (32 x 32 tiles, a
// wave per block, defined further down) gives the payload of both formats and
// the IQ1_S fake quant; iq1s_encode_kernel (16 x 16 tiles, described here)
// gives every choice, the candidates and the IQ1_M fake quant, whose many
// picks per group rescan fewer entries per lane in this layout.
//
// Layout: a wave owns 16 groups (half a block): matrix column j = lane%16 is
// group j; the lane's four accumulator rows are 4*(lane/16)+r of every
// 16-entry tile, so the four lanes of a column cover disjoint quarters of the
// grid.  A 1024-thread workgroup runs 16 waves = 8 blocks per pass and 2
// passes per set of 16 blocks; the workgroups are persistent (one per CU, 4
// waves per SIMD) and stage the grid once in LDS as bf16 ((q+1/8)^2,
// (q-1/8)^2 and q, 96 KiB).
// Index recovery: each lane records the chunk (128 or 256 entries) that last
// lowered each of its 16 minima; once the choice is fixed, the lane of each
// column whose matrix-core minimum is least is found, and the four lanes of
// the column split its entries of that chunk between them and rescan them on
// the VALU (fp32 dot products), lowest entry of least key.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace iqk {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWavesPerWG = 16;
constexpr int kThreads = kWave * kWavesPerWG;        // 1024
constexpr int kBlocksPerPass = kWavesPerWG / 2;      // two waves per block
constexpr int kPasses = 2;
constexpr int kBlocksPerWG = kBlocksPerPass * kPasses;   // 16
constexpr int kTile = 16;                            // grid entries per matrix tile
// Tiles per tracking chunk.  Recording chunks costs the sweep about 4
// instructions per choice and chunk; each pick rescans one lane's entries of
// a chunk, 4 per tile.  IQ1_S with one pick per group (payload, fake quant,
// when this kernel ran them): 16 tiles (256 entries), measured 3 % faster
// than 8; otherwise 8 (128 entries), as small as 4-bit chunk numbers allow
// for 2048 entries (IQ1_M measured 3 % slower with 16).
template <int kFmt, int kMode>
constexpr int chunk_tiles()
{
    return (kFmt == IQ_FMT_IQ1_S && (kMode == kModePayload || kMode == kModeFake)) ? 16 : 8;
}
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

// The 8 values and weights of the wave's local group c (0..15) from the
// wave's LDS copy of its half block: 32 float4 of values, then 32 of
// weights (zeros and ones for a rejected block).
__device__ __forceinline__ void load_group_lds(const float4* s, int c, bool zero, float (&x)[8],
                                               float (&w)[8])
{
    if (zero) {
#pragma unroll
        for (int j = 0; j < 8; ++j) { x[j] = 0.0f; w[j] = 1.0f; }
        return;
    }
    const float4 x0 = s[2 * c], x1 = s[2 * c + 1], w0 = s[32 + 2 * c], w1 = s[33 + 2 * c];
    x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
    x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
    w[0] = w0.x; w[1] = w0.y; w[2] = w0.z; w[3] = w0.w;
    w[4] = w1.x; w[5] = w1.y; w[6] = w1.z; w[7] = w1.w;
}

// The status atomic: the global form in the modes that stage the block in
// LDS (a generic atomic counts as a pending LDS access and would make the
// sweep wait for all of its LDS reads at once), the generic form otherwise
// (with which the payload and fake-quant kernels measured fastest).
template <bool kGlobal>
__device__ __forceinline__ void report_status(int32_t* status, int code)
{
    if constexpr (kGlobal) report(status, code);
    else report_generic(status, code);
}

// Where a lane's group values and weights are read again after the sweep:
// global memory (GlobalGroup), or the wave's LDS copy of its half block
// (LdsGroup), which the modes that pick many choices use.
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

struct LdsGroup {
    const float4* s;
    int c;
    __device__ __forceinline__ void load(bool zero, float (&x)[8], float (&w)[8]) const
    {
        load_group_lds(s, c, zero, x, w);
    }
};

template <bool kLds, class XB>
__device__ __forceinline__ auto group_source(const XB& xb, const float* wblk, int g,
                                             const float4* s, int c)
{
    if constexpr (kLds) return LdsGroup{s, c};
    else return GlobalGroup<XB>{xb, wblk, g};
}

// VALU rescan for choice cs = k + 8*deltabit over tiles t0 .. t0+nt-1 of chunk
// tchunk, rows 4*kbs .. 4*kbs+3 of each tile (the entries one lane of a
// column covers): the lowest entry with the least key (2k+1)*U - 2V/d,
// recomputed in fp32 from the group's values and weights (read again from
// memory rather than held through the sweep).  Returns the entry, writes its
// key.
template <int kChunkTiles, class GS>
__device__ __forceinline__ int rescan(const uint4* __restrict__ sq, int tchunk, int kbs, int t0,
                                      int nt, int cs, const GS& src, bool zero_block, float w64,
                                      float b4, float inv_d, float* key_out)
{
    float x[8], w[8];
    __asm__ volatile("" ::: "memory");
    src.load(zero_block, x, w);
    const float mk = (float)(2 * (cs & 7) + 1);
    const float dl = (cs >> 3) ? -0.25f : 0.25f;      // 2*delta
    const float bd = (cs >> 3) ? b4 : -b4;
    int idx = -1;
    float vbest = 0.0f;
    for (int tt = t0; tt < t0 + nt; ++tt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = (tchunk * kChunkTiles + tt) * kTile + 4 * kbs + r;
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
    *key_out = vbest;
    return idx;
}

// Weighted squared error of group g against d*(2k+1)*(q + delta) for entry
// e and choice cs = k + 8*shift, in fp64 from its definition: the sum of
// w*(x - s*(q + delta))^2, delta = +1/8 for shift 0 and -1/8 for shift 1.
template <int kChunk, class GS>
__device__ __forceinline__ double group_error64(const GS& src, bool zero, const uint4* sq, int e,
                                                int cs, float d)
{
    float x[8], w[8];
    src.load(zero, x, w);
    const uint4 u = sq[e + e / kChunk];
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

// kFmt: IQ_FMT_IQ1_S or IQ_FMT_IQ1_M; kMode: EncodeMode; kDT: the weight's
// iq_dtype_t.
template <int kFmt, int kMode, int kDT>
__global__ __launch_bounds__(kThreads) void iq1s_encode_kernel(Iq1sArgs a)
{
    // IQ1_M: 56-byte blocks, 8 local scales per two groups (16 choice
    // groups), a shift per group.  IQ1_S: 50 bytes, 16 (k, shift) choices per
    // sub-block of four groups.
    constexpr bool kM = kFmt == IQ_FMT_IQ1_M;
    constexpr int kBB = kM ? kBlockBytesM : kBlockBytes;
    constexpr int kChoices = kM ? 8 : 16;
    constexpr int kGroups = kM ? 16 : 8;          // choice groups per block
    // Payloads staged in LDS: one per block, or one per block and choice.
    constexpr int kPayloads = kMode == kModeEvery ? kChoices : 1;
    constexpr int kChunkTiles = chunk_tiles<kFmt, kMode>();
    // The modes that pick several choices per group keep each wave's half
    // block in LDS for their rescans (measured: candidates 5 % faster); the
    // payload and fake-quant modes read global memory again, which kept their
    // sweep's code as it was (the staging variant cost the c2 payload 3 %).
    constexpr bool kStage = kMode == kModeEvery || kMode == kModeCandidates;
    constexpr int kChunk = kTile * kChunkTiles;
    // Entry e sits at e + e/kChunk: one spare slot per chunk, so the lanes of
    // a rescan that read different chunks (a multiple of the 64 banks apart
    // without the slot) spread over the banks.
    constexpr int kSlots = kMaxGrid + kMaxGrid / kChunk;
    __shared__ uint4 sp[kSlots];         // (q[0..7] + 1/8)^2 as bf16
    __shared__ uint4 sm[kSlots];         // (q[0..7] - 1/8)^2 as bf16
    __shared__ uint4 sq[kSlots];         // q[0..7] as bf16
    __shared__ uint16_t sout16[kPayloads * kBlocksPerWG * kBB / 2];
    // Per wave, its half block's values and weights as fp32 (32 + 32 float4),
    // read back by the rescans instead of global memory (kStage modes).
    __shared__ float4 sxw_all[kStage ? kWavesPerWG * 64 : 1];
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
        for (int i = tid; i < kPayloads * kBlocksPerWG * kBB / 2; i += kThreads) sout16[i] = 0;
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
    if (grid_bad && tid == 0) report_status<kStage>(a.status, IQ_ERR_GRID);

    const int col = lane & 15;          // matrix column = group within the half block
    const int kb = lane >> 4;           // K slice of the operands / row quarter of the result
    const int half = wave & 1;
    const int g = half * 16 + col;      // group in block
    const int sub = g >> 2;
    const int lq = g & 3;

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
        float4* sxw = sxw_all + (kStage ? wave * 64 : 0);
        const float* wblk = a.imp ? a.imp + bt * a.g.cols + cb * kBlockElems : nullptr;
        const auto src = group_source<kStage>(xb, wblk, g, sxw, col);

        // Whole-block checks and amax (each lane reads 4 of the 256 values);
        // IQ1_M also sums the squares: per lane ((x0^2 + x1^2) + x2^2) + x3^2,
        // then pairwise across lanes at distances 1, 2, ..., 32.
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
            if (kStage) {
                float4 wv = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
                if (wblk) {
                    wv = reinterpret_cast<const float4*>(wblk)[lane];
                    const float ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (!err && (!(ws[t] >= 0.0f) || !finite_f32(ws[t])))
                            err = IQ_ERR_IMPORTANCE;
                }
                // The lanes holding this wave's half block keep it in LDS.
                if ((lane >> 5) == half) {
                    sxw[lane & 31] = xv;
                    sxw[32 + (lane & 31)] = wv;
                }
            } else if (wblk && !err) {
                const float4 wv = reinterpret_cast<const float4*>(wblk)[lane];
                const float ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (!(ws[t] >= 0.0f) || !finite_f32(ws[t])) err = IQ_ERR_IMPORTANCE;
            }
        }
        if (err && half == 0) report_status<kStage>(a.status, err);
        const bool block_bad = __ballot(err != 0) != 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        if (kM) {
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) ssq = ssq + __shfl_xor(ssq, o);
        }

        uint32_t dh;
        if (a.scales) {
            dh = (uint32_t)a.scales[blk];
        } else if (kM) {
            // anchor clamp(0.58 + 0.035 * amax / rms, 0.65, 0.95); d = 0 for an
            // all-zero block
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
        const bool scale_bad = ((dh & 0x7c00u) == 0x7c00u) || ((dh & 0x8000u) && (dh & 0x7fffu));
        dh &= 0x7fffu;
        if (scale_bad && !block_bad && half == 0 && lane == 0)
            report_status<kStage>(a.status, IQ_ERR_SCALE_RANGE);
        const float d = scale_bad ? 0.0f : f16_bits_to_f32(dh);

        // Forced choices: every wave of the block checks all of them.
        int forced = -1;
        bool choice_bad = false;
        if ((kMode == kModePayload || kMode == kModeFake) && a.choices) {
            int ln = lane;                  // opaque: the address is formed here, not hoisted
            __asm__ volatile("" : "+v"(ln));
            const int cv = ln < kGroups ? a.choices[blk * kGroups + ln] : 0;
            const bool bad = cv < 0 || cv >= kChoices;
            if (bad && half == 0) report_status<kStage>(a.status, IQ_ERR_ARG);
            choice_bad = __ballot(bad) != 0;
            forced = a.choices[blk * kGroups + (kM ? (g >> 1) : sub)];
        }
        const bool zero_block = grid_bad || block_bad || scale_bad || dh == 0u || choice_bad;
        if (choice_bad) forced = -1;

        // The lane's group: values, weights, sums, and its K slice of the
        // three-way bf16 split of -2*w*x and w (slice 3 is zero padding).
        float x[8], w[8];
        src.load(zero_block, x, w);
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
        const float b4d = b4 * inv_d;                 // -2*(-1/8)*B/d; +1/8 takes -b4d

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
                const v4f vq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, opn2wx, zero4, 0, 0, 0);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float mk = (float)(2 * k + 1);
                    const float p0 = __builtin_fmaf(up[0], mk, vq[0]);
                    const float p1 = __builtin_fmaf(up[1], mk, vq[1]);
                    const float p2 = __builtin_fmaf(up[2], mk, vq[2]);
                    const float p3 = __builtin_fmaf(up[3], mk, vq[3]);
                    const float m0 = __builtin_fmaf(um[0], mk, vq[0]);
                    const float m1 = __builtin_fmaf(um[1], mk, vq[1]);
                    const float m2 = __builtin_fmaf(um[2], mk, vq[2]);
                    const float m3 = __builtin_fmaf(um[3], mk, vq[3]);
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

        // Choice costs.  IQ1_S: per sub-block and choice c = k + 8*shift,
        // (2k+1) times the sum of its four groups' least keys (identical float
        // sums in every lane of the sub-block).  IQ1_M: per group and local
        // scale k, the lesser of its two shifts' least keys (the lower shift
        // on equal keys); per scale group, (2k+1) times the sum over its two
        // groups.  A group's least key is the least over its four lanes, plus
        // the -2*delta*sum(wx)/d the sweep left out.
        int cstar = 0;               // IQ1_S: the sub-block's choice; IQ1_M: the local scale
        float cbest = 0.0f;
        float cost[16];
        uint32_t shbits = 0u;        // IQ1_M: bit k = this group's shift under local scale k
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            float m = best[c];
            m = fminf(m, __shfl_xor(m, 16));
            m = fminf(m, __shfl_xor(m, 32));
            m += c < 8 ? -b4d : b4d;
            if (kM) {
                cost[c] = m;
            } else {
                float v = m + __shfl_xor(m, 1);
                v += __shfl_xor(v, 2);
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
                cost[k] = (float)(2 * k + 1) * (v + __shfl_xor(v, 1));
                if (k == 0 || cost[k] < cbest) { cbest = cost[k]; cstar = k; }
            }
        }
        if (forced >= 0) cstar = forced;
        // Payload and fake quant with free choices: the runner-up choice.  The
        // fp32 costs carry rounding of the size of the sums they cancel, so
        // when the runner-up is within 2^-18 of the best's magnitude (32 to 64
        // ulps), both are evaluated again in fp64 from the error's definition
        // with their own entries: the lower error wins, the lower choice on
        // equal errors.  The runner-up goes first through the loop below, as
        // an extra pass.
        constexpr bool kDecides = kMode == kModePayload || kMode == kModeFake;
        int c2 = 0;
        bool near = false;
        if (kDecides && forced < 0) {              // wave-uniform
            float v2 = 0.0f;
            c2 = -1;
#pragma unroll
            for (int c = 0; c < kChoices; ++c)
                if (c != cstar && (c2 < 0 || cost[c] < v2)) { c2 = c; v2 = cost[c]; }
            near = !zero_block && v2 - cbest <= 0x1p-18f * fabsf(cbest);
        }
        const bool refine = kDecides && __ballot(near) != 0;      // wave-uniform
        int idx_alt = 0;
        double err_alt = 0.0;
        // Candidates: the top_c choices by (cost, choice); with a zero scale
        // every choice decodes to zero with entry 0, so the order is 0, 1, ...
        const bool rejected = grid_bad || block_bad || scale_bad || choice_bad;
        const bool zero_scale = !rejected && dh == 0u;
        int used = 0;

        // For each choice to emit: this group's (k, shift) choice cs, its
        // entry (the lane rescans its entries of the chunk that holds its
        // minimum of cs, then the lane of the column whose matrix-core minimum
        // is least is kept), and the payload, decoded values or candidate.
        const int nloop = kMode == kModeEvery ? kChoices
                        : (kMode == kModeCandidates ? a.top_c : (refine ? 2 : 1));
        for (int it = 0; it < nloop; ++it) {
            int ch = kMode == kModeEvery ? it : cstar;
            if (refine && it == 0 && near) ch = c2;
            if (kMode == kModeCandidates) {
                int cr = -1;
                float vr = 0.0f;
#pragma unroll
                for (int c = 0; c < kChoices; ++c) {
                    const bool better = zero_scale ? (cr < 0) : (cr < 0 || cost[c] < vr);
                    if (!((used >> c) & 1) && better) { cr = c; vr = cost[c]; }
                }
                used |= 1 << cr;
                ch = cr;
            }
            int cs = kM ? ch + 8 * (int)((shbits >> ch) & 1u) : ch;
            float lane_min = best[0];
#pragma unroll
            for (int c = 1; c < 16; ++c)
                if (cs == c) lane_min = best[c];
            const int tchunk = (int)((chunk_of[cs >> 3] >> (4 * (cs & 7))) & 0xfu);
            // The lane of the column whose matrix-core minimum is least holds
            // the entry.  Unless two lanes of some column hold equal minima,
            // the four lanes split that lane's entries of its chunk between
            // them (kChunkTiles/4 tiles each) and keep the least key, lowest
            // entry on equal keys; with equal minima every lane rescans its own
            // entries and the lane of least minimum, then lowest entry, wins.
            float cm = fminf(lane_min, __shfl_xor(lane_min, 16));
            cm = fminf(cm, __shfl_xor(cm, 32));
            const uint64_t holders = (__ballot(lane_min == cm) >> col) & 0x0001000100010001ull;
            const bool tie = __ballot(__popcll(holders) > 1) != 0;      // wave-uniform
            int idx;
            float key;
            if (!tie) {
                const int kbs = __builtin_ctzll(holders) >> 4;
                const int tch = __shfl(tchunk, col + 16 * kbs);
                idx = rescan<kChunkTiles>(sq, tch, kbs, kb * (kChunkTiles / 4), kChunkTiles / 4, cs,
                                          src, zero_block, w64, b4, inv_d, &key);
#pragma unroll
                for (int o = 16; o <= 32; o <<= 1) {
                    const float ok = __shfl_xor(key, o);
                    const int oi = __shfl_xor(idx, o);
                    if (ok < key || (ok == key && oi < idx)) { key = ok; idx = oi; }
                }
            } else {
                idx = rescan<kChunkTiles>(sq, tchunk, kb, 0, kChunkTiles, cs, src, zero_block, w64,
                                          b4, inv_d, &key);
#pragma unroll
                for (int o = 16; o <= 32; o <<= 1) {
                    const float om = __shfl_xor(lane_min, o);
                    const int oi = __shfl_xor(idx, o);
                    if (om < lane_min || (om == lane_min && oi < idx)) { lane_min = om; idx = oi; }
                }
            }
            idx = idx < n ? idx : n - 1;
            if (refine) {
                // The choice unit's fp64 error: its four groups (IQ1_S
                // sub-block) or two (IQ1_M scale group), adjacent columns.
                double e = group_error64<kChunk>(src, zero_block, sq, idx, cs, d);
                e += __shfl_xor(e, 1);
                if (!kM) e += __shfl_xor(e, 2);
                if (it == 0) { idx_alt = idx; err_alt = e; continue; }
                if (near && (err_alt < e || (err_alt == e && c2 < cstar))) {
                    ch = c2;
                    cs = kM ? ch + 8 * (int)((shbits >> ch) & 1u) : ch;
                    idx = idx_alt;
                }
            }
            if (kMode == kModeCandidates) {
                // One lane per group writes its 8 errors xhat - x (xhat exact
                // in fp32, one rounding), its code and, once per choice group,
                // the choice.
                if (zero_scale) idx = 0;
                if (kb == 0) {
                    const int unit = kM ? (g >> 1) : sub;
                    const int part = kM ? (g & 1) : lq;
                    const int64_t base = (blk * kGroups + unit) * a.top_c + it;    // [block][unit][r]
                    float xo[8], wo[8];
                    src.load(rejected, xo, wo);
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
                    float4* ep = reinterpret_cast<float4*>(a.cand_err + base * (256 / kGroups) + part * 8);
                    ep[0] = make_float4(ev[0], ev[1], ev[2], ev[3]);
                    ep[1] = make_float4(ev[4], ev[5], ev[6], ev[7]);
                    if (part == 0) a.cand_choice[base] = ch;
                    if (a.cand_codes) {
                        const int shc = (kM && !zero_scale) ? (cs >> 3) : 0;
                        const uint16_t code = kM ? (uint16_t)(idx | (shc << 11)) : (uint16_t)idx;
                        a.cand_codes[base * (kM ? 2 : 4) + part] = rejected ? (uint16_t)0 : code;
                    }
                }
                continue;
            }
            // every choice: payload it; otherwise the one payload
            uint8_t* ob = sout + ((kMode == kModeEvery ? it : 0) * kBlocksPerWG + slot) * kBB;
            if (kM) {
                // IQ1_M: low byte per group; one nibble per group (3 high
                // bits, shift bit); four scale words with the 3-bit local
                // scales of four scale groups and one nibble of d each.
                const int nib = ((idx >> 8) & 7) | ((cs >> 3) << 3);
                const int nib_odd = __shfl_xor(nib, 1);
                int kk = (cs & 7) << (3 * ((g >> 1) & 3));
                kk |= __shfl_xor(kk, 2);
                kk |= __shfl_xor(kk, 4);
                if (!zero_block && kb == 0) {
                    ob[g] = (uint8_t)(idx & 0xff);
                    if ((g & 1) == 0) ob[32 + (g >> 1)] = (uint8_t)(nib | (nib_odd << 4));
                    if ((g & 7) == 0) {
                        const int wd = g >> 3;
                        const uint32_t v = (uint32_t)kk | (((dh >> (4 * wd)) & 0xfu) << 12);
                        ob[48 + 2 * wd] = (uint8_t)(v & 0xff);
                        ob[49 + 2 * wd] = (uint8_t)(v >> 8);
                    }
                }
            } else {
                // IQ1_S: low byte per group, qh word per sub-block, d per block.
                int hi = ((idx >> 8) & 7) << (3 * lq);
                hi |= __shfl_xor(hi, 1);
                hi |= __shfl_xor(hi, 2);
                if (!zero_block && kb == 0) {
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
        // Copy the staged payloads out and clear what was copied (each word
        // by the thread that copied it) for the next set.
        __syncthreads();
        const int64_t first = set * kBlocksPerWG;
        const int64_t left = a.g.nblocks - first;
        const int nb = left < kBlocksPerWG ? (int)left : kBlocksPerWG;
        for (int cs = 0; cs < kPayloads; ++cs) {
            uint16_t* o16 = reinterpret_cast<uint16_t*>(a.out + (cs * a.g.nblocks + first) * kBB);
            uint16_t* s16 = sout16 + cs * kBlocksPerWG * (kBB / 2);
            // An opaque copy of the thread index: the offsets derived from it are
            // recomputed here rather than held (and spilled) across the sets.
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

// ---------------------------------------------------------------------------
// IQ1_S payload encode and fake quant in 32 x 32 matrix tiles: a wave owns a
// whole block.
//
// v_mfma_f32_32x32x16_bf16 takes the block's 32 groups as the columns and 32
// grid entries as the rows (the lane holds 16 of them), so each group is
// covered by two lanes instead of four.  Two operand tables, (q+1/8)^2 and q,
// in LDS; per tile,
// V = -2*sum(wx*q)/d and U(+1/8) from two products each (the group side's
// three exact bf16 parts in the two K halves of the first product and the
// first K half of the second), the 8 keys of shift +1/8 folded, then
// U(-1/8) = U(+1/8) + sum(q*(-w/2)) by two more products on the same
// accumulator, and the 8 keys of shift -1/8.
// ---------------------------------------------------------------------------
constexpr int kW1Tile = 32;
constexpr int kW1ChunkTiles = 4;                       // 128-entry chunks (16 for 2048 entries)
constexpr int kW1Chunk = kW1Tile * kW1ChunkTiles;
constexpr int kW1Slots = kMaxGrid + kMaxGrid / kW1Chunk;

// The 8 keys (2k+1)*U + V of the lane's 16 entries for k = 0..7 folded into
// best[kBase + k] (a tree of three-input minima).
template <int kBase>
__device__ __forceinline__ void fold_wide8(const v16f& u, const v16f& v, float (&best)[16])
{
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float mk = (float)(2 * k + 1);
        float key[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) key[r] = __builtin_fmaf(u[r], mk, v[r]);
        const float a0 = fminf(fminf(key[0], key[1]), key[2]);
        const float a1 = fminf(fminf(key[3], key[4]), key[5]);
        const float a2 = fminf(fminf(key[6], key[7]), key[8]);
        const float a3 = fminf(fminf(key[9], key[10]), key[11]);
        const float a4 = fminf(fminf(key[12], key[13]), key[14]);
        const float a5 = fminf(fminf(key[15], best[kBase + k]), a0);
        best[kBase + k] = fminf(fminf(fminf(fminf(a1, a2), a3), a4), a5);
    }
}

// VALU rescan for choice cs = k + 8*deltabit over rows v0 .. v0+nv-1 of half
// hs in the tiles of chunk `chunk`: the lowest entry with the least key
// (2k+1)*U - 2V/d, recomputed in fp32 from the group's values and weights.
template <class GS>
__device__ __forceinline__ int rescan_w1(const uint4* __restrict__ sq, int chunk, int hs, int v0,
                                         int nv, int cs, const GS& src, bool zero_block, float w64,
                                         float b4, float inv_d, float* key_out)
{
    float x[8], w[8];
    __asm__ volatile("" ::: "memory");
    src.load(zero_block, x, w);
    const float mk = (float)(2 * (cs & 7) + 1);
    const float dl = (cs >> 3) ? -0.25f : 0.25f;      // 2*delta
    const float bd = (cs >> 3) ? b4 : -b4;
    int idx = -1;
    float vbest = 0.0f;
    for (int tt = 0; tt < kW1ChunkTiles; ++tt) {
        for (int v = v0; v < v0 + nv; ++v) {
            const int e = kW1Tile * (chunk * kW1ChunkTiles + tt) + 8 * (v >> 2) + 4 * hs + (v & 3);
            const uint4 u = sq[e + chunk];
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
    *key_out = vbest;
    return idx;
}

// fp64 error of group g against entry e under choice cs (as group_error64,
// with the wide kernel's table skew).
template <class GS>
__device__ __forceinline__ double group_error64_w1(const GS& src, bool zero, const uint4* sq, int e,
                                                   int cs, float d)
{
    float x[8], w[8];
    src.load(zero, x, w);
    const uint4 u = sq[e + e / kW1Chunk];
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

// kFmt: IQ_FMT_IQ1_S (payload or fake quant) or IQ_FMT_IQ1_M (payload);
// kMode: kModePayload or kModeFake; kDT: the weight's iq_dtype_t.
template <int kFmt, int kMode, int kDT>
__global__ __launch_bounds__(kThreads) void iq1s_payload_wide_kernel(Iq1sArgs a)
{
    // IQ1_M: 56-byte blocks, a local scale per two groups (16 choice groups
    // of 8 choices), the shift free per group.
    constexpr bool kM = kFmt == IQ_FMT_IQ1_M;
    constexpr int kBB = kM ? kBlockBytesM : kBlockBytes;
    constexpr int kCG = kM ? 16 : 8;         // choice groups per block
    constexpr int kNC = kM ? 8 : 16;         // choices per choice group
    __shared__ uint4 wsp[kW1Slots];                    // (q[0..7] + 1/8)^2 as bf16
    __shared__ uint4 wsq[kW1Slots];                    // q[0..7] as bf16
    __shared__ uint16_t sout16[kWavesPerWG * kBB / 2];   // the set's payloads
    __shared__ int sgrid_bad;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: block pointers in SGPRs
    const int n = a.grid_size;
    const int nchunks = (n + kW1Chunk - 1) / kW1Chunk;
    const int npad = nchunks * kW1Chunk;

    if (tid == 0) sgrid_bad = 0;
    for (int i = tid; i < kWavesPerWG * kBB / 2; i += kThreads) sout16[i] = 0;
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
            const int at = e + e / kW1Chunk;
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
    const int64_t blk = set * kWavesPerWG + wave;
    if (blk < a.g.nblocks) {                    // wave-uniform
        int ln = lane;                          // opaque: lane offsets are formed per block
        __asm__ volatile("" : "+v"(ln));
        const int g = ln & 31;                  // group = matrix column
        const int hl = ln >> 5;                 // K half / row half
        const int sub = g >> 2;
        const int lq = g & 3;
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
        if (a.choices) {
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

        // chunk_of: 4-bit chunk index of choice c in bits 4*(c%8) of word c/8.
        float best[16], snap[16];
        uint32_t chunk_of[2] = {0u, 0u};
#pragma unroll
        for (int c = 0; c < 16; ++c) { best[c] = __builtin_inff(); snap[c] = best[c]; }
        const v16f zero16 = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f,
                             0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        for (int ch = 0; ch < nchunks; ++ch) {
            for (int tt = 0; tt < kW1ChunkTiles; ++tt) {
                const int at = (ch * kW1ChunkTiles + tt) * kW1Tile + g + ch;
                const v8bf ap = as_v8bf(wsp[at]), aq = as_v8bf(wsq[at]);
                const v16f vq = mfma32(aq, on2, mfma32(aq, on1, zero16));
                v16f uu = mfma32(ap, ow2, mfma32(ap, ow1, zero16));
                fold_wide8<0>(uu, vq, best);
                uu = mfma32(aq, oh2, mfma32(aq, oh1, uu));          // U(-1/8)
                fold_wide8<8>(uu, vq, best);
            }
            const uint32_t chrep = (uint32_t)ch * 0x11111111u;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const uint32_t msk = best[c] < snap[c] ? (0xfu << (4 * (c & 7))) : 0u;
                chunk_of[c >> 3] = (chunk_of[c >> 3] & ~msk) | (chrep & msk);
                snap[c] = best[c];
            }
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

        // Entry for choice cs: the lane of the column whose minimum is least
        // holds it; the two lanes split its entries of the chunk.  With equal
        // minima in the two lanes of any column, every lane rescans its own
        // entries and the lane of least minimum, then lowest entry, wins.
        auto pick = [&](int cs) -> int {
            float lm = best[0];
#pragma unroll
            for (int c = 1; c < 16; ++c)
                if (cs == c) lm = best[c];
            const int tchunk = (int)((chunk_of[cs >> 3] >> (4 * (cs & 7))) & 0xfu);
            const float om = __shfl(lm, ln2 ^ 32);
            const bool tie = __ballot(om == lm) != 0;                // wave-uniform
            int idx;
            float key;
            if (!tie) {
                const int hs = (om < lm) ? (hl2 ^ 1) : hl2;             // holder half
                const int tch = __shfl(tchunk, g2 + 32 * hs);
                idx = rescan_w1(wsq, tch, hs, 8 * hl2, 8, cs, src2, zero_block, w64, b4, inv_d, &key);
                const float ok = __shfl(key, ln2 ^ 32);
                const int oi = __shfl(idx, ln2 ^ 32);
                if (ok < key || (ok == key && oi < idx)) { key = ok; idx = oi; }
            } else {
                idx = rescan_w1(wsq, tchunk, hl2, 0, 16, cs, src2, zero_block, w64, b4, inv_d, &key);
                const int oi = __shfl(idx, ln2 ^ 32);
                if (om < lm || (om == lm && oi < idx)) idx = oi;
            }
            return idx < n ? idx : n - 1;
        };

        // IQ1_M: the (k, shift) choice of this group under its scale group's k
        auto full = [&](int k) { return kM ? k + 8 * (int)((shbits >> k) & 1u) : k; };
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
            double e2 = group_error64_w1(src2, zero_block, wsq, i2, cs2, d);
            double e1 = group_error64_w1(src2, zero_block, wsq, i1, cs, d);
            e2 += quad_xchg<kQuadXor1>(e2);
            e1 += quad_xchg<kQuadXor1>(e1);
            if (!kM) {
                e2 += quad_xchg<kQuadXor2>(e2);
                e1 += quad_xchg<kQuadXor2>(e1);
            }
            idx = i1;
            if (near && (e2 < e1 || (e2 == e1 && c2 < cstar))) { ch = c2; cs = cs2; idx = i2; }
        }

        if (kM) {
            // IQ1_M: low byte per group; one nibble per group (3 high bits,
            // shift bit); four scale words with the 3-bit local scales of four
            // scale groups and one nibble of d each.
            const int nib = ((idx >> 8) & 7) | ((cs >> 3) << 3);
            const int nib_odd = quad_xchg<kQuadXor1>(nib);
            int kk = (ch & 7) << (3 * ((g2 >> 1) & 3));
            kk |= quad_xchg<kQuadXor2>(kk);
            kk |= __shfl(kk, ln2 ^ 4);
            if (!zero_block && hl2 == 0) {
                uint8_t* ob = reinterpret_cast<uint8_t*>(sout16) + wave * kBB;
                ob[g2] = (uint8_t)(idx & 0xff);
                if ((g2 & 1) == 0) ob[32 + (g2 >> 1)] = (uint8_t)(nib | (nib_odd << 4));
                if ((g2 & 7) == 0) {
                    const int wd = g2 >> 3;
                    const uint32_t v = (uint32_t)kk | (((dh >> (4 * wd)) & 0xfu) << 12);
                    ob[48 + 2 * wd] = (uint8_t)(v & 0xff);
                    ob[49 + 2 * wd] = (uint8_t)(v >> 8);
                }
            }
        }
        // IQ1_S: low byte per group, qh word per sub-block, d per block.
        int hi = ((idx >> 8) & 7) << (3 * lq2);
        hi |= quad_xchg<kQuadXor1>(hi);
        hi |= quad_xchg<kQuadXor2>(hi);
        if (!kM && !zero_block && hl2 == 0) {
            uint8_t* ob = reinterpret_cast<uint8_t*>(sout16) + wave * kBB;
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
            const uint4 u = wsq[ez + ez / kW1Chunk];
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
    if (a.out) {
        // Copy the set's payloads out and clear what was copied (each word by
        // the thread that copied it) for the next set.
        __syncthreads();
        const int64_t first = set * kWavesPerWG;
        const int64_t left = a.g.nblocks - first;
        const int nb = left < kWavesPerWG ? (int)left : kWavesPerWG;
        uint16_t* o16 = reinterpret_cast<uint16_t*>(a.out + first * kBB);
        int t0 = tid;
        __asm__ volatile("" : "+v"(t0));
        for (int i = t0; i < nb * (kBB / 2); i += kThreads) {
            o16[i] = sout16[i];
            sout16[i] = 0;
        }
    }
    }
}

template <int kFmt, int kDT>
hipError_t launch_fmt(const Iq1sArgs& a, int mode, hipStream_t stream)
{
    // One workgroup per compute unit (the LDS holds one), or one per set of
    // 16 blocks when there are fewer sets.
    const int64_t sets = (a.g.nblocks + kBlocksPerWG - 1) / kBlocksPerWG;
    const dim3 grid((unsigned)(sets < a.g.cus ? sets : a.g.cus));
    // The payload (both formats) and IQ1_S fake quant run the 32 x 32 kernel;
    // every choice, candidates and IQ1_M fake quant the 16 x 16 one.
    if (mode == kModeEvery) {
        hipLaunchKernelGGL((iq1s_encode_kernel<kFmt, kModeEvery, kDT>), grid, dim3(kThreads), 0,
                           stream, a);
    } else if (mode == kModeFake) {
        if constexpr (kFmt == IQ_FMT_IQ1_S)
            hipLaunchKernelGGL((iq1s_payload_wide_kernel<kFmt, kModeFake, kDT>), grid,
                               dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((iq1s_encode_kernel<kFmt, kModeFake, kDT>), grid, dim3(kThreads), 0,
                               stream, a);
    } else if (mode == kModeCandidates) {
        hipLaunchKernelGGL((iq1s_encode_kernel<kFmt, kModeCandidates, kDT>), grid, dim3(kThreads),
                           0, stream, a);
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
