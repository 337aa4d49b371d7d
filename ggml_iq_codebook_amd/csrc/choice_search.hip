// choice_search.hip -- local-Hessian choice search of 256-column blocks on
// gfx950, in one launch.
//
// The method (NVIDIA Model-Optimizer, "[1/4] Calibrate GGML IQ formats with
// local_hessian" #3158, steps 2-3; "[4/4] Run the local-Hessian choice search
// as one CUDA kernel" #3218): every group of a row has C candidate error
// vectors e_gc (from the every-choice encode); step 2 gives each group the
// candidate with the least e^T H_gg e; step 3 visits the groups twice, in
// order, and moves a group to the candidate that most lowers the row's
// e^T H e with the others held, if it lowers it at all.  With r = H e, the
// change of the row's objective when group g takes candidate c is
// score_c - score_cur, score_c = e_c^T H_gg e_c + 2 e_c^T (r_g - H_gg e_cur).
//
// Layout: a 512-thread workgroup runs 16 rows of one block in lockstep
// (grid.y = the block), with two kinds of waves.  First e_c^T H_gg e_c for
// every candidate, on the matrix cores (v_mfma_f32_16x16x4_f32, fp32
// operands, all eight waves).  Then the sweeps, one workgroup barrier per
// step.  With the groups visited in order, the rest of group g,
// r_g - H_gg e_cur,g = sum over h != g of H_g,h e_h, is the partial sum over
// h outside {g-1, g}, which waves 0-3 form on the matrix cores during the
// step before (each its quarter of K, from the current errors held
// row-major in LDS), plus H_g,g-1 e_g-1 with the errors just decided for
// g-1, which waves 4-7 add themselves.  Waves 4-7 decide, one lane per
// (row, candidate), lane (row, i) also owning column i of the row's rest:
// the lane adds the four partials and the late term for its column, the
// row's rest reaches the lanes of the row by DPP broadcasts, each lane scores
// its candidate from its own error vector, and one DPP reduction across the
// row's 16 lanes gives the lowest index of least score, the current pick
// winning the ties it is in (each lane keeps a bit mask of the groups whose
// pick is its candidate).  A row whose pick moves writes its new errors into
// the error rows.  The partial sums alternate between two buffers, so the
// products of the next group run beside the decision of the current one.
// H operands and candidate vectors are requested two steps ahead; the blocks
// H_g,g-1 are staged in LDS.

#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace iqk {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kProdWaves = 4;    // waves 0-3: products with H; waves 4-7: decisions
constexpr int kRows = 16;        // rows per workgroup
constexpr int kMaxC = 16;

typedef float v4f __attribute__((ext_vector_type(4)));

struct SearchArgs {
    const float* H;          // [nblk][256][256]
    const float* cand;       // [rows][nblk][G][C][L]
    int32_t* picks;          // [rows][nblk][G]
    int32_t* trace;          // NULL or [sweeps+1][rows][nblk][G]
    int64_t rows;
    int64_t nblk;
    int C, sweeps;
};

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Lane exchange within a row of 16 lanes (DPP): rotate by 8 or 4, swap with
// the lane 2 or 1 away inside a quad, or take lane j of the row.  Every lane
// has a source lane in these patterns.
template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xf, 0xf, true);
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, dpp_i<kCtrl>(__builtin_bit_cast(int, v)));
}

constexpr int kRor8 = 0x128, kRor4 = 0x124, kXor2 = 0x4e, kXor1 = 0xb1;

// An integer whose signed order is the order of the float scores (-0 counted
// as +0, so equal scores keep equal keys).
__device__ __forceinline__ int score_key(float v)
{
    const int b = __builtin_bit_cast(int, v + 0.0f);
    return b ^ (int)((uint32_t)(b >> 31) >> 1);
}

// Least key over the 16 lanes of a row; every lane of the row ends with it
// (the four steps reach lanes +8, +4, ^2, ^1 away, which together cover the
// row).
__device__ __forceinline__ int row_min(int v)
{
    v = min(v, dpp_i<kRor8>(v));
    v = min(v, dpp_i<kRor4>(v));
    v = min(v, dpp_i<kXor2>(v));
    return min(v, dpp_i<kXor1>(v));
}

// d[j % 4] += (value of lane j of the row) * c[j], j = 0..15: sixteen FMAs
// whose first operand comes by DPP row broadcast.  The leading s_nop covers
// the wait states between a VALU write of v and its first DPP read.
__device__ __forceinline__ void dot_row16(float v, const float* c, float (&d)[4])
{
    __asm__("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, %4, %5 row_newbcast:0 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %1, %4, %6 row_newbcast:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %2, %4, %7 row_newbcast:2 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %3, %4, %8 row_newbcast:3 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %0, %4, %9 row_newbcast:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %1, %4, %10 row_newbcast:5 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %2, %4, %11 row_newbcast:6 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %3, %4, %12 row_newbcast:7 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %0, %4, %13 row_newbcast:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %1, %4, %14 row_newbcast:9 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %2, %4, %15 row_newbcast:10 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %3, %4, %16 row_newbcast:11 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %0, %4, %17 row_newbcast:12 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %1, %4, %18 row_newbcast:13 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %2, %4, %19 row_newbcast:14 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %3, %4, %20 row_newbcast:15 row_mask:0xf bank_mask:0xf bound_ctrl:1"
            : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3])
            : "v"(v), "v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]), "v"(c[4]), "v"(c[5]), "v"(c[6]),
              "v"(c[7]), "v"(c[8]), "v"(c[9]), "v"(c[10]), "v"(c[11]), "v"(c[12]), "v"(c[13]),
              "v"(c[14]), "v"(c[15]));
}

template <int L>
__global__ __launch_bounds__(kThreads) void choice_search_kernel(SearchArgs a)
{
    constexpr int G = 256 / L;
    constexpr int KH = L / 16;                  // 16-column tiles per group
    // LDS rows are padded (and stay 16-byte aligned) so that the lanes of a
    // wave reading rows, blocks or columns together fall in different banks.
    constexpr int kHR = L + 4;                  // H block row stride
    constexpr int kHB = L * kHR + 4;            // H block stride
    constexpr int kER = 256 + 4;                // error row stride
    constexpr int kQS = G * kMaxC + 16;         // qself row stride
    constexpr int kPR = L + 4;                  // partial rest row stride
    constexpr int kPB = kProdWaves * kRows * kPR;   // one partial buffer
    // H_gg for step 2, then H_g,g-1 for the sweeps
    __shared__ __align__(16) float hblk[G * kHB];
    __shared__ __align__(16) float ecur[kRows * kER];     // current errors, [row][column]
    __shared__ __align__(16) float part[2 * kPB];         // [buffer][wave][row][i]
    __shared__ __align__(16) float qself[kRows * kQS];    // e_gc^T H_gg e_gc, [row][g*C + c]
    __shared__ int pick0[kRows * G];                      // step-2 picks

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int lc = lane & 15;                   // matrix column
    const int lq = lane >> 4;                   // K slot / row quarter
    const int C = a.C;
    const int64_t row0 = (int64_t)blockIdx.x * kRows;
    const int nrows = (int)((a.rows - row0) < kRows ? (a.rows - row0) : kRows);
    const int64_t blk = blockIdx.y;
    const float* __restrict__ Hb = a.H + blk * 65536;
    const int64_t cstride = a.nblk * G * C * L;   // floats per row of cand
    const float* __restrict__ cb = a.cand + blk * (int64_t)G * C * L;
    auto out_index = [&](int64_t slot, int64_t row, int g) -> int64_t {
        return ((slot * a.rows + row) * a.nblk + blk) * G + g;
    };
    auto cand_ptr = [&](int rr, int g, int c) -> const float* {
        return cb + (row0 + rr) * cstride + ((int64_t)g * C + c) * L;
    };
    // H block (g, gx) as [i][j] = H[g*L + i][gx*L + j] into hblk, 16 bytes
    // a thread at a time, every load requested before the first store.
    auto stage_blocks = [&](bool sub) {
        constexpr int kU = G * L * L / 4 / kThreads;            // float4 per thread
        float4 v[kU];
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            const int u = t + kThreads * k;
            const int g = u / (L * L / 4), rem = u % (L * L / 4), ii = rem / (L / 4), j4 = rem % (L / 4);
            const int gx = sub ? (g + G - 1) % G : g;
            v[k] = *reinterpret_cast<const float4*>(&Hb[(g * L + ii) * 256 + gx * L + 4 * j4]);
        }
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            const int u = t + kThreads * k;
            const int g = u / (L * L / 4), rem = u % (L * L / 4), ii = rem / (L / 4), j4 = rem % (L / 4);
            *reinterpret_cast<float4*>(&hblk[g * kHB + ii * kHR + 4 * j4]) = v[k];
        }
    };

    // e_gc^T H_gg e_gc on the matrix cores (all waves): for group g and 16
    // (row, cand) columns n, Y = H_gg E^T (lane: rows 4lq..4lq+3 of each
    // 16-row block of Y, column n = lc), then the column's dot with E, summed
    // over the four lanes of the column.  The K order of the products is
    // permuted (step s of a 16-wide K block takes k = 4lq + s) so that a
    // lane's four operands of a block are the four values of E it also needs
    // for the dot: one 16-byte load per block.  Jobs (group, 16 columns) are
    // spread over the waves and taken kJB at a time, the next batch requested
    // before the current one is used.
    {
        constexpr int kJB = 8;
        const int ntile = C;                      // 16*C (row, cand) columns in tiles of 16
        const int njobs = G * ntile;
        // v / C for 0 <= v < 2^16 without an integer divide: (v + 1/2)/C lies
        // at least 1/(2C) away from an integer, far beyond the float error.
        const float invC = 1.0f / (float)C;
        auto divC = [&](int v) { return (int)(((float)v + 0.5f) * invC); };
        float4 Ec[kJB][KH], En[kJB][KH];
        auto load_batch = [&](int j0, float4 (&E)[kJB][KH]) {
#pragma unroll
            for (int b = 0; b < kJB; ++b) {
                const int job = j0 + kWaves * b;
                const int g = divC(job), n = (job - g * C) * 16 + lc;
                const int rr = divC(n), c = n - rr * C;
                const bool live = job < njobs && rr < nrows;
                const float4* ep = live ? reinterpret_cast<const float4*>(cand_ptr(rr, g, c)) : nullptr;
#pragma unroll
                for (int h = 0; h < KH; ++h)
                    E[b][h] = live ? ep[4 * h + lq] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        };
        // The first batch is requested before the diagonal blocks of H are
        // staged, so the two reads overlap.
        load_batch(wave, Ec);
        stage_blocks(false);
        __syncthreads();
        for (int j0 = wave; j0 < njobs; j0 += kWaves * kJB) {     // wave-uniform
            load_batch(j0 + kWaves * kJB, En);
            float qv[kJB];
#pragma unroll
            for (int b = 0; b < kJB; ++b) {
                const int job = j0 + kWaves * b;
                const int g = divC(job < njobs ? job : 0);
                float q = 0.0f;
#pragma unroll
                for (int ih = 0; ih < KH; ++ih) {                  // rows 16ih.. of Y
                    v4f y = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int kh = 0; kh < KH; ++kh) {
                        const float* hr = &hblk[g * kHB + (16 * ih + lc) * kHR + 16 * kh + 4 * lq];
                        const float4 e4 = Ec[b][kh];
                        y = mfma4(hr[0], e4.x, y);
                        y = mfma4(hr[1], e4.y, y);
                        y = mfma4(hr[2], e4.z, y);
                        y = mfma4(hr[3], e4.w, y);
                    }
                    const float4 ed = Ec[b][ih];
                    q = __builtin_fmaf(ed.x, y[0], q);
                    q = __builtin_fmaf(ed.y, y[1], q);
                    q = __builtin_fmaf(ed.z, y[2], q);
                    q = __builtin_fmaf(ed.w, y[3], q);
                }
                qv[b] = q;
            }
            // The column sums over the four lanes of each column, all jobs of
            // the batch together.
#pragma unroll
            for (int b = 0; b < kJB; ++b) qv[b] += __shfl_xor(qv[b], 16);
#pragma unroll
            for (int b = 0; b < kJB; ++b) qv[b] += __shfl_xor(qv[b], 32);
#pragma unroll
            for (int b = 0; b < kJB; ++b) {
                const int job = j0 + kWaves * b;
                const int g = divC(job), n = (job - g * C) * 16 + lc;
                const int rr = divC(n);
                if (job < njobs && lq == 0) qself[rr * kQS + g * C + (n - rr * C)] = qv[b];
            }
#pragma unroll
            for (int b = 0; b < kJB; ++b)
#pragma unroll
                for (int h = 0; h < KH; ++h) Ec[b][h] = En[b][h];
        }
    }
    __syncthreads();

    // Step 2: each group's best candidate under its own block (lowest index on
    // ties), and the current errors as rows; the blocks H_g,g-1 replace H_gg.
    stage_blocks(true);
    for (int it = t; it < kRows * G; it += kThreads) {
        const int rr = it / G, g = it % G;
        int best = 0;
        for (int c = 1; c < C; ++c)
            if (qself[rr * kQS + g * C + c] < qself[rr * kQS + g * C + best]) best = c;
        pick0[rr * G + g] = best;
        const float4* ep = rr < nrows ? reinterpret_cast<const float4*>(cand_ptr(rr, g, best)) : nullptr;
#pragma unroll
        for (int i4 = 0; i4 < L / 4; ++i4)
            *reinterpret_cast<float4*>(&ecur[rr * kER + g * L + 4 * i4]) =
                ep ? ep[i4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    __syncthreads();
    if (a.trace)
        for (int it = t; it < nrows * G; it += kThreads)
            a.trace[out_index(0, row0 + it / G, it % G)] = pick0[it];

    const bool prod = wave < kProdWaves;        // wave-uniform

    if (prod) {
        // ---------------- product waves ----------------
        // During step g the wave forms its partial rest of group gn = g+1 for
        // the 16 rows: K range 64w .. 64w + 63 in steps of 4 (k = 64w + 4s +
        // lq), the columns of gn and g left out.  Output tile ih holds the
        // columns gn*L + 16ih .. + 15 (lane: columns 4lq..4lq+3 of the tile,
        // row lc); the tiles go to partial buffer (g+1)%2 as [row][column].
        // The H operands (H symmetric: H[k][column]) are requested a step
        // ahead.
        constexpr int kPS = 16;                 // K steps per wave
        constexpr int kGW = 64 / L;             // groups in the wave's K range
        float hP[KH][kPS], hPn[KH][kPS];        // H[64w + 4s + lq][gn*L + 16ih + lc]
        // The wave's B operands, e[row lc][64w + 4s + lq], kept between steps:
        // only the group decided last can have changed.
        float bv[kPS];
#pragma unroll
        for (int s = 0; s < kPS; ++s) bv[s] = ecur[lc * kER + 64 * wave + 4 * s + lq];
        auto load_hP = [&](int gn, float (&h)[KH][kPS]) {
#pragma unroll
            for (int ih = 0; ih < KH; ++ih)
#pragma unroll
                for (int s = 0; s < kPS; ++s)
                    h[ih][s] = Hb[(64 * wave + 4 * s + lq) * 256 + gn * L + 16 * ih + lc];
        };
        auto pstep = [&](int gn, int gx, const float (&h)[KH][kPS], int buf) {
            // the group decided in the step before gx's, if in the wave's range
            const int gp = gx > 0 ? gx - 1 : G - 1;
#pragma unroll
            for (int q = 0; q < kGW; ++q) {
                if (kGW * wave + q == gp) {                         // wave-uniform
#pragma unroll
                    for (int s = q * (L / 4); s < (q + 1) * (L / 4); ++s)
                        bv[s] = ecur[lc * kER + 64 * wave + 4 * s + lq];
                }
            }
            v4f pp[KH];
#pragma unroll
            for (int ih = 0; ih < KH; ++ih) pp[ih] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            // the wave's K range holds 64/L groups; those of gn and gx are left out
#pragma unroll
            for (int q = 0; q < kGW; ++q) {
                const int kg = kGW * wave + q;                      // wave-uniform
                if (kg != gn && kg != gx) {
#pragma unroll
                    for (int s = q * (L / 4); s < (q + 1) * (L / 4); ++s)
#pragma unroll
                        for (int ih = 0; ih < KH; ++ih) pp[ih] = mfma4(h[ih][s], bv[s], pp[ih]);
                }
            }
#pragma unroll
            for (int ih = 0; ih < KH; ++ih)
                *reinterpret_cast<v4f*>(&part[buf * kPB + (wave * kRows + lc) * kPR + 16 * ih + 4 * lq]) = pp[ih];
        };

        // The partial of group 0 (group G-1, decided last, left out).
        load_hP(0, hP);
        load_hP(1 % G, hPn);
        pstep(0, G - 1, hP, 0);
        load_hP(2 % G, hP);
        __syncthreads();                        // X: partial of group 0 in buffer 0
        // Step g: the partial of gn = g+1 with the operands requested two
        // steps before; the operands of the step after next go into the
        // registers just used.  Steps alternate between the two register sets.
        for (int sw = 0; sw < a.sweeps; ++sw) {
#pragma unroll 1
            for (int g = 0; g < G; g += 2) {    // G is even
                pstep(g + 1, g, hPn, 1);
                load_hP((g + 3) % G, hPn);
                __syncthreads();                // X_g
                pstep((g + 2) % G, g + 1, hP, 0);
                load_hP((g + 4) % G, hP);
                __syncthreads();                // X_g+1
            }
        }
    } else {
        // ---------------- decision waves ----------------
        // Lane (srow, scand); pmask bit g = group g's pick is scand.  The lane
        // also owns columns scand + 16h of its row's rest.
        const int dt = t - 64 * kProdWaves;
        const int srow = dt >> 4;
        const int scand = dt & 15;
        const bool scorer = scand < C && srow < nrows;
        uint32_t pmask = 0u;
        for (int g = 0; g < G; ++g) pmask |= (uint32_t)(pick0[srow * G + g] == scand) << g;
        float cv[L], cvn[L];
        // Every lane loads a vector: a lane past the row's candidates or the
        // block's rows reads a real one (its values are never scored).
        const float* cbase = cand_ptr(srow < nrows ? srow : nrows - 1, 0, scand < C ? scand : C - 1);
        auto load_cv = [&](int g, float (&v)[L]) {
            const float4* ep = reinterpret_cast<const float4*>(cbase + g * C * L);
#pragma unroll
            for (int i4 = 0; i4 < L / 4; ++i4) {
                const float4 u = ep[i4];
                v[4 * i4] = u.x; v[4 * i4 + 1] = u.y; v[4 * i4 + 2] = u.z; v[4 * i4 + 3] = u.w;
            }
        };
        // H_g,g-1 e_g-1 for the lane's columns of group g, from the errors
        // of g-1 in the error rows (the lanes of a row read the same row).
        // The lane's row of H_g,g-1 (row scand + 16h), read at the start of
        // the step whose late term it serves, beside the partials.
        auto load_hrow = [&](int g, float4 (&hv)[KH][L / 4]) {
#pragma unroll
            for (int h = 0; h < KH; ++h) {
                const float* hr = &hblk[g * kHB + (scand + 16 * h) * kHR];
#pragma unroll
                for (int j4 = 0; j4 < L / 4; ++j4) hv[h][j4] = *reinterpret_cast<const float4*>(hr + 4 * j4);
            }
        };
        auto late = [&](int g, float (&lr)[KH], const float4 (&hv)[KH][L / 4]) {
            const int gp = g > 0 ? g - 1 : G - 1;
            const float* er = &ecur[srow * kER + gp * L];
#pragma unroll
            for (int h = 0; h < KH; ++h) {
                float d4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int j4 = 0; j4 < L / 4; ++j4) {
                    const float4 h4 = hv[h][j4];
                    const float4 e4 = *reinterpret_cast<const float4*>(er + 4 * j4);
                    d4[0] = __builtin_fmaf(h4.x, e4.x, d4[0]);
                    d4[1] = __builtin_fmaf(h4.y, e4.y, d4[1]);
                    d4[2] = __builtin_fmaf(h4.z, e4.z, d4[2]);
                    d4[3] = __builtin_fmaf(h4.w, e4.w, d4[3]);
                }
                lr[h] = (d4[0] + d4[1]) + (d4[2] + d4[3]);
            }
        };
        float lr[KH];
        const int qc = scand < C ? scand : 0;
        float qnext = qself[srow * kQS + qc];     // group 0
        float4 hv[KH][L / 4];
        load_cv(0, cv);
        load_cv(1 % G, cvn);
        load_hrow(0, hv);
        late(0, lr, hv);
        __syncthreads();                        // X: partial of group 0 in buffer 0
        // Step g: group g decided with its candidate vector requested two
        // steps before (cur); once it is used, the vector of the group after
        // next goes into the same registers.  Its late term
        // (lr, formed in the step before) and the four partials give the
        // rest; after the decision the row's errors of g are current in the
        // error rows, and the late term of the next group follows.
        auto dstep = [&](int g, float (&cur)[L]) {
            const int gn = g + 1 < G ? g + 1 : 0;
            const int g2 = gn + 1 < G ? gn + 1 : 0;
            // e_c^T H_gg e_c of this step's group, read during the step
            // before; the next group's is requested now.
            const float qs = qnext;
            qnext = qself[srow * kQS + gn * C + qc];
            load_hrow(gn, hv);
            const float* pb = part + (g & 1) * kPB;
            float r[KH];
#pragma unroll
            for (int h = 0; h < KH; ++h) {
                const int i = scand + 16 * h;
                float v = pb[(0 * kRows + srow) * kPR + i];
#pragma unroll
                for (int w = 1; w < kProdWaves; ++w) v += pb[(w * kRows + srow) * kPR + i];
                r[h] = v + lr[h];
            }
            // The candidate's dot with the row's rest: column j of tile h
            // comes from lane j of the row (DPP row broadcast).  Lanes that
            // score nothing keep the largest key, above any score's.
            int key;
            {
                float d4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int h = 0; h < KH; ++h) dot_row16(r[h], &cur[16 * h], d4);
                const float dot = (d4[0] + d4[1]) + (d4[2] + d4[3]);
                const float sc = __builtin_fmaf(2.0f, dot, qs);
                const int sk = sc == sc ? score_key(sc) : 0x7ffffffe;   // a NaN after every number
                key = scorer ? sk : 0x7fffffff;
            }
            // The least score of the row (DPP), then the row's lanes that
            // hold it (a ballot, 16 bits per row): the group keeps its pick if
            // the pick holds it (only a strictly lower score moves it), else
            // moves to the lowest candidate that does.
            const bool mine = (pmask >> g) & 1u;
            const int m = row_min(key);
            const int rsh = 16 * (lane >> 4);
            const uint32_t req = (uint32_t)(__ballot(key == m) >> rsh) & 0xffffu;
            const uint32_t rcur = (uint32_t)(__ballot(mine) >> rsh) & 0xffffu;
            const bool move = req != 0u && (req & rcur) == 0u;
            const int bc = __builtin_ctz(req | 0x10000u);
            // A row whose pick moves writes its new errors of group g.
            if (move && scand == bc) {
#pragma unroll
                for (int i4 = 0; i4 < L / 4; ++i4)
                    *reinterpret_cast<float4*>(&ecur[srow * kER + g * L + 4 * i4]) =
                        make_float4(cur[4 * i4], cur[4 * i4 + 1], cur[4 * i4 + 2], cur[4 * i4 + 3]);
            }
            if (move) pmask = (pmask & ~(1u << g)) | ((uint32_t)(scand == bc) << g);
            // The vector of the group after next, into the registers just
            // used (a wait for the next group's must not wait for it).
            load_cv(g2, cur);
            // the row's errors of g (written by this wave) before the late
            // term of gn reads them
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            late(gn, lr, hv);
            __syncthreads();                    // X_g: g decided, the partial of gn ready
        };
        for (int sw = 0; sw < a.sweeps; ++sw) {
#pragma unroll 1
            for (int g = 0; g < G; g += 2) {    // G is even
                dstep(g, cv);
                dstep(g + 1, cvn);
            }
            if (a.trace && srow < nrows)
                for (int g = 0; g < G; ++g)
                    if ((pmask >> g) & 1u) a.trace[out_index(sw + 1, row0 + srow, g)] = scand;
        }
        if (srow < nrows)
            for (int g = 0; g < G; ++g)
                if ((pmask >> g) & 1u) a.picks[((row0 + srow) * a.nblk + blk) * G + g] = scand;
    }
}

}  // namespace

hipError_t launch_choice_search(const float* H, const float* cand, int64_t rows, int64_t nblk,
                                int G, int C, int sweeps, int32_t* picks, int32_t* trace,
                                hipStream_t stream)
{
    SearchArgs a{H, cand, picks, trace, rows, nblk, C, sweeps};
    const dim3 grid((unsigned)((rows + kRows - 1) / kRows), (unsigned)nblk);
    if (G == 16)
        hipLaunchKernelGGL(choice_search_kernel<16>, grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(choice_search_kernel<32>, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace iqk
