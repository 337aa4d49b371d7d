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
// Layout: a 256-thread workgroup runs 16 rows of one block in lockstep
// (grid.y = the block).  The products with H run on the matrix cores
// (v_mfma_f32_16x16x4_f32, fp32 operands): e_c^T H_gg e_c for every
// candidate, and for each step the rest of the next group gn,
// r_gn - H_gn,gn e_gn = sum over the other groups h of H_gn,h e_h, formed
// afresh from the current errors (no running r = H e is kept): the four waves
// sum their quarters of K, leaving out gn and the group being decided, while
// that group is decided, and the wave of each of gn's 16-column tiles adds
// the decided group's part after.
// The decision runs in the scorer layout, lane (row, candidate) =
// (t/16, t%16): each lane scores its candidate from its own error vector and
// the row's rest; one DPP reduction across the row's 16 lanes gives the lowest
// index of least score, the current pick winning the ties it is in (each lane
// keeps a bit mask of the groups whose pick is its candidate).  Two barriers
// per step; the next step's H operands and candidate vectors are requested a
// step ahead.

#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace iqk {
namespace {

constexpr int kThreads = 256;
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

// Lane exchange within a row of 16 lanes (DPP): rotate by 8 or 4, or swap with
// the lane 2 or 1 away inside a quad.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 kCtrl, 0xf, 0xf, false));
}

constexpr int kRor8 = 0x128, kRor4 = 0x124, kXor2 = 0x4e, kXor1 = 0xb1;

// Least value over the 16 lanes of a row; every lane of the row ends with it
// (the four steps reach lanes +8, +4, ^2, ^1 away, which together cover the
// row).
__device__ __forceinline__ float row_min(float v)
{
    v = fminf(v, dpp_f<kRor8>(v));
    v = fminf(v, dpp_f<kRor4>(v));
    v = fminf(v, dpp_f<kXor2>(v));
    return fminf(v, dpp_f<kXor1>(v));
}

template <int L>
__global__ __launch_bounds__(kThreads) void choice_search_kernel(SearchArgs a)
{
    constexpr int G = 256 / L;
    constexpr int KS = L / 4;                   // matrix-core K steps per group
    constexpr int KH = L / 16;                  // 16-column tiles per group
    // LDS rows are padded (and stay 16-byte aligned) so that the lanes of a
    // wave reading rows, blocks or columns together fall in different banks.
    constexpr int kHR = L + 4;                  // H_gg row stride
    constexpr int kHB = L * kHR + 4;            // H_gg block stride
    constexpr int kQS = G * kMaxC + 16;         // qself row stride
    __shared__ __align__(16) float hdiag[G * kHB];        // H_gg blocks [g][i][j]
    __shared__ __align__(16) float ecurT[256 * kRows];      // current errors, [column][row]
    __shared__ __align__(16) float part[4 * KH * 64 * 4]; // the waves' partial rest tiles
    __shared__ __align__(16) float enew[L * kRows];       // the decided group's errors, [i][row]
    __shared__ __align__(16) float rest[kRows * kHR];     // r_g - H_gg e_cur,g, [row][i]
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

    for (int i = t; i < G * L * L; i += kThreads) {
        const int g = i / (L * L), rem = i % (L * L), ii = rem / L, jj = rem % L;
        hdiag[g * kHB + ii * kHR + jj] = Hb[(g * L + ii) * 256 + g * L + jj];
    }
    __syncthreads();

    // e_gc^T H_gg e_gc on the matrix cores: for group g and 16 (row, cand)
    // columns n, Y = H_gg E^T (lane: rows 4lq..4lq+3 of each 16-row block of
    // Y, column n = lc), then the column's dot with E, summed over the four
    // lanes of the column.  The K order of the products is permuted (step s of
    // a 16-wide K block takes k = 4lq + s) so that a lane's four operands of a
    // block are the four values of E it also needs for the dot: one 16-byte
    // load per block.  Jobs (group, 16 columns) are spread over the waves and
    // taken kJB at a time, the next batch requested before the current one is
    // used.
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
                const int job = j0 + 4 * b;
                const int g = divC(job), n = (job - g * C) * 16 + lc;
                const int rr = divC(n), c = n - rr * C;
                const bool live = job < njobs && rr < nrows;
                const float* ep = live ? cand_ptr(rr, g, c) : nullptr;
#pragma unroll
                for (int h = 0; h < KH; ++h) {
                    if (live) {
                        E[b][h] = make_float4(ep[16 * h + 4 * lq], ep[16 * h + 4 * lq + 1],
                                              ep[16 * h + 4 * lq + 2], ep[16 * h + 4 * lq + 3]);
                    } else {
                        E[b][h] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                    }
                }
            }
        };
        load_batch(wave, Ec);
        for (int j0 = wave; j0 < njobs; j0 += 4 * kJB) {           // wave-uniform
            load_batch(j0 + 4 * kJB, En);
            float qv[kJB];
#pragma unroll
            for (int b = 0; b < kJB; ++b) {
                const int job = j0 + 4 * b;
                const int g = divC(job < njobs ? job : 0);
                float q = 0.0f;
#pragma unroll
                for (int ih = 0; ih < KH; ++ih) {                  // rows 16ih.. of Y
                    v4f y = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int kh = 0; kh < KH; ++kh) {
                        const float* hr = &hdiag[g * kHB + (16 * ih + lc) * kHR + 16 * kh + 4 * lq];
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
                const int job = j0 + 4 * b;
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
    // ties), and the current errors as columns.
    for (int it = t; it < kRows * G; it += kThreads) {
        const int rr = it / G, g = it % G;
        int best = 0;
        for (int c = 1; c < C; ++c)
            if (qself[rr * kQS + g * C + c] < qself[rr * kQS + g * C + best]) best = c;
        pick0[rr * G + g] = best;
        const float* ep = rr < nrows ? cand_ptr(rr, g, best) : nullptr;
#pragma unroll
        for (int i = 0; i < L; ++i) ecurT[(g * L + i) * kRows + rr] = rr < nrows ? ep[i] : 0.0f;
    }
    __syncthreads();
    if (a.trace)
        for (int it = t; it < nrows * G; it += kThreads)
            a.trace[out_index(0, row0 + it / G, it % G)] = pick0[it];

    // Scorer layout: lane (srow, scand); pmask bit g = group g's pick is scand.
    const int srow = t >> 4;
    const int scand = t & 15;
    const bool scorer = scand < C && srow < nrows;
    uint32_t pmask = 0u;
    for (int g = 0; g < G; ++g) pmask |= (uint32_t)(pick0[srow * G + g] == scand) << g;

    // The rest of group gn for the 16 rows, r_gn - H_gn,gn e_gn: the sum over
    // the other groups h of H_gn,h e_h, formed afresh for every step on the
    // matrix cores (no running r = H e is kept).  Output tile ih holds the
    // columns gn*L + 16ih .. + 15 (lane: columns 4lq..4lq+3 of the tile, row
    // lc).  The part that does not depend on the group gx being decided runs
    // before its decision: wave w takes the K range 64w .. 64w + 63 in steps
    // of 4 (k = 64w + 4s + lq) with the columns of gn and gx left out, and puts
    // its partial tiles in LDS.  After the decision, wave ih adds the four
    // partials of tile ih in a fixed order, then H_gn,gx e_gx with the errors
    // just decided, and writes the rest.  The H operands (H symmetric:
    // H[k][column]) are requested a step ahead.
    constexpr int kPS = 16;                     // K steps per wave
    float hP[KH][kPS], hPn[KH][kPS];            // H[64w + 4s + lq][gn*L + 16ih + lc]
    float hX[KS], hXn[KS];                      // H[gx*L + 4s + lq][gn*L + 16w + lc], w < KH
    auto load_hP = [&](int gn, float (&h)[KH][kPS]) {
#pragma unroll
        for (int ih = 0; ih < KH; ++ih)
#pragma unroll
            for (int s = 0; s < kPS; ++s)
                h[ih][s] = Hb[(64 * wave + 4 * s + lq) * 256 + gn * L + 16 * ih + lc];
    };
    auto load_hX = [&](int gn, int gx, float (&h)[KS]) {
        if (wave >= KH) return;                                 // wave-uniform
#pragma unroll
        for (int s = 0; s < KS; ++s) h[s] = Hb[(gx * L + 4 * s + lq) * 256 + gn * L + 16 * wave + lc];
    };
    // The wave's partial tiles, columns of gn and gx (gx < 0: none) left out
    // (wave-uniform conditions).  The errors in LDS do not change while this
    // runs: a decision stages its group's new errors apart and they are copied
    // in after the next barrier.  All B operands are read before the products
    // start.
    auto partial = [&](int gn, int gx, v4f (&p)[KH]) {
        float bv[kPS];
#pragma unroll
        for (int s = 0; s < kPS; ++s) bv[s] = ecurT[(64 * wave + 4 * s + lq) * kRows + lc];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ih = 0; ih < KH; ++ih) p[ih] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < kPS; ++s) {
            const int kg = (64 * wave + 4 * s) / L;             // wave-uniform
            if (kg != gn && kg != gx) {
#pragma unroll
                for (int ih = 0; ih < KH; ++ih) p[ih] = mfma4(hP[ih][s], bv[s], p[ih]);
            }
        }
    };
    auto store_partial = [&](const v4f (&p)[KH]) {
#pragma unroll
        for (int ih = 0; ih < KH; ++ih)
            *reinterpret_cast<v4f*>(&part[((wave * KH + ih) * 64 + lane) * 4]) = p[ih];
    };
    auto finish_rest = [&](int gx) {
        if (wave >= KH) return;                                 // wave-uniform
        const int ih = wave;
        v4f d = *reinterpret_cast<const v4f*>(&part[(ih * 64 + lane) * 4]);
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            const v4f o = *reinterpret_cast<const v4f*>(&part[((w * KH + ih) * 64 + lane) * 4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) d[i] += o[i];
        }
        if (gx >= 0) {
#pragma unroll
            for (int s = 0; s < KS; ++s) d = mfma4(hX[s], enew[(4 * s + lq) * kRows + lc], d);
        }
        *reinterpret_cast<float4*>(&rest[lc * kHR + 16 * ih + 4 * lq]) =
            make_float4(d[0], d[1], d[2], d[3]);
    };

    // The first group's rest (no group being decided).
    v4f pp[KH];
    load_hP(0, hP);
    partial(0, -1, pp);
    store_partial(pp);
    __syncthreads();
    finish_rest(-1);

    // The step operands, one step ahead: the scorer's candidate vector and the
    // H operands of the next rest.
    float cv[L], cvn[L];
    auto load_cv = [&](int g, float (&v)[L]) {
        if (scorer) {
            const float* ep = cand_ptr(srow, g, scand);
#pragma unroll
            for (int i = 0; i < L; ++i) v[i] = ep[i];
        } else {
#pragma unroll
            for (int i = 0; i < L; ++i) v[i] = 0.0f;
        }
    };
    load_cv(0, cv);
    load_hP(1, hP);
    load_hX(1, 0, hX);
    __syncthreads();

    for (int sw = 0; sw < a.sweeps; ++sw) {
        for (int g = 0; g < G; ++g) {
            const int gn = g + 1 < G ? g + 1 : 0;
            const int gnn = gn + 1 < G ? gn + 1 : 0;
            load_cv(gn, cvn);
            // The next group's rest without group g, while group g is decided.
            partial(gn, g, pp);
            load_hP(gnn, hPn);
            load_hX(gnn, gn, hXn);
            // Scores, the decision and the error update of group g.
            float sc = __builtin_inff();
            if (scorer) {
                float dot = 0.0f;
#pragma unroll
                for (int i = 0; i < L; ++i) dot = __builtin_fmaf(cv[i], rest[srow * kHR + i], dot);
                sc = __builtin_fmaf(2.0f, dot, qself[srow * kQS + g * C + scand]);
            }
            // The least score of the row (DPP), then the row's lanes that hold
            // it (a ballot, 16 bits per row): the group keeps its pick if the
            // pick holds it (only a strictly lower score moves it), else moves
            // to the lowest candidate that does.
            const bool mine = (pmask >> g) & 1u;
            const float m = row_min(sc);
            const int rsh = 16 * (lane >> 4);
            const uint32_t req = (uint32_t)(__ballot(sc == m) >> rsh) & 0xffffu;
            const uint32_t rcur = (uint32_t)(__ballot(mine) >> rsh) & 0xffffu;
            const bool move = req != 0u && (req & rcur) == 0u;
            const int bc = __builtin_ctz(req | 0x10000u);
            // The row's new errors of group g (the new pick's, or the current
            // pick's when it stays), staged for the rest of gn.
            if (move ? scand == bc : mine) {
#pragma unroll
                for (int i = 0; i < L; ++i) enew[i * kRows + srow] = cv[i];
            }
            if (move) pmask = (pmask & ~(1u << g)) | ((uint32_t)(scand == bc) << g);
            store_partial(pp);
            __syncthreads();

            // The rest of gn with the errors of g just decided; the rows that
            // moved update their errors of g.
            finish_rest(g);
            if (move && scand == bc) {
#pragma unroll
                for (int i = 0; i < L; ++i) ecurT[(g * L + i) * kRows + srow] = cv[i];
            }
#pragma unroll
            for (int i = 0; i < L; ++i) cv[i] = cvn[i];
#pragma unroll
            for (int ih = 0; ih < KH; ++ih)
#pragma unroll
                for (int s = 0; s < kPS; ++s) hP[ih][s] = hPn[ih][s];
#pragma unroll
            for (int s = 0; s < KS; ++s) hX[s] = hXn[s];
            __syncthreads();
        }
        if (a.trace && srow < nrows)
            for (int g = 0; g < G; ++g)
                if ((pmask >> g) & 1u) a.trace[out_index(sw + 1, row0 + srow, g)] = scand;
    }
    if (srow < nrows)
        for (int g = 0; g < G; ++g)
            if ((pmask >> g) & 1u) a.picks[((row0 + srow) * a.nblk + blk) * G + g] = scand;
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
