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
// (grid.y = the block).  r (256 columns x 16 rows) lives in registers in the
// matrix-core accumulator layout: wave w holds columns 64w..64w+63 as four
// 16x16 tiles, lane l holding columns 4(l/16)..4(l/16)+3 of a tile for row
// l%16.  The products with H run on the matrix cores (v_mfma_f32_16x16x4_f32,
// fp32 operands): e_c^T H_gg e_c for every candidate, the initial r = H e, each
// step's rank-L update r += H[:,g] de, and the next group's
// rest = r_g - H_gg e_cur,g (by the wave that owns that group's columns).  The
// decision runs in the scorer layout, lane (row, candidate) = (t/16, t%16):
// each lane scores its candidate from its own error vector and the row's rest;
// DPP reductions across the row's 16 lanes give the lowest index of least
// score and the current pick's score (each lane keeps a bit mask of the groups
// whose pick is its candidate).  Two barriers per step; the next step's H rows
// and candidate vectors are requested a step ahead.
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

template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xf, 0xf, false);
}

constexpr int kRor8 = 0x128, kRor4 = 0x124, kXor2 = 0x4e, kXor1 = 0xb1;

template <int kCtrl>
__device__ __forceinline__ void argmin_step(float& v, int& i)
{
    const float ov = dpp_f<kCtrl>(v);
    const int oi = dpp_i<kCtrl>(i);
    if (ov < v || (ov == v && oi < i)) { v = ov; i = oi; }
}

// Least value over the 16 lanes of a row, lowest index among equal values;
// every lane of the row ends with the result (the four steps reach lanes
// +8, +4, ^2, ^1 away, which together cover the row).
__device__ __forceinline__ void row_argmin(float& v, int& i)
{
    argmin_step<kRor8>(v, i);
    argmin_step<kRor4>(v, i);
    argmin_step<kXor2>(v, i);
    argmin_step<kXor1>(v, i);
}

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
    __shared__ __align__(16) float ecurT[256 * kRows];    // current errors, [column][row]
    __shared__ __align__(16) float dltT[L * kRows];       // e_new - e_cur of the group, [i][row]
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

    // r = H e on the matrix cores: wave w's tiles j = 0..3 (columns
    // 64w + 16j ..), K over all 256 columns in 64 steps of 4; the H operand
    // (H symmetric: H[k][column]) streamed from L2 eight steps at a time, one
    // batch ahead.
    v4f r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    {
        constexpr int kB = 16;
        float ha[4][kB], hn[4][kB];
        auto load_batch = [&](int s0, float (&h)[4][kB]) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int s = 0; s < kB; ++s)
                    h[j][s] = Hb[(4 * (s0 + s) + lq) * 256 + 64 * wave + 16 * j + lc];
        };
        load_batch(0, ha);
        for (int s0 = 0; s0 < 64; s0 += kB) {
            load_batch(s0 + kB < 64 ? s0 + kB : s0, hn);
#pragma unroll
            for (int s = 0; s < kB; ++s) {
                const float bv = ecurT[(4 * (s0 + s) + lq) * kRows + lc];
#pragma unroll
                for (int j = 0; j < 4; ++j) r[j] = mfma4(ha[j][s], bv, r[j]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int s = 0; s < kB; ++s) ha[j][s] = hn[j][s];
        }
    }

    // rest of group gn = r_gn - H_gn,gn e_cur,gn on the matrix cores (the
    // accumulator starts from the r tile), by the wave that owns the group's
    // columns, written to LDS.
    auto make_rest = [&](int gn) {
        if (wave != ((gn * L) >> 6)) return;                    // wave-uniform
#pragma unroll
        for (int ih = 0; ih < KH; ++ih) {
            const int jt = ((gn * L) & 63) / 16 + ih;
            v4f d = r[0];
#pragma unroll
            for (int j = 1; j < 4; ++j)
                if (jt == j) d = r[j];
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int k = 4 * s + lq;
                const float A = -hdiag[gn * kHB + (16 * ih + lc) * kHR + k];
                d = mfma4(A, ecurT[(gn * L + k) * kRows + lc], d);
            }
            *reinterpret_cast<float4*>(&rest[lc * kHR + 16 * ih + 4 * lq]) =
                make_float4(d[0], d[1], d[2], d[3]);
        }
    };
    make_rest(0);

    // The step operands, one group ahead: the scorer's candidate vector and
    // the group's H rows for the update.
    float cv[L], cvn[L];
    float hA[4][KS], hAn[4][KS];
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
    auto load_hA = [&](int g, float (&h)[4][KS]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int s = 0; s < KS; ++s)
                h[j][s] = Hb[(g * L + 4 * s + lq) * 256 + 64 * wave + 16 * j + lc];
    };
    load_cv(0, cv);
    load_hA(0, hA);
    __syncthreads();

    for (int sw = 0; sw < a.sweeps; ++sw) {
        for (int g = 0; g < G; ++g) {
            const int gn = g + 1 < G ? g + 1 : 0;
            // Scores, the decision and the error update of group g.
            load_cv(gn, cvn);
            float sc = __builtin_inff();
            if (scorer) {
                float dot = 0.0f;
#pragma unroll
                for (int i = 0; i < L; ++i) dot = __builtin_fmaf(cv[i], rest[srow * kHR + i], dot);
                sc = __builtin_fmaf(2.0f, dot, qself[srow * kQS + g * C + scand]);
            }
            const bool mine = (pmask >> g) & 1u;
            const float scur = row_min(mine ? sc : __builtin_inff());
            float bs = sc;
            int bc = scand;
            row_argmin(bs, bc);
            const bool move = bs < scur;          // a strict improvement only
            if (move && scand == bc) {
#pragma unroll
                for (int i = 0; i < L; ++i) {
                    const int at = (g * L + i) * kRows + srow;
                    dltT[i * kRows + srow] = cv[i] - ecurT[at];
                    ecurT[at] = cv[i];
                }
            } else if (!move && scand == 0) {
#pragma unroll
                for (int i = 0; i < L; ++i) dltT[i * kRows + srow] = 0.0f;
            }
            if (move) pmask = (pmask & ~(1u << g)) | ((uint32_t)(scand == bc) << g);
#pragma unroll
            for (int i = 0; i < L; ++i) cv[i] = cvn[i];
            __syncthreads();

            // r += H[:, g] de on the matrix cores; the owner of the next group
            // then forms its rest.
            load_hA(gn, hAn);
            float bdl[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) bdl[s] = dltT[(4 * s + lq) * kRows + lc];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int s = 0; s < KS; ++s) r[j] = mfma4(hA[j][s], bdl[s], r[j]);
            make_rest(gn);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int s = 0; s < KS; ++s) hA[j][s] = hAn[j][s];
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
