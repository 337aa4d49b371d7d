// choice_search.hip -- local-Hessian choice search of one 256-column block on
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
// Layout: a 256-thread workgroup runs 16 rows in lockstep; thread t owns
// column t of r for all 16 rows (registers), so the rank-L update
// r += H[:, g] (e_new - e_cur) reads L rows of the symmetric H, coalesced, once
// per workgroup and step.  The diagonal blocks H_gg, the rows' current errors,
// e_c^T H_gg e_c and the per-step vectors live in LDS.  The 32 steps of a row
// are serial, so every global read on the step path is issued one step ahead
// (the next group's H rows and candidate vectors) and arrives while the
// current step computes.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace iqk {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;        // rows per workgroup
constexpr int kMaxC = 16;

struct SearchArgs {
    const float* H;          // [nblk][256][256]
    const float* cand;       // [rows][nblk][G][C][L]
    int32_t* picks;          // [rows][nblk][G]
    int32_t* trace;          // NULL or [sweeps+1][rows][nblk][G]
    int64_t rows;
    int64_t nblk;
    int C, sweeps;
};

template <int L>
__global__ __launch_bounds__(kThreads) void choice_search_kernel(SearchArgs a)
{
    constexpr int G = 256 / L;
    __shared__ float hdiag[G * L * L];          // H_gg blocks: [g][i][j]
    __shared__ float ecur[kRows][256];
    __shared__ float qself[kRows][G * kMaxC];   // e_gc^T H_gg e_gc, [g*C + c]
    __shared__ float cst[kRows][kMaxC][L];      // candidate vectors of the current group
    __shared__ float rg[kRows][L];              // r restricted to group g
    __shared__ float rest[kRows][L];
    __shared__ float dlt[kRows][L];             // e_new - e_cur of group g
    __shared__ float score[kRows][kMaxC];
    __shared__ int pick[kRows][G];
    __shared__ int changed[kRows];

    const int t = threadIdx.x;
    const int C = a.C;
    const int64_t row0 = (int64_t)blockIdx.x * kRows;
    const int nrows = (int)((a.rows - row0) < kRows ? (a.rows - row0) : kRows);
    // This workgroup's 256-column block: its H and its slice of every row.
    const int64_t blk = blockIdx.y;
    const float* __restrict__ Hb = a.H + blk * 65536;
    const int64_t cstride = a.nblk * G * C * L;   // floats per row of cand
    const float* __restrict__ cb = a.cand + blk * (int64_t)G * C * L;
    auto out_index = [&](int64_t sweep_slot, int64_t row, int g) -> int64_t {
        return ((sweep_slot * a.rows + row) * a.nblk + blk) * G + g;
    };

    for (int i = t; i < G * L * L; i += kThreads) {
        const int g = i / (L * L), rem = i % (L * L), ii = rem / L, jj = rem % L;
        hdiag[i] = Hb[(g * L + ii) * 256 + g * L + jj];
    }
    __syncthreads();

    // e_gc^T H_gg e_gc for every (row, group, candidate).
    for (int it = t; it < kRows * G * C; it += kThreads) {
        const int rr = it / (G * C), gc = it % (G * C), g = gc / C;
        float q = 0.0f;
        if (rr < nrows) {
            const float* ep = cb + (row0 + rr) * cstride + (int64_t)gc * L;
            float e[L];
#pragma unroll
            for (int j = 0; j < L; ++j) e[j] = ep[j];
            const float* hb = hdiag + g * L * L;
#pragma unroll 4
            for (int i = 0; i < L; ++i) {
                float y = 0.0f;
#pragma unroll
                for (int j = 0; j < L; ++j) y = __builtin_fmaf(hb[i * L + j], e[j], y);
                q = __builtin_fmaf(e[i], y, q);
            }
        }
        qself[rr][gc] = q;
    }
    __syncthreads();

    // Step 2: each group's best candidate under its own block (lowest index on ties).
    for (int it = t; it < kRows * G; it += kThreads) {
        const int rr = it / G, g = it % G;
        int best = 0;
        for (int c = 1; c < C; ++c)
            if (qself[rr][g * C + c] < qself[rr][g * C + best]) best = c;
        pick[rr][g] = best;
        if (rr < nrows) {
            const float* ep = cb + (row0 + rr) * cstride + ((int64_t)g * C + best) * L;
#pragma unroll
            for (int i = 0; i < L; ++i) ecur[rr][g * L + i] = ep[i];
        } else {
#pragma unroll
            for (int i = 0; i < L; ++i) ecur[rr][g * L + i] = 0.0f;
        }
    }
    __syncthreads();
    if (a.trace)
        for (int it = t; it < nrows * G; it += kThreads)
            a.trace[out_index(0, row0 + it / G, it % G)] = pick[it / G][it % G];

    // r = H e (thread t owns column t; H is symmetric, so H[u][t] is read),
    // 16 rows of H in flight at a time.
    float r[kRows];
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) r[rr] = 0.0f;
    for (int u0 = 0; u0 < 256; u0 += 16) {
        float h[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) h[i] = Hb[(u0 + i) * 256 + t];
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int rr = 0; rr < kRows; ++rr) r[rr] = __builtin_fmaf(h[i], ecur[rr][u0 + i], r[rr]);
    }

    // Score threads: (row, candidate) = (t / C, t % C).  Their candidate vector
    // of the current group and the H rows of the current group are loaded one
    // step ahead.
    const bool scorer = t < kRows * C;
    const int srow = scorer ? t / C : 0;
    const int scand = scorer ? t % C : 0;
    const bool srow_ok = scorer && srow < nrows;
    float cv[L];
    float hrow[L];
    auto load_step = [&](int g) {
        if (srow_ok) {
            const float* ep = cb + (row0 + srow) * cstride + ((int64_t)g * C + scand) * L;
#pragma unroll
            for (int i = 0; i < L; ++i) cv[i] = ep[i];
        } else {
#pragma unroll
            for (int i = 0; i < L; ++i) cv[i] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < L; ++i) hrow[i] = Hb[(g * L + i) * 256 + t];
    };
    load_step(0);

    for (int sw = 0; sw < a.sweeps; ++sw) {
        for (int g = 0; g < G; ++g) {
            // A: r of group g to LDS.
            if (t >= g * L && t < g * L + L) {
#pragma unroll
                for (int rr = 0; rr < kRows; ++rr) rg[rr][t - g * L] = r[rr];
            }
            __syncthreads();
            // B: rest = r_g - H_gg e_cur,g
            for (int it = t; it < kRows * L; it += kThreads) {
                const int rr = it / L, i = it % L;
                const float* hb = hdiag + g * L * L + i * L;
                float y = 0.0f;
#pragma unroll
                for (int j = 0; j < L; ++j) y = __builtin_fmaf(hb[j], ecur[rr][g * L + j], y);
                rest[rr][i] = rg[rr][i] - y;
            }
            __syncthreads();
            // C: score_c = e_c^T H_gg e_c + 2 e_c . rest; the candidate vector
            // goes to LDS for the decision.
            if (scorer) {
                float dot = 0.0f;
#pragma unroll
                for (int i = 0; i < L; ++i) {
                    dot = __builtin_fmaf(cv[i], rest[srow][i], dot);
                    cst[srow][scand][i] = cv[i];
                }
                score[srow][scand] = __builtin_fmaf(2.0f, dot, qself[srow][g * C + scand]);
            }
            __syncthreads();
            // D: the lowest-index minimum, taken only on a strict improvement.
            if (t < kRows) {
                const int rr = t;
                int best = 0;
                for (int c = 1; c < C; ++c)
                    if (score[rr][c] < score[rr][best]) best = c;
                const int cur = pick[rr][g];
                const bool move = rr < nrows && score[rr][best] < score[rr][cur];
                changed[rr] = move;
                if (move) {
#pragma unroll
                    for (int i = 0; i < L; ++i) {
                        const float en = cst[rr][best][i];
                        dlt[rr][i] = en - ecur[rr][g * L + i];
                        ecur[rr][g * L + i] = en;
                    }
                    pick[rr][g] = best;
                }
            }
            __syncthreads();
            // E: r += H[:, g-block] * delta for the rows that moved, then the
            // next step's H rows and candidate vectors are requested.
#pragma unroll
            for (int rr = 0; rr < kRows; ++rr) {
                if (changed[rr]) {
                    float acc = r[rr];
#pragma unroll
                    for (int i = 0; i < L; ++i) acc = __builtin_fmaf(hrow[i], dlt[rr][i], acc);
                    r[rr] = acc;
                }
            }
            load_step(g + 1 < G ? g + 1 : 0);
        }
        __syncthreads();
        if (a.trace)
            for (int it = t; it < nrows * G; it += kThreads)
                a.trace[out_index(sw + 1, row0 + it / G, it % G)] = pick[it / G][it % G];
    }
    __syncthreads();
    for (int it = t; it < nrows * G; it += kThreads)
        a.picks[((row0 + it / G) * a.nblk + blk) * G + it % G] = pick[it / G][it % G];
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
