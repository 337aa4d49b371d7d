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
// (grid.y = the block), with two kinds of waves.  The products with H run on
// the matrix cores (v_mfma_f32_16x16x4_f32, fp32 operands): first
// e_c^T H_gg e_c for every candidate (all eight waves), then, for each step of
// the sweeps, the rest of the next group gn, r_gn - H_gn,gn e_gn = sum over
// the other groups h of H_gn,h e_h, formed afresh from the current errors (no
// running r = H e is kept).  Waves 0-3 compute those products: while group g
// is being decided, each sums its quarter of K, leaving out gn and g; after
// the decision each adds its quarter of H_gn,g e_g with g's new errors and
// leaves its partial rest in LDS.  Waves 4-7 decide, one lane per (row,
// candidate): the rest of g is the sum of the four partials, each lane scores
// its candidate from its own error vector and that rest, and one DPP
// reduction across the row's 16 lanes gives the lowest index of least score,
// the current pick winning the ties it is in (each lane keeps a bit mask of
// the groups whose pick is its candidate).  The two kinds of waves share the
// SIMDs, so the products of the next group run beside the decision of the
// current one; two barriers per step.  The next step's H operands and
// candidate vectors are requested a step ahead.

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
    constexpr int KH = L / 16;                  // 16-column tiles per group
    // LDS rows are padded (and stay 16-byte aligned) so that the lanes of a
    // wave reading rows, blocks or columns together fall in different banks.
    constexpr int kHR = L + 4;                  // H_gg row stride, rest row stride
    constexpr int kHB = L * kHR + 4;            // H_gg block stride
    constexpr int kQS = G * kMaxC + 16;         // qself row stride
    constexpr int kPR = L + 4;                  // partial rest row stride
    __shared__ __align__(16) float hdiag[G * kHB];        // H_gg blocks [g][i][j]
    __shared__ __align__(16) float ecurT[256 * kRows];    // current errors, [column][row]
    __shared__ __align__(16) float part[kProdWaves * kRows * kPR];  // [wave][row][i]
    __shared__ __align__(16) float enew[kRows * kPR];     // the decided group's errors, [row][i]
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
        for (int i = t; i < G * L * L; i += kThreads) {
            const int g = i / (L * L), rem = i % (L * L), ii = rem / L, jj = rem % L;
            hdiag[g * kHB + ii * kHR + jj] = Hb[(g * L + ii) * 256 + g * L + jj];
        }
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
    // ties), and the current errors as columns.
    for (int it = t; it < kRows * G; it += kThreads) {
        const int rr = it / G, g = it % G;
        int best = 0;
        for (int c = 1; c < C; ++c)
            if (qself[rr * kQS + g * C + c] < qself[rr * kQS + g * C + best]) best = c;
        pick0[rr * G + g] = best;
        const float4* ep = rr < nrows ? reinterpret_cast<const float4*>(cand_ptr(rr, g, best)) : nullptr;
#pragma unroll
        for (int i4 = 0; i4 < L / 4; ++i4) {
            const float4 v = ep ? ep[i4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            ecurT[(g * L + 4 * i4) * kRows + rr] = v.x;
            ecurT[(g * L + 4 * i4 + 1) * kRows + rr] = v.y;
            ecurT[(g * L + 4 * i4 + 2) * kRows + rr] = v.z;
            ecurT[(g * L + 4 * i4 + 3) * kRows + rr] = v.w;
        }
    }
    __syncthreads();
    if (a.trace)
        for (int it = t; it < nrows * G; it += kThreads)
            a.trace[out_index(0, row0 + it / G, it % G)] = pick0[it];

    const bool prod = wave < kProdWaves;        // wave-uniform

    if (prod) {
        // ---------------- product waves ----------------
        // The wave's partial rest of group gn for the 16 rows: K range
        // 64w .. 64w + 63 in steps of 4 (k = 64w + 4s + lq), the columns of gn
        // and gx (gx < 0: none) left out.  Output tile ih holds the columns
        // gn*L + 16ih .. + 15 (lane: columns 4lq..4lq+3 of the tile, row lc).
        // Then its quarter of the late product H_gn,gx e_gx (k = gx*L +
        // (L/4)w + 4s + lq, s < KH) with gx's new errors, and the tiles go to
        // part[w] as [row][column].  The H operands (H symmetric: H[k][column])
        // are requested a step ahead.
        constexpr int kPS = 16;                 // K steps per wave
        float hP[KH][kPS], hPn[KH][kPS];        // H[64w + 4s + lq][gn*L + 16ih + lc]
        float hX[KH][KH], hXn[KH][KH];          // H[gx*L + (L/4)w + 4s + lq][gn*L + 16ih + lc]
        auto load_hP = [&](int gn, float (&h)[KH][kPS]) {
#pragma unroll
            for (int ih = 0; ih < KH; ++ih)
#pragma unroll
                for (int s = 0; s < kPS; ++s)
                    h[ih][s] = Hb[(64 * wave + 4 * s + lq) * 256 + gn * L + 16 * ih + lc];
        };
        auto load_hX = [&](int gn, int gx, float (&h)[KH][KH]) {
#pragma unroll
            for (int ih = 0; ih < KH; ++ih)
#pragma unroll
                for (int s = 0; s < KH; ++s)
                    h[ih][s] = Hb[(gx * L + (L / 4) * wave + 4 * s + lq) * 256 + gn * L + 16 * ih + lc];
        };
        auto partial = [&](int gn, int gx, v4f (&p)[KH]) {
            float bv[kPS];
#pragma unroll
            for (int s = 0; s < kPS; ++s) bv[s] = ecurT[(64 * wave + 4 * s + lq) * kRows + lc];
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
        auto store_part = [&](const v4f (&p)[KH]) {
#pragma unroll
            for (int ih = 0; ih < KH; ++ih)
                *reinterpret_cast<v4f*>(&part[(wave * kRows + lc) * kPR + 16 * ih + 4 * lq]) = p[ih];
        };

        // The rest of group 0 (no group being decided).
        v4f pp[KH];
        load_hP(0, hP);
        partial(0, -1, pp);
        store_part(pp);
        load_hP(1 % G, hP);
        load_hX(1 % G, 0, hX);
        __syncthreads();                        // part holds the rest of group 0
        // One step: the products of gn beside the decision of g, with the
        // operands requested the step before (cur); the next step's go into
        // nxt once cur's are in use.  Steps alternate between the two register
        // sets, so a load is first used about a step after it was issued.
        auto pstep = [&](int g, float (&hPc)[KH][kPS], float (&hXc)[KH][KH],
                         float (&hPx)[KH][kPS], float (&hXx)[KH][KH]) {
            const int gn = g + 1 < G ? g + 1 : 0;
            const int gnn = gn + 1 < G ? gn + 1 : 0;
            float bv[kPS];
#pragma unroll
            for (int s = 0; s < kPS; ++s) bv[s] = ecurT[(64 * wave + 4 * s + lq) * kRows + lc];
#pragma unroll
            for (int ih = 0; ih < KH; ++ih) pp[ih] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < kPS; ++s) {
                const int kg = (64 * wave + 4 * s) / L;             // wave-uniform
                if (kg != gn && kg != g) {
#pragma unroll
                    for (int ih = 0; ih < KH; ++ih) pp[ih] = mfma4(hPc[ih][s], bv[s], pp[ih]);
                }
            }
            // The next step's H operands, requested once this step's are in
            // use (a wait for these must not wait for those).
            load_hP(gnn, hPx);
            load_hX(gnn, gn, hXx);
            __syncthreads();                    // A: g decided, its errors in enew
#pragma unroll
            for (int s = 0; s < KH; ++s) {
                const float b = enew[lc * kPR + (L / 4) * wave + 4 * s + lq];
#pragma unroll
                for (int ih = 0; ih < KH; ++ih) pp[ih] = mfma4(hXc[ih][s], b, pp[ih]);
            }
            store_part(pp);
            __syncthreads();                    // B: part holds the rest of gn
        };
        for (int sw = 0; sw < a.sweeps; ++sw) {
#pragma unroll 1
            for (int g = 0; g < G; g += 2) {    // G is even
                pstep(g, hP, hX, hPn, hXn);
                pstep(g + 1, hPn, hXn, hP, hX);
            }
        }
    } else {
        // ---------------- decision waves ----------------
        // Lane (srow, scand); pmask bit g = group g's pick is scand.
        const int dt = t - 64 * kProdWaves;
        const int srow = dt >> 4;
        const int scand = dt & 15;
        const bool scorer = scand < C && srow < nrows;
        uint32_t pmask = 0u;
        for (int g = 0; g < G; ++g) pmask |= (uint32_t)(pick0[srow * G + g] == scand) << g;
        float cv[L], cvn[L];
        auto load_cv = [&](int g, float (&v)[L]) {
            if (scorer) {
                const float4* ep = reinterpret_cast<const float4*>(cand_ptr(srow, g, scand));
#pragma unroll
                for (int i4 = 0; i4 < L / 4; ++i4) {
                    const float4 u = ep[i4];
                    v[4 * i4] = u.x; v[4 * i4 + 1] = u.y; v[4 * i4 + 2] = u.z; v[4 * i4 + 3] = u.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < L; ++i) v[i] = 0.0f;
            }
        };
        load_cv(0, cv);
        __syncthreads();                        // part holds the rest of group 0
        // One step: group g decided with its candidate vector requested the
        // step before (cur); the next group's goes into nxt.
        auto dstep = [&](int g, float (&cur)[L], float (&nxt)[L]) {
            const int gn = g + 1 < G ? g + 1 : 0;
            // The rest of g: the four partials summed in a fixed order, one
            // column (two for L = 32) per lane, then the whole row read back by
            // the row's 16 lanes (one wave: in order in LDS).
#pragma unroll
            for (int h = 0; h < KH; ++h) {
                const int i = scand + 16 * h;
                float v = part[(0 * kRows + srow) * kPR + i];
#pragma unroll
                for (int w = 1; w < kProdWaves; ++w) v += part[(w * kRows + srow) * kPR + i];
                rest[srow * kHR + i] = v;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float sc = __builtin_inff();
            if (scorer) {
                float d4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int i4 = 0; i4 < L / 4; ++i4) {
                    const float4 r4 = *reinterpret_cast<const float4*>(&rest[srow * kHR + 4 * i4]);
                    d4[0] = __builtin_fmaf(cur[4 * i4], r4.x, d4[0]);
                    d4[1] = __builtin_fmaf(cur[4 * i4 + 1], r4.y, d4[1]);
                    d4[2] = __builtin_fmaf(cur[4 * i4 + 2], r4.z, d4[2]);
                    d4[3] = __builtin_fmaf(cur[4 * i4 + 3], r4.w, d4[3]);
                }
                const float dot = (d4[0] + d4[1]) + (d4[2] + d4[3]);
                sc = __builtin_fmaf(2.0f, dot, qself[srow * kQS + g * C + scand]);
            }
            // The least score of the row (DPP), then the row's lanes that
            // hold it (a ballot, 16 bits per row): the group keeps its pick if
            // the pick holds it (only a strictly lower score moves it), else
            // moves to the lowest candidate that does.
            const bool mine = (pmask >> g) & 1u;
            const float m = row_min(sc);
            const int rsh = 16 * (lane >> 4);
            const uint32_t req = (uint32_t)(__ballot(sc == m) >> rsh) & 0xffffu;
            const uint32_t rcur = (uint32_t)(__ballot(mine) >> rsh) & 0xffffu;
            const bool move = req != 0u && (req & rcur) == 0u;
            const int bc = __builtin_ctz(req | 0x10000u);
            // The row's new errors of group g (the new pick's, or the current
            // pick's when it stays).
            if (move ? scand == bc : mine) {
#pragma unroll
                for (int i4 = 0; i4 < L / 4; ++i4)
                    *reinterpret_cast<float4*>(&enew[srow * kPR + 4 * i4]) =
                        make_float4(cur[4 * i4], cur[4 * i4 + 1], cur[4 * i4 + 2], cur[4 * i4 + 3]);
            }
            if (move) pmask = (pmask & ~(1u << g)) | ((uint32_t)(scand == bc) << g);
            // The next group's candidate vector, requested once this one's is
            // used (a wait for this one must not wait for that).
            load_cv(gn, nxt);
            __syncthreads();                    // A: g decided, its errors in enew
            // g's errors into the error columns (the product waves read them
            // from the next step on)
#pragma unroll
            for (int h = 0; h < KH; ++h) {
                const int i = scand + 16 * h;
                ecurT[(g * L + i) * kRows + srow] = enew[srow * kPR + i];
            }
            __syncthreads();                    // B: part holds the rest of gn
        };
        for (int sw = 0; sw < a.sweeps; ++sw) {
#pragma unroll 1
            for (int g = 0; g < G; g += 2) {    // G is even
                dstep(g, cv, cvn);
                dstep(g + 1, cvn, cv);
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
