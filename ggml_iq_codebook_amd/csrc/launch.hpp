// launch.hpp -- host-side launchers of the HIP kernels, called by the C-ABI
// entry points in api.hip after argument validation.  Each returns the
// hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iqk {

// Geometry of the weight/payload being processed.  Blocks are numbered
// row-major over [batch][rows][cols/256].
struct BlockGeom {
    int64_t nblocks;          // batch * rows * (cols / 256)
    int64_t blocks_per_row;   // cols / 256
    int64_t blocks_per_batch; // rows * (cols / 256)
    int64_t cols;
    int cus;                  // compute units of the device (sizes persistent grids)
};

// What an encode launch writes: the payload; the payload under every one of
// the 16 choices ([16][nblocks][block_bytes]); the decoded values (and the
// payload when `out` is given); or the top-C candidates.
enum EncodeMode { kModePayload = 0, kModeEvery = 1, kModeFake = 2, kModeCandidates = 3 };

// IQ1_S and IQ1_M (fmt = IQ_FMT_IQ1_S or IQ_FMT_IQ1_M) share one kernel.
// wdtype: the weight's iq_dtype_t (w points at values of that type).
hipError_t launch_iq1_encode(int fmt, int wdtype, const void* w, const float* imp,
                             const float* grid, int grid_size, const uint16_t* scales,
                             const int32_t* choices, uint8_t* out, float* xhat, int mode,
                             int32_t* status, const BlockGeom& g, hipStream_t stream);

hipError_t launch_iq2xs_encode(int wdtype, const void* w, const float* imp, const float* grid,
                               int grid_size, const uint16_t* scales, const int32_t* choices,
                               uint8_t* out, float* xhat, int mode, int32_t* status,
                               const BlockGeom& g, hipStream_t stream);

hipError_t launch_iq1_candidates(int fmt, int wdtype, const void* w, const float* imp,
                                 const float* grid, int grid_size, int top_c, float* cand_err,
                                 int32_t* cand_choice, uint16_t* cand_codes, int32_t* status,
                                 const BlockGeom& g, hipStream_t stream);

hipError_t launch_iq2xs_candidates(int wdtype, const void* w, const float* imp, const float* grid,
                                   int grid_size, int top_c, float* cand_err, int32_t* cand_choice,
                                   uint16_t* cand_codes, int32_t* status, const BlockGeom& g,
                                   hipStream_t stream);

hipError_t launch_dequant(int fmt, const uint8_t* packed, const float* grid, int grid_size,
                          float* out, int32_t* status, const BlockGeom& g, hipStream_t stream);

hipError_t launch_choice_search(const float* H, const float* cand, int64_t rows, int64_t nblk,
                                int G, int C, int sweeps, int32_t* picks, int32_t* trace,
                                hipStream_t stream);

}  // namespace iqk
