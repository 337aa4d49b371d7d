// api.hip -- the extern "C" entry points of libiqcodec.so declared in
// include/iq_codec.h: argument validation, the gfx950 device check, and the
// stream-ordered launches.  No device memory is allocated here: the one word
// the library owns on a device (the status of calls made with status = NULL)
// is a file-scope device variable.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "iq_codec.h"
#include "launch.hpp"

namespace {

constexpr int kMaxDevices = 64;
// Per device: 0 = not checked, 1 = gfx950, 2 = other; and its compute units.
std::atomic<int> g_device_kind[kMaxDevices];
std::atomic<int> g_device_cus[kMaxDevices];

// Also records the device's compute units in g (when given): persistent
// launches size their grid by it.
iq_status_t check_device(iqk::BlockGeom* g = nullptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return IQ_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return IQ_ERR_DEVICE;
    int kind = g_device_kind[dev].load(std::memory_order_acquire);
    if (kind == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return IQ_ERR_HIP;
        kind = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_device_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1,
                                std::memory_order_relaxed);
        g_device_kind[dev].store(kind, std::memory_order_release);
    }
    if (g) g->cus = g_device_cus[dev].load(std::memory_order_relaxed);
    return kind == 1 ? IQ_OK : IQ_ERR_DEVICE;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Geometry of [batch][rows][cols] with every size positive and cols % 256 == 0.
iq_status_t geometry(int64_t batch, int64_t rows, int64_t cols, iqk::BlockGeom* g)
{
    if (batch <= 0 || rows <= 0 || cols <= 0 || (cols % 256) != 0) return IQ_ERR_SHAPE;
    const int64_t bpr = cols / 256;
    // Keep every element index below 2^62 and the launch grid below 2^31 workgroups.
    if (rows > (INT64_C(1) << 40) / bpr || batch > (INT64_C(1) << 40) / (rows * bpr))
        return IQ_ERR_SHAPE;
    g->blocks_per_row = bpr;
    g->blocks_per_batch = rows * bpr;
    g->nblocks = batch * rows * bpr;
    g->cols = cols;
    g->cus = 1;
    if (g->nblocks > (INT64_C(1) << 34)) return IQ_ERR_SHAPE;
    return IQ_OK;
}

iq_status_t from_hip(hipError_t e) { return e == hipSuccess ? IQ_OK : IQ_ERR_HIP; }

// ---------------------------------------------------------------------------
// Calls made with status = NULL synchronize their stream and return the first
// data error.  The kernels still need a device word to report into: each GPU
// holds one in this file-scope variable (the library allocates nothing).  In
// host code its name only stands in for the symbol; the device address is
// taken once per device with hipGetSymbolAddress, with that device current,
// and kept in g_sync_word.  A per-device lock, held from clearing the word to
// reading it back after the stream has drained, serializes such calls, so two
// host threads never share the word at once.
// ---------------------------------------------------------------------------

__device__ __align__(256) int32_t sync_status_word[1];

__global__ void clear_sync_word_kernel(int32_t* word) { word[0] = 0; }

std::mutex g_sync_mutex[kMaxDevices];
int32_t* g_sync_word[kMaxDevices];    // guarded by g_sync_mutex[dev]

// Runs launch(status) when the caller gave a status word.  Otherwise clears
// the device's own word, runs launch(word), waits for the stream and returns
// the word: IQ_OK, or the first data error code the kernels reported.
template <class Launch>
iq_status_t run_with_status(int32_t* status, hipStream_t stream, Launch&& launch)
{
    if (status) return from_hip(launch(status));
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return IQ_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return IQ_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_sync_mutex[dev]);
    if (!g_sync_word[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(sync_status_word)) != hipSuccess || !p)
            return IQ_ERR_HIP;
        g_sync_word[dev] = static_cast<int32_t*>(p);
    }
    int32_t* word = g_sync_word[dev];
    hipLaunchKernelGGL(clear_sync_word_kernel, dim3(1), dim3(1), 0, stream, word);
    if (hipGetLastError() != hipSuccess) return IQ_ERR_HIP;
    if (launch(word) != hipSuccess) return IQ_ERR_HIP;
    int32_t host = 0;
    if (hipMemcpyAsync(&host, word, sizeof(host), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return IQ_ERR_HIP;
    return static_cast<iq_status_t>(host);
}

bool known_format(iq_format_t fmt)
{
    return fmt == IQ_FMT_IQ1_S || fmt == IQ_FMT_IQ2_XS || fmt == IQ_FMT_IQ1_M;
}

int grid_max(iq_format_t fmt) { return fmt == IQ_FMT_IQ2_XS ? 512 : 2048; }

int num_choices(iq_format_t fmt) { return fmt == IQ_FMT_IQ1_M ? 8 : 16; }

// Bytes per weight value, 0 for an unknown type.
size_t dtype_bytes(iq_dtype_t t)
{
    switch (t) {
    case IQ_DTYPE_F32: return 4;
    case IQ_DTYPE_BF16: return 2;
    case IQ_DTYPE_F16: return 2;
    case IQ_DTYPE_F64: return 8;
    }
    return 0;
}

hipError_t launch_encode(iq_format_t fmt, iq_dtype_t wdtype, const void* w,
                         const float* importance, const float* grid, int32_t grid_size,
                         const uint16_t* scales, const int32_t* choices, uint8_t* out,
                         float* xhat, int mode, int32_t* status, const iqk::BlockGeom& g,
                         hipStream_t stream)
{
    return fmt == IQ_FMT_IQ2_XS
        ? iqk::launch_iq2xs_encode((int)wdtype, w, importance, grid, grid_size, scales, choices,
                                   out, xhat, mode, status, g, stream)
        : iqk::launch_iq1_encode((int)fmt, (int)wdtype, w, importance, grid, grid_size, scales,
                                 choices, out, xhat, mode, status, g, stream);
}

}  // namespace

extern "C" {

iq_status_t iq_format_info(iq_format_t fmt, iq_format_info_t* out)
{
    if (!out) return IQ_ERR_NULL;
    if (fmt == IQ_FMT_IQ1_S) {
        *out = iq_format_info_t{256, 50, 8, 11, 2048, 8, 16};
    } else if (fmt == IQ_FMT_IQ2_XS) {
        *out = iq_format_info_t{256, 74, 8, 9, 512, 16, 16};
    } else if (fmt == IQ_FMT_IQ1_M) {
        *out = iq_format_info_t{256, 56, 8, 11, 2048, 16, 8};
    } else {
        return IQ_ERR_FORMAT;
    }
    return IQ_OK;
}

const char* iq_status_str(iq_status_t st)
{
    switch (st) {
    case IQ_OK: return "ok";
    case IQ_ERR_NULL: return "a required pointer is NULL";
    case IQ_ERR_FORMAT: return "unknown or unsupported format";
    case IQ_ERR_SHAPE: return "bad shape (empty, or cols not a multiple of 256, or too large)";
    case IQ_ERR_GRID: return "bad grid (size out of range, or values the format does not allow)";
    case IQ_ERR_NONFINITE: return "non-finite weight";
    case IQ_ERR_IMPORTANCE: return "negative or non-finite importance";
    case IQ_ERR_SCALE_RANGE: return "super-block scale out of fp16 range";
    case IQ_ERR_ARG: return "argument out of range";
    case IQ_ERR_CODE: return "payload grid index beyond the grid";
    case IQ_ERR_HIP: return "HIP runtime error";
    case IQ_ERR_DEVICE: return "current device is not gfx950";
    }
    return "unknown status";
}

iq_status_t iq_encode(iq_format_t fmt, iq_dtype_t wdtype, const void* w, int64_t batch,
                      int64_t rows, int64_t cols, const float* importance, const float* grid,
                      int32_t grid_size, const uint16_t* scales, const int32_t* choices,
                      uint8_t* out, int32_t* status, hipStream_t stream)
{
    if (!known_format(fmt)) return IQ_ERR_FORMAT;
    iqk::BlockGeom g;
    iq_status_t st = geometry(batch, rows, cols, &g);
    if (st) return st;
    if (!w || !grid || !out) return IQ_ERR_NULL;
    if (grid_size < 1 || grid_size > grid_max(fmt)) return IQ_ERR_GRID;
    if (dtype_bytes(wdtype) == 0) return IQ_ERR_ARG;
    if (!aligned(w, 16) || !aligned(grid, 16) || (importance && !aligned(importance, 16)) ||
        !aligned(out, 2) || (scales && !aligned(scales, 2)) || (choices && !aligned(choices, 4)) ||
        (status && !aligned(status, 4)))
        return IQ_ERR_ARG;
    st = check_device(&g);
    if (st) return st;
    return run_with_status(status, stream, [&](int32_t* s) {
        return launch_encode(fmt, wdtype, w, importance, grid, grid_size, scales, choices, out,
                             nullptr, iqk::kModePayload, s, g, stream);
    });
}

iq_status_t iq_encode_every_choice(iq_format_t fmt, iq_dtype_t wdtype, const void* w,
                                   int64_t batch, int64_t rows, int64_t cols,
                                   const float* importance, const float* grid, int32_t grid_size,
                                   const uint16_t* scales, uint8_t* out, int32_t* status,
                                   hipStream_t stream)
{
    if (!known_format(fmt)) return IQ_ERR_FORMAT;
    iqk::BlockGeom g;
    iq_status_t st = geometry(batch, rows, cols, &g);
    if (st) return st;
    if (!w || !grid || !out) return IQ_ERR_NULL;
    if (grid_size < 1 || grid_size > grid_max(fmt)) return IQ_ERR_GRID;
    if (dtype_bytes(wdtype) == 0) return IQ_ERR_ARG;
    if (!aligned(w, 16) || !aligned(grid, 16) || (importance && !aligned(importance, 16)) ||
        !aligned(out, 2) || (scales && !aligned(scales, 2)) || (status && !aligned(status, 4)))
        return IQ_ERR_ARG;
    st = check_device(&g);
    if (st) return st;
    return run_with_status(status, stream, [&](int32_t* s) {
        return launch_encode(fmt, wdtype, w, importance, grid, grid_size, scales, nullptr, out,
                             nullptr, iqk::kModeEvery, s, g, stream);
    });
}

iq_status_t iq_fake_quant(iq_format_t fmt, iq_dtype_t wdtype, const void* w, int64_t batch,
                          int64_t rows, int64_t cols, const float* importance, const float* grid,
                          int32_t grid_size, const uint16_t* scales, const int32_t* choices,
                          float* xhat, uint8_t* out, int32_t* status, hipStream_t stream)
{
    if (!known_format(fmt)) return IQ_ERR_FORMAT;
    iqk::BlockGeom g;
    iq_status_t st = geometry(batch, rows, cols, &g);
    if (st) return st;
    if (!w || !grid || !xhat) return IQ_ERR_NULL;
    if (grid_size < 1 || grid_size > grid_max(fmt)) return IQ_ERR_GRID;
    if (dtype_bytes(wdtype) == 0) return IQ_ERR_ARG;
    if (!aligned(w, 16) || !aligned(grid, 16) || (importance && !aligned(importance, 16)) ||
        !aligned(xhat, 16) || (out && !aligned(out, 2)) || (scales && !aligned(scales, 2)) ||
        (choices && !aligned(choices, 4)) || (status && !aligned(status, 4)))
        return IQ_ERR_ARG;
    // The decoded values may not overlap the weights: a block's values are
    // written while the other half of the block may still be reading them.
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(w), x0 = reinterpret_cast<uintptr_t>(xhat);
    const uintptr_t wbytes = static_cast<uintptr_t>(g.nblocks) * 256u * dtype_bytes(wdtype);
    const uintptr_t xbytes = static_cast<uintptr_t>(g.nblocks) * 256u * sizeof(float);
    if (x0 < w0 + wbytes && w0 < x0 + xbytes) return IQ_ERR_ARG;
    st = check_device(&g);
    if (st) return st;
    return run_with_status(status, stream, [&](int32_t* s) {
        return launch_encode(fmt, wdtype, w, importance, grid, grid_size, scales, choices, out,
                             xhat, iqk::kModeFake, s, g, stream);
    });
}

iq_status_t iq_dequant(iq_format_t fmt, const uint8_t* packed, int64_t batch, int64_t rows,
                       int64_t cols, const float* grid, int32_t grid_size, float* out,
                       int32_t* status, hipStream_t stream)
{
    if (!known_format(fmt)) return IQ_ERR_FORMAT;
    iqk::BlockGeom g;
    iq_status_t st = geometry(batch, rows, cols, &g);
    if (st) return st;
    if (!packed || !grid || !out) return IQ_ERR_NULL;
    if (grid_size < 1 || grid_size > grid_max(fmt)) return IQ_ERR_GRID;
    if (!aligned(grid, 16) || !aligned(out, 16) || (status && !aligned(status, 4)))
        return IQ_ERR_ARG;
    st = check_device(&g);
    if (st) return st;
    return run_with_status(status, stream, [&](int32_t* s) {
        return iqk::launch_dequant((int)fmt, packed, grid, grid_size, out, s, g, stream);
    });
}

iq_status_t iq_encode_candidates(iq_format_t fmt, iq_dtype_t wdtype, const void* w, int64_t rows,
                                 int64_t cols, const float* importance, const float* grid,
                                 int32_t grid_size, int32_t top_c, float* cand_err,
                                 int32_t* cand_choice, uint16_t* cand_codes, int32_t* status,
                                 hipStream_t stream)
{
    if (!known_format(fmt)) return IQ_ERR_FORMAT;
    iqk::BlockGeom g;
    iq_status_t st = geometry(1, rows, cols, &g);
    if (st) return st;
    if (!w || !grid || !cand_err || !cand_choice) return IQ_ERR_NULL;
    if (grid_size < 1 || grid_size > grid_max(fmt)) return IQ_ERR_GRID;
    if (top_c < 1 || top_c > num_choices(fmt)) return IQ_ERR_ARG;
    if (dtype_bytes(wdtype) == 0) return IQ_ERR_ARG;
    if (!aligned(w, 16) || !aligned(grid, 16) || (importance && !aligned(importance, 16)) ||
        !aligned(cand_err, 16) || !aligned(cand_choice, 4) ||
        (cand_codes && !aligned(cand_codes, 2)) || (status && !aligned(status, 4)))
        return IQ_ERR_ARG;
    st = check_device(&g);
    if (st) return st;
    return run_with_status(status, stream, [&](int32_t* s) {
        if (fmt != IQ_FMT_IQ2_XS)
            return iqk::launch_iq1_candidates((int)fmt, (int)wdtype, w, importance, grid, grid_size,
                                              top_c, cand_err, cand_choice, cand_codes, s, g,
                                              stream);
        return iqk::launch_iq2xs_candidates((int)wdtype, w, importance, grid, grid_size, top_c,
                                            cand_err, cand_choice, cand_codes, s, g, stream);
    });
}

iq_status_t iq_choice_search(const float* H, const float* cand_err, int64_t rows, int32_t G,
                             int32_t C, int32_t sweeps, int32_t* picks, int32_t* trace,
                             hipStream_t stream)
{
    return iq_choice_search_blocks(H, cand_err, rows, 1, G, C, sweeps, picks, trace, stream);
}

iq_status_t iq_choice_search_blocks(const float* H, const float* cand_err, int64_t rows,
                                    int64_t nblk, int32_t G, int32_t C, int32_t sweeps,
                                    int32_t* picks, int32_t* trace, hipStream_t stream)
{
    if (rows <= 0 || rows > (INT64_C(1) << 34) || nblk <= 0 || nblk > 65535 ||
        rows * nblk > (INT64_C(1) << 34))
        return IQ_ERR_SHAPE;
    if (!H || !cand_err || !picks) return IQ_ERR_NULL;
    if ((G != 8 && G != 16) || C < 1 || C > 16 || sweeps < 0 || sweeps > 8) return IQ_ERR_ARG;
    if (!aligned(H, 4) || !aligned(cand_err, 16) || !aligned(picks, 4) || (trace && !aligned(trace, 4)))
        return IQ_ERR_ARG;
    iq_status_t st = check_device();
    if (st) return st;
    return from_hip(iqk::launch_choice_search(H, cand_err, rows, nblk, G, C, sweeps, picks, trace,
                                              stream));
}

}  // extern "C"
