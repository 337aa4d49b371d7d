/*
 * iq_codec.h -- C-ABI of libiqcodec.so: the importance-weighted codebook-search
 * encode of the GGML IQ1_S and IQ2_XS weight formats, their decode, the top-C
 * candidate emission and the local-Hessian choice search, as hand-written HIP
 * kernels for AMD Instinct MI355X (gfx950).
 *
 * Sources: the NVIDIA Model-Optimizer pull-request pages
 *   - "Add IQ tests and release notes" (#2450), code review: block layouts,
 *     scale predictor, 16-way choice, tie rule, worked decode example;
 *   - "Weight the IQ1 encoders by the square root of GPTQ's Hessian diagonal"
 *     (#2723): the weighted objective sum w*(x - s*(q + delta))^2 and the rule
 *     that uniform importance reproduces the unweighted payload;
 *   - "Register each GGML IQ format once" (#2525), IQ2_S commit body,
 *     "What's distinctive about it": IQ2_XS's parity-coded signs;
 *   - "[4/4] Run the local-Hessian choice search as one CUDA kernel" (#3218)
 *     with the embedded #3157 (fixed choices), #3158 (local_hessian steps 1-3)
 *     and #3159 (every-choice encode) bodies.
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise; the caller
 *     allocates and owns every buffer.  The library allocates no device memory.
 *   - Calls are asynchronous and ordered on `stream` (NULL = the null stream).
 *     Argument and shape errors are returned synchronously before any launch,
 *     and nothing is written; the format is checked first, then the shape,
 *     then the pointers, then sizes and alignment (fp32 arrays read or
 *     written as vectors need 16-byte alignment, 16-bit arrays 2-byte
 *     alignment).  Data errors found on the device (non-finite weight, bad
 *     importance, scale out of fp16 range, payload index beyond the grid) are
 *     written to `*status` with an atomic compare-and-swap from 0, so the first
 *     code to land sticks; the library never clears `*status`: the caller
 *     zeroes it.  Blocks with a data error are written as zeros.
 *   - `status` may be NULL in every call that takes it.  The call then
 *     reports into a status word of the library's own (one per device, a
 *     file-scope device variable: nothing is allocated), waits for `stream`
 *     to drain, and returns the first data error code, or IQ_OK.  Such calls
 *     block the host, cannot be captured in a graph, and are serialized per
 *     device by a lock the library holds until the word has been read back.
 *   - Concurrent calls that share `status` or an output buffer race.
 *   - Layouts are row-major and contiguous.  Weights are [batch][rows][cols]
 *     with cols a positive multiple of 256, stored as fp32, bf16, fp16 or fp64
 *     (iq_dtype_t); a 256-value block is cols/256 of a row; the packed payload
 *     is [batch][rows][cols/256][block_bytes] uint8.
 */
#ifndef IQ_CODEC_H
#define IQ_CODEC_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    IQ_FMT_IQ1_S = 0,   /* 2048-entry ternary grid, 50-byte blocks (1.5625 bpw) */
    IQ_FMT_IQ2_XS = 1,  /* 512-entry magnitude grid, 74-byte blocks (2.3125 bpw) */
    IQ_FMT_IQ1_M = 2    /* the IQ1_S grid, 56-byte blocks (1.75 bpw): a 3-bit local scale per
                           16 values, a shift per group, d in the top nibbles of the scale words */
} iq_format_t;

/* Storage type of the weights given to the encode calls (#2450 code review:
 * the encoders take float32, float64, float16 and bfloat16 weights).  Every
 * value is read as fp32 -- exactly for bf16 and fp16, rounded to nearest even
 * for fp64 (an fp64 value beyond fp32's range becomes infinite and its block
 * is rejected as non-finite) -- and the encode is that of the fp32 values. */
typedef enum {
    IQ_DTYPE_F32 = 0,
    IQ_DTYPE_BF16 = 1,
    IQ_DTYPE_F16 = 2,
    IQ_DTYPE_F64 = 3
} iq_dtype_t;

typedef enum {
    IQ_OK = 0,
    IQ_ERR_NULL = 1,          /* a required pointer is NULL */
    IQ_ERR_FORMAT = 2,        /* unknown format, or not supported by this call */
    IQ_ERR_SHAPE = 3,         /* empty tensor, cols not a multiple of 256, size overflow */
    IQ_ERR_GRID = 4,          /* grid_size outside [1, 2^index_bits], or (device) a grid
                                 value that is not ternary (IQ1_S) / not finite and >= 0 (IQ2_XS) */
    IQ_ERR_NONFINITE = 5,     /* (device) a weight is NaN or infinite */
    IQ_ERR_IMPORTANCE = 6,    /* (device) an importance value is negative or not finite */
    IQ_ERR_SCALE_RANGE = 7,   /* (device) super-block scale beyond fp16, or a pinned scale
                                 that is negative, infinite or NaN */
    IQ_ERR_ARG = 8,           /* a count out of range (top_c, G, C, sweeps, choice values),
                                 an unknown weight dtype, a misaligned pointer */
    IQ_ERR_CODE = 9,          /* (device) a payload grid index beyond grid_size */
    IQ_ERR_HIP = 10,          /* a HIP runtime call or kernel launch failed */
    IQ_ERR_DEVICE = 11        /* the current device is not a gfx950 GPU */
} iq_status_t;

typedef struct {
    int32_t block_elems;    /* 256 values per super-block */
    int32_t block_bytes;    /* 50 (IQ1_S) or 74 (IQ2_XS) */
    int32_t group;          /* 8 values per grid entry */
    int32_t index_bits;     /* 11 (IQ1_S, IQ1_M) or 9 (IQ2_XS) */
    int32_t grid_max;       /* 2048 or 512 entries at most */
    int32_t choice_groups;  /* choice groups per block: 8 sub-blocks of 32 (IQ1_S),
                               16 scale groups of 16 (IQ2_XS, IQ1_M) */
    int32_t num_choices;    /* 16: IQ1_S k + 8*deltabit, IQ2_XS local scale k;
                               8: IQ1_M local scale k (the shift is free per group) */
} iq_format_info_t;

/* Geometry of a format (#2450 review: 50/74-byte blocks; #2525 IQ1_M bodies:
 * 1.75 bpw; #3157: choice_groups and num_choices recorded per format).  `out`
 * is a HOST pointer. */
iq_status_t iq_format_info(iq_format_t fmt, iq_format_info_t* out);

/* Human-readable name of a status code (static string, never NULL). */
const char* iq_status_str(iq_status_t st);

/*
 * iq_encode -- importance-weighted exhaustive codebook-search encode (#2450
 * review: scale predictor, 16-way choice, lowest index wins; #2723: objective
 * sum w*(x - s*(q+delta))^2 with the local scale and delta shared by the 4
 * groups of a 32-value sub-block; #2525/#2512: IQ2_XS signs with the weakest
 * element flipped for even parity).
 *
 *   wdtype     the storage type of w (see iq_dtype_t).
 *   w          [batch][rows][cols] weights in wdtype, 16-byte aligned.
 *   importance NULL (uniform) or [batch][cols] fp32, finite and >= 0, one value
 *              per input column (#2723).
 *   grid       [grid_size][8] fp32.  IQ1_S: values in {-1, 0, +1};
 *              IQ2_XS: finite magnitudes >= 0.
 *   scales     NULL (predict d = fp16((amax/16.875)*0.61) for IQ1_S,
 *              fp16((amax/155)*0.61) for IQ2_XS, and for IQ1_M
 *              fp16((amax/16.875)*clamp(0.58 + 0.035*amax/rms, 0.65, 0.95))
 *              with rms over the block's 256 values, #2525 IQ1_M body "A
 *              scale-anchor correction") or pinned fp16 bits
 *              [batch][rows][cols/256] (#3197 static scales).
 *   choices    NULL (search every choice) or forced per-choice-group picks
 *              [batch][rows][cols/256][choice_groups] int32 in [0, num_choices)
 *              (#3157): IQ1_S c = k + 8*deltabit, IQ2_XS and IQ1_M c = k (IQ1_M
 *              keeps each group's shift free).  Only the rest is searched then;
 *              a value out of range zeroes its block and sets
 *              *status = IQ_ERR_ARG.
 * IQ1_M ties: the lower shift, then the lower entry (#2525 IQ1_M CUDA body).
 *   out        [batch][rows][cols/256][block_bytes] uint8.
 *   status     NULL, or one int32 (see the conventions above).
 * Errors: IQ_ERR_NULL, IQ_ERR_FORMAT, IQ_ERR_SHAPE, IQ_ERR_GRID, IQ_ERR_DEVICE,
 * IQ_ERR_HIP synchronously; the device codes through *status, or as the
 * return value when status is NULL.
 */
iq_status_t iq_encode(iq_format_t fmt, iq_dtype_t wdtype, const void* w, int64_t batch,
                      int64_t rows, int64_t cols, const float* importance, const float* grid,
                      int32_t grid_size, const uint16_t* scales, const int32_t* choices,
                      uint8_t* out, int32_t* status, hipStream_t stream);

/*
 * iq_encode_every_choice -- the payload under every choice from one sweep
 * ("[2/4] Encode every GGML IQ choice in one pass" #3159): out[c] is, byte for
 * byte, the iq_encode payload with every choice group forced to c.  The input
 * of the local-Hessian search, which scores each choice's decoded error.
 *
 *   wdtype, w, importance, grid, scales, status: as iq_encode.
 *   out  [num_choices][batch][rows][cols/256][block_bytes] uint8 (choice-major;
 *        16 payloads for IQ1_S and IQ2_XS, 8 for IQ1_M).
 * Errors as iq_encode; a block with a data error is zero in all 16 payloads.
 */
iq_status_t iq_encode_every_choice(iq_format_t fmt, iq_dtype_t wdtype, const void* w,
                                   int64_t batch, int64_t rows, int64_t cols,
                                   const float* importance, const float* grid, int32_t grid_size,
                                   const uint16_t* scales, uint8_t* out, int32_t* status,
                                   hipStream_t stream);

/*
 * iq_fake_quant -- encode and decode in one pass: the fp32 weights the
 * payload stands for, which the fake-quant forward uses and re-encodes after
 * every optimizer step ("Re-encode GGML weights after every optimizer step, so
 * Megatron QAD updates their codes" #3210, with the static scales of #3197:
 * re-encode under pinned d).  xhat is, bit for bit,
 * iq_dequant(iq_encode(...)) with the same arguments.
 *
 *   wdtype, w, importance, grid, scales, choices, status: as iq_encode.
 *   xhat  [batch][rows][cols] fp32 output (whatever wdtype is); may not
 *         overlap w.
 *   out   NULL, or the payload [batch][rows][cols/256][block_bytes] as well.
 * Errors as iq_encode (IQ_ERR_ARG also when xhat overlaps w); a block with a
 * data error decodes to zeros.
 */
iq_status_t iq_fake_quant(iq_format_t fmt, iq_dtype_t wdtype, const void* w, int64_t batch,
                          int64_t rows, int64_t cols, const float* importance, const float* grid,
                          int32_t grid_size, const uint16_t* scales, const int32_t* choices,
                          float* xhat, uint8_t* out, int32_t* status, hipStream_t stream);

/*
 * iq_dequant -- decode a payload to fp32 (#2450 review worked example:
 * IQ1_S value = d*(2k+1)*(q + delta), delta = -1/8 when bit 15 is set;
 * IQ2_XS value = d*(2k+1)*sign*q with the 8th sign of a group implied by even
 * parity; IQ1_M value = d*(2k+1)*(q + delta) with d reassembled from the scale
 * words' top nibbles, k per 16 values and delta per group).  Every decoded
 * value is exact in fp32 (IQ2_XS: for grid magnitudes of at most 8
 * significant bits).
 *
 *   packed  [batch][rows][cols/256][block_bytes] uint8.
 *   grid    [grid_size][8] fp32 (the grid the payload was encoded with).
 *   out     [batch][rows][cols] fp32.
 *   status  NULL or one int32 (see the conventions above); IQ_ERR_CODE if an
 *           index is >= grid_size (that group decodes to zeros).
 */
iq_status_t iq_dequant(iq_format_t fmt, const uint8_t* packed, int64_t batch, int64_t rows,
                       int64_t cols, const float* grid, int32_t grid_size, float* out,
                       int32_t* status, hipStream_t stream);

/*
 * iq_encode_candidates -- the encode's sweep with a candidate epilogue, the
 * input of the local-Hessian choice search (#3158 step 1, #3159 every-choice
 * encode): for every choice group of every 256-column block (IQ2_XS and
 * IQ1_M: 16 scale groups of 16 columns, choice = local scale k; IQ1_S: 8
 * sub-blocks of 32 columns, choice c = k + 8*deltabit), the top_c choices
 * ordered by (weighted cost, choice), each with its grid codes and its error
 * vector xhat - x over the group's columns (xhat formed exactly, one rounding
 * of xhat - x).  A zero super-block scale orders the choices 0, 1, ... with
 * entry 0.
 *
 *   wdtype, w   [rows][cols] weights in wdtype (as iq_encode); importance NULL
 *               or [cols]; grid as iq_encode.  x in xhat - x is the weight read
 *               as fp32.
 *   top_c       1..num_choices (16, or 8 for IQ1_M).
 *   cand_err    IQ2_XS, IQ1_M [rows][cols/256][16][top_c][16],
 *               IQ1_S [rows][cols/256][8][top_c][32] fp32.
 *   cand_choice [rows][cols/256][G][top_c] int32 (G = 16 or 8).
 *   cand_codes  NULL, or IQ2_XS [..][top_c][2] uint16 (index | mask<<9 per group),
 *               IQ1_M [..][top_c][2] (index | shift<<11 per group),
 *               IQ1_S [..][top_c][4] uint16 (the grid index of each group).
 *   status      NULL or one int32 (see the conventions above); a block with a
 *               data error is all zeros.
 */
iq_status_t iq_encode_candidates(iq_format_t fmt, iq_dtype_t wdtype, const void* w, int64_t rows,
                                 int64_t cols, const float* importance, const float* grid,
                                 int32_t grid_size, int32_t top_c, float* cand_err,
                                 int32_t* cand_choice, uint16_t* cand_codes, int32_t* status,
                                 hipStream_t stream);

/*
 * iq_choice_search -- local-Hessian choice search of one 256-column block
 * (#3158 steps 2-3; #3218 one launch per block): per row, give each group the
 * candidate with the least e^T H_gg e, then visit the groups in ascending
 * order `sweeps` times, each taking the candidate that most lowers the row's
 * e^T H e with the other groups held, only on a strict improvement; ties go to
 * the lowest candidate index.
 *
 *   H        [256][256] fp32, symmetric (the caller damps it).
 *   cand_err [rows][G][C][256/G] fp32 candidate error vectors, 16-byte aligned
 *            (each vector is read as 16-byte words; IQ_ERR_ARG otherwise).
 *   G        8 or 16 groups; C in 1..16 candidates; sweeps in 0..8.
 *   picks    [rows][G] int32 output, candidate indices.
 *   trace    NULL or [sweeps+1][rows][G] int32: picks after step 2 and after
 *            every sweep.
 */
iq_status_t iq_choice_search(const float* H, const float* cand_err, int64_t rows, int32_t G,
                             int32_t C, int32_t sweeps, int32_t* picks, int32_t* trace,
                             hipStream_t stream);

/*
 * iq_choice_search_blocks -- the same search for many 256-column blocks in
 * one launch, each block with its own H ("[4/4] Run the local-Hessian choice
 * search as one CUDA kernel" #3218 fuses the search of one block; the pages'
 * MoE calibration has many small blocks, where per-block launches dominate).
 * iq_choice_search is this call with nblk = 1.
 *
 *   H        [nblk][256][256] fp32, each symmetric.
 *   cand_err [rows][nblk][G][C][256/G] fp32: what iq_encode_candidates writes
 *            for a [rows][256*nblk] weight.
 *   nblk     1..65535 (IQ_ERR_SHAPE otherwise).
 *   picks    [rows][nblk][G] int32; trace NULL or [sweeps+1][rows][nblk][G].
 * G, C, sweeps and the errors as iq_choice_search.
 */
iq_status_t iq_choice_search_blocks(const float* H, const float* cand_err, int64_t rows,
                                    int64_t nblk, int32_t G, int32_t C, int32_t sweeps,
                                    int32_t* picks, int32_t* trace, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* IQ_CODEC_H */
