"""Python binding of libiqcodec.so: MI355X-native importance-weighted IQ1_S /
IQ2_XS codebook-search encode, decode, candidate emission and local-Hessian
choice search.

This module only marshals arguments: it checks tensors, takes their device
pointers and the current HIP stream from PyTorch, and calls the C-ABI declared
in ``include/iq_codec.h``.  Every step of the computation runs in the HIP
kernels of the library.  There is no CPU path: if the library is not built, or
the device is not a gfx950 GPU, calls raise.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (device memory and streams; loads the HIP runtime first)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libiqcodec.so")

FORMATS = {"iq1_s": 0, "iq2_xs": 1, "iq1_m": 2}
BLOCK_BYTES = {"iq1_s": 50, "iq2_xs": 74, "iq1_m": 56}
CHOICE_GROUPS = {"iq1_s": 8, "iq2_xs": 16, "iq1_m": 16}
NUM_CHOICES = {"iq1_s": 16, "iq2_xs": 16, "iq1_m": 8}

STATUS = {
    0: "IQ_OK", 1: "IQ_ERR_NULL", 2: "IQ_ERR_FORMAT", 3: "IQ_ERR_SHAPE", 4: "IQ_ERR_GRID",
    5: "IQ_ERR_NONFINITE", 6: "IQ_ERR_IMPORTANCE", 7: "IQ_ERR_SCALE_RANGE", 8: "IQ_ERR_ARG",
    9: "IQ_ERR_CODE", 10: "IQ_ERR_HIP", 11: "IQ_ERR_DEVICE",
}


class IQError(RuntimeError):
    """A non-zero iq_status_t from the library."""

    def __init__(self, code: int, where: str):
        self.code = int(code)
        self.name = STATUS.get(self.code, "unknown")
        super().__init__("%s: %s (%d): %s" % (where, self.name, self.code, _status_str(self.code)))


class _FormatInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("block_elems", "block_bytes", "group", "index_bits",
                                               "grid_max", "choice_groups", "num_choices")]


_lib = None


def load(build_if_missing: bool = True):
    """Load libiqcodec.so (building it first only if it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise ImportError("libiqcodec.so is not built (run ggml_iq_codebook_amd.build.build())")
        from . import build as _build
        _build.build()
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.iq_format_info.argtypes = [ctypes.c_int, ctypes.POINTER(_FormatInfo)]
    L.iq_format_info.restype = ctypes.c_int
    L.iq_status_str.argtypes = [ctypes.c_int]
    L.iq_status_str.restype = ctypes.c_char_p
    L.iq_encode.argtypes = [ctypes.c_int, ctypes.c_int, P, i64, i64, i64, P, P, i32, P, P, P, P, P]
    L.iq_encode.restype = ctypes.c_int
    L.iq_encode_every_choice.argtypes = [ctypes.c_int, ctypes.c_int, P, i64, i64, i64, P, P, i32,
                                         P, P, P, P]
    L.iq_encode_every_choice.restype = ctypes.c_int
    L.iq_fake_quant.argtypes = [ctypes.c_int, ctypes.c_int, P, i64, i64, i64, P, P, i32, P, P, P,
                                P, P, P]
    L.iq_fake_quant.restype = ctypes.c_int
    L.iq_dequant.argtypes = [ctypes.c_int, P, i64, i64, i64, P, i32, P, P, P]
    L.iq_dequant.restype = ctypes.c_int
    L.iq_encode_candidates.argtypes = [ctypes.c_int, ctypes.c_int, P, i64, i64, P, P, i32, i32, P,
                                       P, P, P, P]
    L.iq_encode_candidates.restype = ctypes.c_int
    L.iq_choice_search.argtypes = [P, P, i64, i32, i32, i32, P, P, P]
    L.iq_choice_search.restype = ctypes.c_int
    L.iq_choice_search_blocks.argtypes = [P, P, i64, i64, i32, i32, i32, P, P, P]
    L.iq_choice_search_blocks.restype = ctypes.c_int
    _lib = L
    return L


def _status_str(code: int) -> str:
    try:
        return load().iq_status_str(int(code)).decode()
    except Exception:  # pragma: no cover - only for messages
        return ""


def _check(code: int, where: str):
    if code != 0:
        raise IQError(code, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev_tensor(t, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _fmt(fmt):
    if fmt not in FORMATS:
        raise ValueError("unknown format %r" % (fmt,))
    return FORMATS[fmt]


def format_info(fmt: str) -> dict:
    info = _FormatInfo()
    _check(load().iq_format_info(_fmt(fmt), ctypes.byref(info)), "iq_format_info")
    return {n: getattr(info, n) for n, _ in _FormatInfo._fields_}


def _status_arg(status, check, device):
    """The status word to pass.  None with ``check``: NULL, so that the library
    synchronizes the stream and returns the first data error as the call's
    code.  None without ``check``: a fresh zeroed word nobody reads (the call
    stays asynchronous).  Otherwise the caller's int32 tensor."""
    if status is None:
        return None if check else torch.zeros(1, dtype=torch.int32, device=device)
    _dev_tensor(status, torch.int32, "status")
    return status


def _raise_on_status(status, check, where):
    """With ``check`` and a caller's status word: synchronize and raise on a
    data error (with a NULL word the call's own code has been checked)."""
    if not check or status is None:
        return
    code = int(status.item())
    if code:
        raise IQError(code, where)


# Storage types of the weight (iq_dtype_t): the encode reads each value as
# fp32 (exactly, or rounded to nearest even from fp64).
WEIGHT_DTYPES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2, torch.float64: 3}


def _weight(w):
    """The iq_dtype_t code of a weight tensor, after the device checks."""
    if not isinstance(w, torch.Tensor):
        raise TypeError("w must be a torch.Tensor")
    if w.dtype not in WEIGHT_DTYPES:
        raise TypeError("w must be float32, bfloat16, float16 or float64, got %s" % (w.dtype,))
    _dev_tensor(w, w.dtype, "w")
    return WEIGHT_DTYPES[w.dtype]


def _encode_args(w, grid, importance, fmt, scales, choices):
    """Checks shared by the encode calls; returns (fmt code, dtype code, B, R, C,
    squeeze, scales)."""
    f = _fmt(fmt)
    dt = _weight(w)
    squeeze = w.dim() == 2
    if w.dim() not in (2, 3):
        raise ValueError("w must be [rows, cols] or [batch, rows, cols]")
    B, R, C = (1, *w.shape) if squeeze else w.shape
    _dev_tensor(grid, torch.float32, "grid")
    if grid.dim() != 2 or grid.shape[1] != 8:
        raise ValueError("grid must be [n, 8]")
    if importance is not None:
        _dev_tensor(importance, torch.float32, "importance")
        if importance.numel() != B * C:
            raise ValueError("importance must have batch*cols = %d values" % (B * C))
    if scales is not None:
        if scales.dtype == torch.int16:
            scales = scales.view(torch.uint16) if hasattr(torch, "uint16") else scales
        if not scales.is_cuda or not scales.is_contiguous() or scales.element_size() != 2:
            raise ValueError("scales must be a contiguous 16-bit GPU tensor of fp16 bits")
        if scales.numel() != B * R * (C // 256):
            raise ValueError("scales must have one value per block")
    if choices is not None:
        _dev_tensor(choices, torch.int32, "choices")
        if choices.numel() != B * R * (C // 256) * CHOICE_GROUPS[fmt]:
            raise ValueError("choices must have %d values per block" % CHOICE_GROUPS[fmt])
    return f, dt, B, R, C, squeeze, scales


def _out_tensor(out, shape, dtype, device, name):
    n = 1
    for v in shape:
        n *= v
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _dev_tensor(out, dtype, name)
    if out.numel() != n:
        raise ValueError("%s has the wrong size" % name)
    return out


def encode(w, grid, importance=None, *, fmt="iq1_s", scales=None, choices=None, out=None,
           status=None, check=True):
    """Encode a [batch, rows, cols] (or [rows, cols]) weight (fp32, bf16, fp16 or
    fp64, read as fp32).

    Returns the packed payload [batch, rows, cols/256, block_bytes] uint8 (the
    batch dimension is dropped again for a 2-D weight).  ``importance`` is
    [batch, cols] / [cols]; ``scales`` pinned fp16 bits [batch, rows, cols/256]
    (int16/uint16 tensor); ``choices`` forced picks [batch, rows, cols/256, G].
    With ``check`` the call synchronizes and raises IQError on a data error.
    """
    f, dt, B, R, C, squeeze, scales = _encode_args(w, grid, importance, fmt, scales, choices)
    out = _out_tensor(out, (B, R, C // 256, BLOCK_BYTES[fmt]), torch.uint8, w.device, "out")
    status = _status_arg(status, check, w.device)
    code = load().iq_encode(f, dt, _ptr(w), B, R, C, _ptr(importance), _ptr(grid), grid.shape[0],
                            _ptr(scales), _ptr(choices), _ptr(out), _ptr(status), _stream())
    _check(code, "iq_encode")
    _raise_on_status(status, check, "iq_encode")
    return out[0] if squeeze else out


def encode_every_choice(w, grid, importance=None, *, fmt="iq1_s", scales=None, out=None,
                        status=None, check=True):
    """The payload under every choice (16, or 8 for IQ1_M), from one sweep.

    Returns [num_choices, batch, rows, cols/256, block_bytes] uint8 (no batch
    dimension for a 2-D weight); entry c equals ``encode(..., choices=full(c))``.
    """
    f, dt, B, R, C, squeeze, scales = _encode_args(w, grid, importance, fmt, scales, None)
    out = _out_tensor(out, (NUM_CHOICES[fmt], B, R, C // 256, BLOCK_BYTES[fmt]), torch.uint8,
                      w.device, "out")
    status = _status_arg(status, check, w.device)
    code = load().iq_encode_every_choice(f, dt, _ptr(w), B, R, C, _ptr(importance), _ptr(grid),
                                         grid.shape[0], _ptr(scales), _ptr(out), _ptr(status),
                                         _stream())
    _check(code, "iq_encode_every_choice")
    _raise_on_status(status, check, "iq_encode_every_choice")
    return out[:, 0] if squeeze else out


def fake_quant(w, grid, importance=None, *, fmt="iq1_s", scales=None, choices=None, out=None,
               packed=False, status=None, check=True):
    """Encode and decode in one pass: the fp32 weight the payload stands for
    (fp32 whatever the weight's storage type).

    Returns xhat shaped like ``w`` (bit for bit ``dequant(encode(...))``), or
    (xhat, payload) with ``packed=True``.
    """
    f, dt, B, R, C, squeeze, scales = _encode_args(w, grid, importance, fmt, scales, choices)
    xhat = _out_tensor(out, (B, R, C), torch.float32, w.device, "out")
    pk = (torch.empty((B, R, C // 256, BLOCK_BYTES[fmt]), dtype=torch.uint8, device=w.device)
          if packed else None)
    status = _status_arg(status, check, w.device)
    code = load().iq_fake_quant(f, dt, _ptr(w), B, R, C, _ptr(importance), _ptr(grid),
                                grid.shape[0], _ptr(scales), _ptr(choices), _ptr(xhat), _ptr(pk),
                                _ptr(status), _stream())
    _check(code, "iq_fake_quant")
    _raise_on_status(status, check, "iq_fake_quant")
    if squeeze:
        xhat = xhat[0]
        pk = None if pk is None else pk[0]
    return (xhat, pk) if packed else xhat


def dequant(packed, grid, *, fmt="iq1_s", out=None, status=None, check=True):
    """Decode [batch, rows, cols/256, block_bytes] (or without batch) to fp32."""
    f = _fmt(fmt)
    _dev_tensor(packed, torch.uint8, "packed")
    _dev_tensor(grid, torch.float32, "grid")
    squeeze = packed.dim() == 3
    if packed.dim() not in (3, 4) or packed.shape[-1] != BLOCK_BYTES[fmt]:
        raise ValueError("packed must be [(batch,) rows, cols/256, %d]" % BLOCK_BYTES[fmt])
    B, R, NB, _ = (1, *packed.shape) if squeeze else packed.shape
    C = NB * 256
    if out is None:
        out = torch.empty((B, R, C), dtype=torch.float32, device=packed.device)
    else:
        _dev_tensor(out, torch.float32, "out")
        if out.numel() != B * R * C:
            raise ValueError("out has the wrong size")
    status = _status_arg(status, check, packed.device)
    code = load().iq_dequant(f, _ptr(packed), B, R, C, _ptr(grid), grid.shape[0], _ptr(out),
                             _ptr(status), _stream())
    _check(code, "iq_dequant")
    _raise_on_status(status, check, "iq_dequant")
    return out[0] if squeeze else out


def encode_candidates(w, grid, importance=None, *, fmt="iq2_xs", top_c=8, codes=False,
                      status=None, check=True):
    """Top-C choices per choice group of every 256-column block of [rows, cols].

    IQ2_XS, IQ1_M: 16 scale groups of 16 columns; IQ1_S: 8 sub-blocks of 32
    columns.  Returns (cand_err [rows, cols/256, G, top_c, 256/G] fp32,
    cand_choice [rows, cols/256, G, top_c] int32, cand_codes [..., 2 (IQ2_XS,
    IQ1_M) or 4 (IQ1_S)] uint16 viewed as int16, or None).
    """
    f = _fmt(fmt)
    dt = _weight(w)
    if w.dim() != 2:
        raise ValueError("w must be [rows, cols]")
    R, C = w.shape
    _dev_tensor(grid, torch.float32, "grid")
    if importance is not None:
        _dev_tensor(importance, torch.float32, "importance")
        if importance.numel() != C:
            raise ValueError("importance must have cols values")
    NB = C // 256
    G = CHOICE_GROUPS[fmt]
    tc = max(int(top_c), 0)
    err = torch.empty((R, NB, G, tc, 256 // G), dtype=torch.float32, device=w.device)
    ch = torch.empty((R, NB, G, tc), dtype=torch.int32, device=w.device)
    ncode = 4 if fmt == "iq1_s" else 2
    cc = (torch.empty((R, NB, G, tc, ncode), dtype=torch.int16, device=w.device)
          if codes else None)
    status = _status_arg(status, check, w.device)
    code = load().iq_encode_candidates(f, dt, _ptr(w), R, C, _ptr(importance), _ptr(grid),
                                       grid.shape[0], int(top_c), _ptr(err), _ptr(ch), _ptr(cc),
                                       _ptr(status), _stream())
    _check(code, "iq_encode_candidates")
    _raise_on_status(status, check, "iq_encode_candidates")
    return err, ch, cc


def choice_search(H, cand_err, *, sweeps=2, trace=False):
    """Local-Hessian choice search.

    One block: H [256, 256] fp32 symmetric, cand_err [rows, G, C, 256/G];
    returns picks [rows, G] int32 (and the trace [sweeps+1, rows, G]).
    Many blocks in one launch: H [nblk, 256, 256], cand_err
    [rows, nblk, G, C, 256/G]; returns picks [rows, nblk, G] (and the trace
    [sweeps+1, rows, nblk, G]).
    """
    _dev_tensor(H, torch.float32, "H")
    _dev_tensor(cand_err, torch.float32, "cand_err")
    if H.dim() == 2:
        if H.shape != (256, 256):
            raise ValueError("H must be [256, 256]")
        if cand_err.dim() != 4 or cand_err.shape[1] * cand_err.shape[3] != 256:
            raise ValueError("cand_err must be [rows, G, C, 256/G]")
        R, G, C, _ = cand_err.shape
        NB = 1
        pshape, tshape = (R, G), (sweeps + 1, R, G)
    else:
        if H.dim() != 3 or H.shape[1:] != (256, 256):
            raise ValueError("H must be [nblk, 256, 256]")
        if (cand_err.dim() != 5 or cand_err.shape[1] != H.shape[0]
                or cand_err.shape[2] * cand_err.shape[4] != 256):
            raise ValueError("cand_err must be [rows, nblk, G, C, 256/G]")
        R, NB, G, C, _ = cand_err.shape
        pshape, tshape = (R, NB, G), (sweeps + 1, R, NB, G)
    picks = torch.empty(pshape, dtype=torch.int32, device=H.device)
    tr = torch.empty(tshape, dtype=torch.int32, device=H.device) if trace else None
    code = load().iq_choice_search_blocks(_ptr(H), _ptr(cand_err), R, NB, G, C, int(sweeps),
                                          _ptr(picks), _ptr(tr), _stream())
    _check(code, "iq_choice_search_blocks")
    return (picks, tr) if trace else picks
