"""CPU oracle of the IQ1_S / IQ2_XS codebook-search encode and choice search.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
bench's ``cpu_baseline`` leg may import this package.  The product path
(``ggml_iq_codebook_amd``) never imports it, and the two share no code: the
arithmetic lives in ``iq_oracle.c`` (plain C, float64, OpenMP over blocks),
which this module loads with ctypes.  Every function below cites, in
``iq_oracle.c``, the passage of the NVIDIA Model-Optimizer pages it follows.

Layouts match the C-ABI of the product so results can be compared directly:
weights ``[batch, rows, cols]`` float32, importance ``[batch, cols]`` or None,
packed ``[batch, rows, cols/256, block_bytes]`` uint8.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "iq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BLOCK_BYTES = {"iq1_s": 50, "iq2_xs": 74, "iq1_m": 56}
NUM_CHOICE_GROUPS = {"iq1_s": 8, "iq2_xs": 16, "iq1_m": 16}
NUM_CHOICES = {"iq1_s": 16, "iq2_xs": 16, "iq1_m": 8}
_ENCODE = {"iq1_s": "orc_iq1s_encode", "iq2_xs": "orc_iq2xs_encode", "iq1_m": "orc_iq1m_encode"}
_DECODE = {"iq1_s": "orc_iq1s_decode", "iq2_xs": "orc_iq2xs_decode", "iq1_m": "orc_iq1m_decode"}

ERRORS = {1: "non-finite weight", 2: "negative or non-finite importance",
          3: "scale out of fp16 range", 4: "bad argument", 5: "grid index beyond the grid"}


class OracleError(ValueError):
    pass


def build(force: bool = True) -> str:
    """Compile iq_oracle.c into liboracle.so (gcc, -O2, OpenMP, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None

# A test build of the oracle to load instead of liboracle.so: the mutation
# tests point this at copies of iq_oracle.c with a planted mistake.
_LIB_OVERRIDE = os.environ.get("IQ_ORACLE_LIB")


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=False)
            L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_predict_scale.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float]
        L.orc_predict_scale.restype = ctypes.c_uint16
        for name in _ENCODE.values():
            f = getattr(L, name)
            f.argtypes = [P, P, i64, P, i32, P, P, P]
            f.restype = ctypes.c_int
        for name in _DECODE.values():
            f = getattr(L, name)
            f.argtypes = [P, i64, P, i32, P]
            f.restype = ctypes.c_int
        L.orc_iq1m_candidates.argtypes = [P, P, i64, P, i32, i32, P, P, P]
        L.orc_iq1m_candidates.restype = ctypes.c_int
        L.orc_iq1m_anchor.argtypes = [P, ctypes.c_float]
        L.orc_iq1m_anchor.restype = ctypes.c_float
        L.orc_iq1m_predict.argtypes = [P, i64, P]
        L.orc_iq1m_predict.restype = None
        L.orc_iq2xs_candidates.argtypes = [P, P, i64, P, i32, i32, P, P, P]
        L.orc_iq2xs_candidates.restype = ctypes.c_int
        L.orc_iq1s_candidates.argtypes = [P, P, i64, P, i32, i32, P, P, P]
        L.orc_iq1s_candidates.restype = ctypes.c_int
        L.orc_choice_search.argtypes = [P, P, i64, i32, i32, i32, P, P]
        L.orc_choice_search.restype = ctypes.c_int
        L.orc_choice_objective.argtypes = [P, P, i32, i32, P]
        L.orc_choice_objective.restype = ctypes.c_double
        L.orc_choice_replay.argtypes = [P, P, i32, i32, i32, P, ctypes.c_double,
                                        ctypes.POINTER(ctypes.c_double)]
        L.orc_choice_replay.restype = ctypes.c_int
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_num_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _blocks(w: np.ndarray, importance):
    """[B,R,C] weight -> [nblk,256] blocks, plus the per-block importance."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim == 2:
        w = w[None]
    B, R, C = w.shape
    if C % 256 or w.size == 0:
        raise OracleError("cols must be a positive multiple of 256")
    x = w.reshape(-1, 256)
    imp = None
    if importance is not None:
        imp = np.ascontiguousarray(importance, dtype=np.float32).reshape(B, C)
        imp = np.ascontiguousarray(np.broadcast_to(imp[:, None, :], (B, R, C))).reshape(-1, 256)
    return w.shape, x, imp


# --------------------------------------------------------------------------
# scale
# --------------------------------------------------------------------------

def f32_to_f16_bits(v: float) -> int:
    return int(lib().orc_f32_to_f16(float(v)))


def f16_bits_to_float(h: int) -> float:
    return float(lib().orc_f16_to_f64(int(h)))


def predict_scale_bits(amax: float, fmt: str = "iq1_s") -> int:
    """fp16 bits of (amax / divisor) * 0.61, computed in fp32 (IQ1_S, IQ2_XS)."""
    divisor = 16.875 if fmt == "iq1_s" else 155.0
    return int(lib().orc_predict_scale(float(amax), divisor, 0.61))


def iq1m_anchor(block) -> float:
    """The IQ1_M peak-to-RMS anchor of one 256-value block (fp32)."""
    x = np.ascontiguousarray(block, dtype=np.float32).reshape(256)
    return float(lib().orc_iq1m_anchor(_ptr(x), float(np.abs(x).max())))


# --------------------------------------------------------------------------
# encode / decode
# --------------------------------------------------------------------------

def encode(fmt: str, w, grid, importance=None, scales=None, choices=None) -> np.ndarray:
    """Exhaustive importance-weighted encode.  Returns [B,R,C/256,bytes] uint8.

    scales: None or fp16 bits [B,R,C/256] (pinned super-block scales).
    choices: None or [B,R,C/256,G] forced per-choice-group picks.
    """
    shape, x, imp = _blocks(w, importance)
    B, R, C = shape
    nblk = x.shape[0]
    grid = np.ascontiguousarray(grid, dtype=np.float32)
    nb = BLOCK_BYTES[fmt]
    out = np.zeros((nblk, nb), dtype=np.uint8)
    sc = None if scales is None else np.ascontiguousarray(scales, dtype=np.uint16).reshape(nblk)
    ch = None
    if choices is not None:
        G = NUM_CHOICE_GROUPS[fmt]
        ch = np.ascontiguousarray(choices, dtype=np.int32).reshape(nblk, G)
        if ch.min() < 0 or ch.max() >= NUM_CHOICES[fmt]:
            raise OracleError("choice out of range")
    f = getattr(lib(), _ENCODE[fmt])
    st = f(_ptr(x), _ptr(imp), nblk, _ptr(grid), grid.shape[0], _ptr(sc), _ptr(ch), _ptr(out))
    if st:
        raise OracleError(ERRORS.get(st, "error %d" % st))
    return out.reshape(B, R, C // 256, nb)


def encode_every_choice(fmt: str, w, grid, importance=None, scales=None) -> np.ndarray:
    """The payload under every choice: [16, B, R, C/256, bytes], entry c being
    the encode with every choice group forced to c, which is how the
    every-choice encode is defined ("[2/4] Encode every GGML IQ choice in one
    pass" #3159, usage: packed[c] equals the forced encode with choices full
    of c)."""
    B, R, C = np.shape(w)
    G = NUM_CHOICE_GROUPS[fmt]
    return np.stack([encode(fmt, w, grid, importance, scales,
                            choices=np.full((B, R, C // 256, G), c, dtype=np.int32))
                     for c in range(NUM_CHOICES[fmt])])


def fake_quant(fmt: str, w, grid, importance=None, scales=None, choices=None) -> np.ndarray:
    """The decoded encode, float64 [B, R, C]: what a fake-quant forward uses
    ("Re-encode GGML weights after every optimizer step" #3210)."""
    return decode(fmt, encode(fmt, w, grid, importance, scales, choices), grid)


def encode_blocks(fmt: str, x, grid, imp=None, scales=None) -> np.ndarray:
    """Encode independent 256-value blocks: x [n, 256], imp None or [n, 256]
    (each block's own importance slice), scales None or fp16 bits [n].
    Returns [n, block_bytes]."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, 256)
    n = x.shape[0]
    imp = None if imp is None else np.ascontiguousarray(imp, dtype=np.float32).reshape(n, 256)
    grid = np.ascontiguousarray(grid, dtype=np.float32)
    nb = BLOCK_BYTES[fmt]
    out = np.zeros((n, nb), dtype=np.uint8)
    sc = None if scales is None else np.ascontiguousarray(scales, dtype=np.uint16).reshape(n)
    f = getattr(lib(), _ENCODE[fmt])
    st = f(_ptr(x), _ptr(imp), n, _ptr(grid), grid.shape[0], _ptr(sc), None, _ptr(out))
    if st:
        raise OracleError(ERRORS.get(st, "error %d" % st))
    return out


def block_errors(fmt: str, packed_blocks, x, grid, imp=None) -> np.ndarray:
    """Weighted squared error per choice group of independent blocks:
    packed_blocks [n, bytes], x [n, 256], imp None or [n, 256] -> [n, G]."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, 256)
    n = x.shape[0]
    nb = BLOCK_BYTES[fmt]
    xhat = decode(fmt, np.ascontiguousarray(packed_blocks).reshape(n, 1, nb), grid).reshape(n, 256)
    wt = np.ones((n, 256)) if imp is None else np.asarray(imp, dtype=np.float64).reshape(n, 256)
    e = wt * (x.astype(np.float64) - xhat) ** 2
    G = NUM_CHOICE_GROUPS[fmt]
    return e.reshape(n, G, 256 // G).sum(axis=2)


def predict_scales(fmt: str, w) -> np.ndarray:
    """fp16 bits of the predicted scale of every 256-value block of w."""
    x = np.ascontiguousarray(w, dtype=np.float32).reshape(-1, 256)
    if fmt == "iq1_m":
        out = np.zeros(x.shape[0], dtype=np.uint16)
        lib().orc_iq1m_predict(_ptr(x), x.shape[0], _ptr(out))
        return out
    amax = np.abs(x).max(axis=1)
    return np.array([predict_scale_bits(a, fmt) for a in amax], dtype=np.uint16)


def decode(fmt: str, packed, grid, strict: bool = True) -> np.ndarray:
    """Decode to float64, shape [..., cols].  An index beyond the grid raises
    (strict) or decodes its group to zero."""
    nb = BLOCK_BYTES[fmt]
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    lead = p.shape[:-2]
    nblk = p.size // nb
    grid = np.ascontiguousarray(grid, dtype=np.float32)
    out = np.zeros((nblk, 256), dtype=np.float64)
    f = getattr(lib(), _DECODE[fmt])
    st = f(_ptr(p), nblk, _ptr(grid), grid.shape[0], _ptr(out))
    if st and strict:
        raise OracleError(ERRORS.get(st, "error %d" % st))
    return out.reshape(*lead, p.shape[-2] * 256)


def iq2xs_candidates(w, grid, importance=None, top_c: int = 8):
    """Top-C local scales per 16-column scale group with their error vectors.

    Returns cand_err [B*R*C/256, 16, top_c, 16] float32 (xhat - x),
    cand_choice [.., 16, top_c] int32 and cand_codes [.., 16, top_c, 2] uint16.
    """
    shape, x, imp = _blocks(w, importance)
    nblk = x.shape[0]
    grid = np.ascontiguousarray(grid, dtype=np.float32)
    err = np.zeros((nblk, 16, top_c, 16), dtype=np.float32)
    ch = np.zeros((nblk, 16, top_c), dtype=np.int32)
    codes = np.zeros((nblk, 16, top_c, 2), dtype=np.uint16)
    st = lib().orc_iq2xs_candidates(_ptr(x), _ptr(imp), nblk, _ptr(grid), grid.shape[0], top_c,
                                    _ptr(err), _ptr(ch), _ptr(codes))
    if st:
        raise OracleError(ERRORS.get(st, "error %d" % st))
    return err, ch, codes


def iq1s_candidates(w, grid, importance=None, top_c: int = 8):
    """Top-C choices c = k + 8*deltabit per 32-column IQ1_S sub-block with their
    error vectors.

    Returns cand_err [B*R*C/256, 8, top_c, 32] float32 (xhat - x),
    cand_choice [.., 8, top_c] int32 and cand_codes [.., 8, top_c, 4] uint16
    (the four grid entries).
    """
    shape, x, imp = _blocks(w, importance)
    nblk = x.shape[0]
    grid = np.ascontiguousarray(grid, dtype=np.float32)
    err = np.zeros((nblk, 8, top_c, 32), dtype=np.float32)
    ch = np.zeros((nblk, 8, top_c), dtype=np.int32)
    codes = np.zeros((nblk, 8, top_c, 4), dtype=np.uint16)
    st = lib().orc_iq1s_candidates(_ptr(x), _ptr(imp), nblk, _ptr(grid), grid.shape[0], top_c,
                                   _ptr(err), _ptr(ch), _ptr(codes))
    if st:
        raise OracleError(ERRORS.get(st, "error %d" % st))
    return err, ch, codes


def iq1m_candidates(w, grid, importance=None, top_c: int = 8):
    """Top-C local scales k (of 8) per 16-column IQ1_M scale group with their
    error vectors (each group's shift is searched freely under k).

    Returns cand_err [B*R*C/256, 16, top_c, 16] float32, cand_choice
    [.., 16, top_c] int32 and cand_codes [.., 16, top_c, 2] uint16
    (entry | shift << 11).
    """
    shape, x, imp = _blocks(w, importance)
    nblk = x.shape[0]
    grid = np.ascontiguousarray(grid, dtype=np.float32)
    err = np.zeros((nblk, 16, top_c, 16), dtype=np.float32)
    ch = np.zeros((nblk, 16, top_c), dtype=np.int32)
    codes = np.zeros((nblk, 16, top_c, 2), dtype=np.uint16)
    st = lib().orc_iq1m_candidates(_ptr(x), _ptr(imp), nblk, _ptr(grid), grid.shape[0], top_c,
                                   _ptr(err), _ptr(ch), _ptr(codes))
    if st:
        raise OracleError(ERRORS.get(st, "error %d" % st))
    return err, ch, codes


def candidates(fmt: str, w, grid, importance=None, top_c: int = 8):
    """The top-C candidates of any format (see the per-format functions)."""
    f = {"iq1_s": iq1s_candidates, "iq2_xs": iq2xs_candidates, "iq1_m": iq1m_candidates}[fmt]
    return f(w, grid, importance, top_c)


# --------------------------------------------------------------------------
# choice search
# --------------------------------------------------------------------------

def choice_search(H, cand_err, sweeps: int = 2):
    """cand_err [rows, G, C, 256/G]; returns (picks [rows,G], trace [sweeps+1,rows,G])."""
    H = np.ascontiguousarray(H, dtype=np.float32)
    cand = np.ascontiguousarray(cand_err, dtype=np.float32)
    rows, G, C, L = cand.shape
    picks = np.zeros((rows, G), dtype=np.int32)
    trace = np.zeros((sweeps + 1, rows, G), dtype=np.int32)
    st = lib().orc_choice_search(_ptr(H), _ptr(cand), rows, G, C, sweeps, _ptr(picks), _ptr(trace))
    if st:
        raise OracleError(ERRORS.get(st, "error %d" % st))
    return picks, trace


def choice_objective(H, cand_err, picks) -> np.ndarray:
    """J = e^T H e per row for the given picks (float64)."""
    H = np.ascontiguousarray(H, dtype=np.float32)
    cand = np.ascontiguousarray(cand_err, dtype=np.float32)
    picks = np.ascontiguousarray(picks, dtype=np.int32)
    rows, G, C, L = cand.shape
    out = np.empty(rows)
    for r in range(rows):
        out[r] = lib().orc_choice_objective(_ptr(H), _ptr(cand[r]), G, C, _ptr(picks[r]))
    return out


def choice_replay(H, cand_row, trace_row, tol: float):
    """Check another implementation's decisions on one row; (fail_index, worst)."""
    H = np.ascontiguousarray(H, dtype=np.float32)
    cand = np.ascontiguousarray(cand_row, dtype=np.float32)
    tr = np.ascontiguousarray(trace_row, dtype=np.int32)
    G, C, L = cand.shape
    worst = ctypes.c_double(0.0)
    fail = lib().orc_choice_replay(_ptr(H), _ptr(cand), G, C, tr.shape[0] - 1, _ptr(tr), tol,
                                   ctypes.byref(worst))
    return int(fail), float(worst.value)


# --------------------------------------------------------------------------
# float64 error of a payload against the weight (used to judge ties)
# --------------------------------------------------------------------------

def unit_errors(fmt: str, packed, w, grid, importance=None) -> np.ndarray:
    """Weighted squared error per choice group (IQ1_S: 32 values, IQ2_XS and IQ1_M: 16).

    Returns [nblk, G] float64: sum over the unit of w * (x - xhat)^2.
    """
    shape, x, imp = _blocks(w, importance)
    xhat = decode(fmt, packed, grid).reshape(-1, 256)
    wt = np.ones_like(x, dtype=np.float64) if imp is None else imp.astype(np.float64)
    e = wt * (x.astype(np.float64) - xhat) ** 2
    G = NUM_CHOICE_GROUPS[fmt]
    return e.reshape(-1, G, 256 // G).sum(axis=2)
