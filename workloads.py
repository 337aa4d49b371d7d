"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and lays them out.  It holds none of the
codec's arithmetic (no scale prediction, no search, no packing), so the oracle
and the HIP path can both take their inputs from here without sharing code.

Recipes (numpy ``default_rng``, drawn in float64, cast to float32):

* Grids: a random permutation of the 3**8 ternary patterns, first ``n`` kept,
  each pattern read as 8 base-3 digits (digit j = element j).  IQ1_S maps the
  digits {0,1,2} to {-1,0,+1}; IQ2_XS maps them to the magnitudes {1,3,5}.
  All entries are distinct.  The real GGML tables are third-party data and
  are not reproduced; the grid is an input of every call.
* Weights: 0.02 * N(0,1), or 0.02 * Student-t with 5 degrees of freedom.
* Importance: the square root of a lognormal(0,1) Hessian diagonal, i.e.
  exp(N(0,1) / 2), one value per input column.
* Block Hessian: H = U^-1 U^-T with U upper-triangular, diagonal 1+|N(0,1)|,
  strict upper part 0.05 * N(0,1); formed in float64, symmetrised, cast to
  float32.
"""

from __future__ import annotations

import numpy as np

IQ1S_GRID_SIZE = 2048
IQ2XS_GRID_SIZE = 512


def _ternary_patterns(n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    codes = rng.permutation(3 ** 8)[:n]
    digits = np.empty((n, 8), dtype=np.int64)
    v = codes.copy()
    for j in range(8):
        digits[:, j] = v % 3
        v //= 3
    return digits


def iq1s_grid(n: int = IQ1S_GRID_SIZE, seed: int = 0) -> np.ndarray:
    """[n, 8] float32 ternary grid with values in {-1, 0, +1}, distinct rows."""
    d = _ternary_patterns(n, seed)
    return (d - 1).astype(np.float32)


def iq2xs_grid(n: int = IQ2XS_GRID_SIZE, seed: int = 0) -> np.ndarray:
    """[n, 8] float32 magnitude grid with values in {1, 3, 5}, distinct rows."""
    d = _ternary_patterns(n, seed)
    return (2 * d + 1).astype(np.float32)


def iq2xs_wide_grid(n: int = IQ2XS_GRID_SIZE, seed: int = 0) -> np.ndarray:
    """[n, 8] float32 magnitude grid with values in {8, 25, 43}, distinct rows:
    integer magnitudes whose squares (625, 1849) need more than bf16's 8
    significant bits."""
    d = _ternary_patterns(n, seed)
    return np.array([8.0, 25.0, 43.0], np.float32)[d]


def iq2xs_real_grid(n: int = IQ2XS_GRID_SIZE, seed: int = 0) -> np.ndarray:
    """[n, 8] float32 magnitude grid of arbitrary positive values, uniform in
    [0.25, 6)."""
    rng = np.random.default_rng(seed)
    return rng.uniform(0.25, 6.0, size=(n, 8)).astype(np.float32)


def normal_weight(shape, seed: int, std: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (std * rng.standard_normal(size=shape)).astype(np.float32)


def student_t_weight(shape, seed: int, scale: float = 0.02, df: float = 5.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_t(df, size=shape)).astype(np.float32)


def lognormal_importance(shape, seed: int) -> np.ndarray:
    """sqrt(exp(N(0,1))) = exp(N(0,1)/2), float32."""
    rng = np.random.default_rng(seed)
    return np.exp(0.5 * rng.standard_normal(size=shape)).astype(np.float32)


def block_hessian(n: int = 256, seed: int = 7) -> np.ndarray:
    rng = np.random.default_rng(seed)
    u = np.triu(0.05 * rng.standard_normal((n, n)), k=1)
    u[np.diag_indices(n)] = 1.0 + np.abs(rng.standard_normal(n))
    uinv = np.linalg.inv(u)
    h = uinv @ uinv.T
    h = 0.5 * (h + h.T)
    return h.astype(np.float32)


# --------------------------------------------------------------------------
# The five workloads.  Each returns a dict of numpy arrays.
# --------------------------------------------------------------------------

def c1_iq1s_small():
    """IQ1_S, one 64x256 weight, 0.02*N(0,1) seed 0, no importance."""
    return {"fmt": "iq1_s", "w": normal_weight((1, 64, 256), 0), "importance": None,
            "grid": iq1s_grid()}


def c2_iq1s_4096():
    """IQ1_S weighted, 4096x4096, weight seed 1, importance seed 2."""
    return {"fmt": "iq1_s", "w": normal_weight((1, 4096, 4096), 1),
            "importance": lognormal_importance((1, 4096), 2), "grid": iq1s_grid()}


def c3_iq2xs_4096():
    """IQ2_XS weighted, 4096x4096 0.02*t5 weight seed 3, importance seed 4."""
    return {"fmt": "iq2_xs", "w": student_t_weight((1, 4096, 4096), 3),
            "importance": lognormal_importance((1, 4096), 4), "grid": iq2xs_grid()}


def c4_moe_batch():
    """16 experts of 1536x4096, 0.02*N(0,1) seed 5, per-expert importance seed 6."""
    return {"fmt": "iq1_s", "w": normal_weight((16, 1536, 4096), 5),
            "importance": lognormal_importance((16, 4096), 6), "grid": iq1s_grid()}


def c5_choice_search():
    """4096 rows x one 256-column block of the IQ2_XS weight, H from seed 7."""
    h = block_hessian(256, 7)
    w = student_t_weight((1, 4096, 4096), 3)[:, :, :256].copy()
    imp = np.sqrt(np.diag(h).astype(np.float64)).astype(np.float32)[None, :]
    return {"fmt": "iq2_xs", "w": w, "importance": imp, "grid": iq2xs_grid(), "H": h,
            "top_c": 8, "sweeps": 2}


def c5_iq1s_choice_search():
    """The search workload for IQ1_S: 4096 rows x the first 256 columns of the
    IQ1_S weight (seed 1), H from seed 7, importance sqrt(diag H), top-8 of the
    16 (k, delta) choices per 32-column sub-block (G = 8)."""
    h = block_hessian(256, 7)
    w = normal_weight((1, 4096, 4096), 1)[:, :, :256].copy()
    imp = np.sqrt(np.diag(h).astype(np.float64)).astype(np.float32)[None, :]
    return {"fmt": "iq1_s", "w": w, "importance": imp, "grid": iq1s_grid(), "H": h,
            "top_c": 8, "sweeps": 2}


def c5_weight_choice_search():
    """Local-Hessian calibration of a whole IQ2_XS weight: the 4096x4096 weight
    of c3 (seed 3), one H per 256-column block (seeds 7..22), importance
    sqrt(diag H) per column, top-8 candidates, 16 blocks searched in one launch."""
    hs = np.stack([block_hessian(256, 7 + b) for b in range(16)])
    w = student_t_weight((1, 4096, 4096), 3)
    imp = np.sqrt(np.concatenate([np.diag(h) for h in hs]).astype(np.float64)).astype(np.float32)
    return {"fmt": "iq2_xs", "w": w, "importance": imp[None, :], "grid": iq2xs_grid(), "H": hs,
            "top_c": 8, "sweeps": 2}


def c2_iq1m_4096():
    """IQ1_M weighted encode of the IQ1_S workload's 4096x4096 weight (seed 1),
    importance seed 2, the IQ1_S grid (IQ1_M shares it)."""
    return dict(c2_iq1s_4096(), fmt="iq1_m")


CONFIGS = {
    "c1": c1_iq1s_small,
    "c2": c2_iq1s_4096,
    "c3": c3_iq2xs_4096,
    "c4": c4_moe_batch,
    "c5": c5_choice_search,
    "c5_iq1s": c5_iq1s_choice_search,
    "c5_weight": c5_weight_choice_search,
    "c2_iq1m": c2_iq1m_4096,
}
