"""Comparison of HIP payloads with the oracle's, under the tie rule.

Codes must be bit-exact, except on floating-point ties: where a choice group
(IQ1_S 32-value sub-block, IQ2_XS and IQ1_M 16-value scale group) differs, the float64
weighted error of the HIP pick must agree with the oracle's within 1e-6
relative.  The scale bytes must always be bit-exact.
"""

import numpy as np

import oracle

TIE_RTOL = 1e-6


def scale_bits(fmt, packed):
    """fp16 bits of every block's d: bytes 0-1, or for IQ1_M the top nibbles of
    its four scale words."""
    p = np.ascontiguousarray(packed).reshape(-1, oracle.BLOCK_BYTES[fmt]).astype(np.int64)
    if fmt == "iq1_m":
        sc = p[:, 48:56:2] | (p[:, 49:56:2] << 8)
        return ((sc[:, 0] >> 12) | ((sc[:, 1] >> 8) & 0x00F0) | ((sc[:, 2] >> 4) & 0x0F00)
                | (sc[:, 3] & 0xF000))
    return p[:, 0] | (p[:, 1] << 8)


def grid_for(fmt, n=None, seed=0):
    """The seeded grid of a format (IQ1_M uses the IQ1_S grid)."""
    import workloads
    if fmt == "iq2_xs":
        return workloads.iq2xs_grid(min(n or 512, 512), seed=seed)
    return workloads.iq1s_grid(min(n or 2048, 2048), seed=seed)


def unit_codes(fmt, packed):
    """Per choice group, the bytes that encode it: [n, G, k] uint8."""
    p = np.ascontiguousarray(packed).reshape(-1, oracle.BLOCK_BYTES[fmt])
    if fmt == "iq1_m":
        qs = p[:, 0:32].reshape(-1, 16, 2)
        nib = p[:, 32:48].reshape(-1, 16, 1)
        sc = p[:, 48:56:2].astype(np.int64) | (p[:, 49:56:2].astype(np.int64) << 8)
        k = np.stack([(sc >> (3 * t)) & 7 for t in range(4)], axis=2).reshape(-1, 16, 1)
        return np.concatenate([qs, nib, k.astype(np.uint8)], axis=2)
    if fmt == "iq1_s":
        low = p[:, 2:34].reshape(-1, 8, 4)
        qh = p[:, 34:50].reshape(-1, 8, 2)
        return np.concatenate([low, qh], axis=2)
    codes = p[:, 2:66].reshape(-1, 16, 4)
    nib = p[:, 66:74]
    scales = np.stack([nib & 15, nib >> 4], axis=2).reshape(-1, 16, 1)
    return np.concatenate([codes, scales.astype(np.uint8)], axis=2)


def compare_payloads(fmt, got, ref, x, grid, imp=None, max_tie_frac=0.005):
    """got/ref [n, bytes]; x [n, 256]; imp None or [n, 256].  Returns the number
    of tie units; raises AssertionError on a real mismatch."""
    nb = oracle.BLOCK_BYTES[fmt]
    got = np.ascontiguousarray(got).reshape(-1, nb)
    ref = np.ascontiguousarray(ref).reshape(-1, nb)
    assert got.shape == ref.shape
    np.testing.assert_array_equal(scale_bits(fmt, got), scale_bits(fmt, ref),
                                  err_msg="scale bits differ")
    diff = np.any(unit_codes(fmt, got) != unit_codes(fmt, ref), axis=2)     # [n, G]
    nd = int(diff.sum())
    if nd == 0:
        return 0
    rows = np.nonzero(diff.any(axis=1))[0]
    xi = np.asarray(x, dtype=np.float32).reshape(-1, 256)[rows]
    ii = None if imp is None else np.asarray(imp, dtype=np.float32).reshape(-1, 256)[rows]
    eg = oracle.block_errors(fmt, got[rows], xi, grid, ii)
    er = oracle.block_errors(fmt, ref[rows], xi, grid, ii)
    d = diff[rows]
    rel = np.abs(eg - er) / np.maximum(er, 1e-300)
    worst = float(rel[d].max())
    assert worst <= TIE_RTOL, (
        "%d differing units, worst relative error gap %.3g (> %g); first block %d"
        % (nd, worst, TIE_RTOL, int(rows[0])))
    assert nd <= max_tie_frac * diff.size, "%d tie units of %d" % (nd, diff.size)
    return nd


def near_tie_blocks(fmt, nblk=32, seed=0, weighted=True, steps=40):
    """Blocks built so that one choice group's best two choices differ by a
    weighted error just above the tie bar: the values of that group are scaled
    by a factor found by bisection (every block's d pinned) until the oracle's
    runner-up choice costs between 1.1e-6 and 4e-6 relative more than its
    best.  A search whose choice between the two is decided by fp32 rounding
    gets some of these wrong.  Returns (w [1, nblk, 256], grid, imp or None,
    scales [1, nblk] uint16, unit per block, relative gap per block: inf where
    no factor in [0.6, 1.6] reorders the two)."""
    import workloads
    grid = grid_for(fmt, None, seed)
    w0 = workloads.student_t_weight((1, nblk, 256), 100 + seed)
    imp = workloads.lognormal_importance((1, 256), 200 + seed) if weighted else None
    d = oracle.predict_scales(fmt, w0).reshape(1, nblk)
    G = oracle.NUM_CHOICE_GROUPS[fmt]
    L = 256 // G
    nc = oracle.NUM_CHOICES[fmt]
    unit = np.arange(nblk) % G
    target = 1.1e-6 * (4.0 / 1.1) ** ((np.arange(nblk) % 8) / 7.0)
    sel = np.zeros((nblk, 256), bool)
    for b in range(nblk):
        sel[b, L * unit[b]:L * (unit[b] + 1)] = True
    ib = None if imp is None else np.broadcast_to(imp.reshape(1, 256), (nblk, 256))

    def scaled(alpha):
        x = w0.reshape(nblk, 256).astype(np.float64)
        x = np.where(sel, x * alpha[:, None], x).astype(np.float32)
        return x.reshape(1, nblk, 256)

    def unit_errors(w, ch):
        # weighted error of every block's target unit with its choices forced to ch
        c = np.broadcast_to(ch[:, None], (nblk, G)).reshape(1, nblk, 1, G).astype(np.int32)
        p = oracle.encode(fmt, w, grid, imp, scales=d, choices=c).reshape(nblk, -1)
        return oracle.block_errors(fmt, p, w.reshape(nblk, 256), grid, ib)[np.arange(nblk), unit]

    def all_errors(w):
        ev = oracle.encode_every_choice(fmt, w, grid, imp, scales=d).reshape(nc, nblk, -1)
        return np.stack([oracle.block_errors(fmt, ev[c], w.reshape(nblk, 256), grid, ib)
                         [np.arange(nblk), unit] for c in range(nc)], 1)      # [nblk, nc]

    def excess(w, c1, c2):
        e1 = unit_errors(w, c1)
        return (unit_errors(w, c2) - e1) / e1 - target

    e = all_errors(w0)
    order = np.argsort(e, axis=1, kind="stable")
    c1, c2 = order[:, 0], order[:, 1]
    lo = np.ones(nblk)
    hi = np.full(nblk, np.nan)
    for f in (0.98, 1.02, 0.95, 1.05, 0.9, 1.1, 0.8, 1.25, 0.6, 1.6):
        a = np.where(np.isnan(hi), f, hi)
        below = excess(scaled(a), c1, c2) < 0
        hi = np.where(np.isnan(hi) & below, f, hi)
    ok = ~np.isnan(hi) & (excess(scaled(lo), c1, c2) > 0)
    hi = np.where(ok, hi, 1.0)
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        below = excess(scaled(mid), c1, c2) < 0
        hi = np.where(below, mid, hi)
        lo = np.where(below, lo, mid)
    w = scaled(lo)
    e = np.sort(all_errors(w), axis=1)
    gap = (e[:, 1] - e[:, 0]) / e[:, 0]
    return w, grid, imp, d.astype(np.uint16), unit, np.where(ok, gap, np.inf)
