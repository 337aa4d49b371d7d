"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests runs the HIP path.  Each one checks the oracle against
something other than itself: values printed on the pages (golden fixtures),
library routines (numpy's IEEE float16 conversion and float32 arithmetic),
closed forms, joint brute force on tiny grids, and invariants the pages state.
"""

import itertools

import numpy as np
import pytest

import oracle
import workloads
from tests.golden.load import load

# --------------------------------------------------------------------------
# helpers independent of the oracle's C code
# --------------------------------------------------------------------------


def np_predict_scale_bits(amax, divisor):
    """Closed form d = fp16((amax / divisor) * 0.61) in IEEE float32 (numpy)."""
    t = np.float32(amax) / np.float32(divisor)
    t = np.float32(t * np.float32(0.61))
    return int(np.array([t], dtype=np.float32).astype(np.float16).view(np.uint16)[0])


def f16(bits):
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def iq1s_fields(packed):
    """Field extraction as the code review of #2450 prints it:
    qh from bytes 34..49 little-endian, low bytes 2..33 as [8 sub-blocks, 4],
    entry = low | ((qh >> [0,3,6,9]) & 7) << 8, local scale = (qh >> 12) & 7,
    delta sign = qh >> 15."""
    b = packed.reshape(-1, 50).astype(np.int64)
    d = b[:, 0] | (b[:, 1] << 8)
    qh = b[:, 34:50:2] | (b[:, 35:50:2] << 8)
    low = b[:, 2:34].reshape(-1, 8, 4)
    shifts = np.array([0, 3, 6, 9])
    entries = low | (((qh[:, :, None] >> shifts) & 7) << 8)
    return d, entries, (qh >> 12) & 7, qh >> 15


def iq2xs_fields(packed):
    b = packed.reshape(-1, 74).astype(np.int64)
    d = b[:, 0] | (b[:, 1] << 8)
    codes = b[:, 2:66:2] | (b[:, 3:66:2] << 8)
    sc = b[:, 66:74]
    scales = np.stack([sc & 15, sc >> 4], axis=2).reshape(-1, 16)
    return d, codes & 0x1FF, codes >> 9, scales


def iq1m_fields(packed):
    """IQ1_M fields: d's fp16 bits from the top nibbles of the four scale words
    (word w carries bits 4w..4w+3); per group the entry and the shift bit; per
    scale group the 3-bit local scale."""
    b = packed.reshape(-1, 56).astype(np.int64)
    sc = b[:, 48:56:2] | (b[:, 49:56:2] << 8)
    d = sum((sc[:, w] >> 12) << (4 * w) for w in range(4))
    nib = np.stack([b[:, 32:48] & 15, b[:, 32:48] >> 4], axis=2).reshape(-1, 32)
    ent = b[:, 0:32] | ((nib & 7) << 8)
    k = np.stack([(sc >> (3 * t)) & 7 for t in range(4)], axis=2).reshape(-1, 16)
    return d, ent, nib >> 3, k


def payload_d(fmt, p):
    """fp16 bits of every block's d."""
    if fmt == "iq1_m":
        return iq1m_fields(p)[0]
    b = p.reshape(-1, oracle.BLOCK_BYTES[fmt]).astype(np.int64)
    return b[:, 0] | (b[:, 1] << 8)


def payload_choices(fmt, p):
    """Per choice group, the choice the payload carries."""
    if fmt == "iq1_s":
        _, _, k, sgn = iq1s_fields(p)
        return k + 8 * sgn
    if fmt == "iq2_xs":
        return iq2xs_fields(p)[3]
    return iq1m_fields(p)[3]


def fmt_grid(fmt, n=None):
    if fmt == "iq2_xs":
        return workloads.iq2xs_grid(n or 512)
    return workloads.iq1s_grid(n or 2048)


# --------------------------------------------------------------------------
# fp16 conversion and the scale predictor
# --------------------------------------------------------------------------


def test_f32_to_f16_matches_numpy_ieee_conversion():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, 2 ** -24, 2 ** -25,
                  3 * 2 ** -26, 1.5 * 2 ** -24, 2 ** -14, 2 ** -14 - 2 ** -30,
                  1 + 2 ** -11, 1 + 3 * 2 ** -11, 6.1e-5, np.inf, -np.inf]),
    ]).astype(np.float32)
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_bits(v) for v in vals], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)


def test_f16_to_float_is_exact():
    bits = np.arange(0, 0x7C00, 7, dtype=np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_bits_to_float(int(b)) for b in bits])
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("fmt,divisor", [("iq1_s", 16.875), ("iq2_xs", 155.0)])
def test_scale_predictor_closed_form(fmt, divisor):
    # #2450 review: d = (amax / 16.875) * 0.61 with fp16 rounding (IQ1_S);
    # the IQ2_XS divisor 31*5 follows the same pattern (top local multiplier
    # times the largest grid value); #2513 "Testing" names an IQ2_XS clamp
    # without printing its value.
    rng = np.random.default_rng(1)
    amaxes = np.abs(rng.standard_normal(5000) * 10.0 ** rng.integers(-7, 4, 5000)).astype(np.float32)
    for a in amaxes:
        assert oracle.predict_scale_bits(a, fmt) == np_predict_scale_bits(a, divisor)


def test_encoded_scale_bytes_follow_the_closed_form():
    w = workloads.normal_weight((1, 16, 512), 11)
    grid = workloads.iq1s_grid(64)
    p = oracle.encode("iq1_s", w, grid)
    d, _, _, _ = iq1s_fields(p)
    amax = np.abs(w.reshape(-1, 256)).max(axis=1)
    np.testing.assert_array_equal(d, [np_predict_scale_bits(a, 16.875) for a in amax])
    w2 = workloads.student_t_weight((1, 8, 512), 12)
    p2 = oracle.encode("iq2_xs", w2, workloads.iq2xs_grid(32))
    d2, _, _, _ = iq2xs_fields(p2)
    amax2 = np.abs(w2.reshape(-1, 256)).max(axis=1)
    np.testing.assert_array_equal(d2, [np_predict_scale_bits(a, 155.0) for a in amax2])


# --------------------------------------------------------------------------
# layouts: the printed worked example and a hand-built IQ2_XS block
# --------------------------------------------------------------------------


def test_iq1s_worked_example_decodes_as_printed():
    g = load("iq1s_worked_example.txt")
    grid = workloads.iq1s_grid()
    blk = np.zeros(50, dtype=np.uint8)
    blk[0] = int(g["d_fp16_bits"]) & 0xFF
    blk[1] = int(g["d_fp16_bits"]) >> 8
    low = np.array([17, 200, 3, 99], dtype=np.uint8)
    blk[2:6] = low
    qh = int(g["qh"])
    blk[34] = qh & 0xFF
    blk[35] = qh >> 8
    out = oracle.decode("iq1_s", blk.reshape(1, 1, 50), grid).reshape(256)
    assert f16(int(g["d_fp16_bits"])) == g["d"]
    high = [int(h) for h in g["high_bits"]]
    for l in range(4):
        e = int(low[l]) | (high[l] << 8)
        want = g["group_scale"] * (grid[e].astype(np.float64) + g["delta"])
        np.testing.assert_array_equal(out[8 * l: 8 * l + 8], want)
    # sub-blocks 1..7: qh = 0 -> local scale 0 (scale d), delta +1/8, entry 0
    np.testing.assert_array_equal(out[32:40], g["d"] * (grid[0] + 0.125))
    d, ent, k, sgn = iq1s_fields(blk)
    assert k[0, 0] == g["local_scale"] and sgn[0, 0] == 1
    assert list(ent[0, 0] >> 8) == high


def test_iq2xs_hand_block_decodes_as_worked_out():
    g = load("iq2xs_hand_block.txt")
    grid = np.zeros((8, 8), dtype=np.float32)
    grid[0] = g["grid_entry_0"]
    grid[3] = g["grid_entry_3"]
    blk = np.zeros(74, dtype=np.uint8)
    blk[0] = int(g["d_fp16_bits"]) & 0xFF
    blk[1] = int(g["d_fp16_bits"]) >> 8
    for gi, key in ((0, "code_group0"), (1, "code_group1")):
        c = int(g[key])
        blk[2 + 2 * gi] = c & 0xFF
        blk[3 + 2 * gi] = c >> 8
    blk[66] = int(g["byte66"])
    out = oracle.decode("iq2_xs", blk.reshape(1, 1, 74), grid).reshape(256)
    np.testing.assert_array_equal(out[0:8], g["expected_group0"])
    np.testing.assert_array_equal(out[8:16], g["expected_group1"])
    np.testing.assert_array_equal(out[16:24], g["expected_group2"])
    np.testing.assert_array_equal(out[24:32], g["expected_group2"])


def test_block_geometry():
    # #2450 review: 50 / 74 bytes per 256 values, 1.5625 / 2.3125 bits per weight,
    # packed shape (N, cols // 256, bytes).
    w = workloads.normal_weight((1, 3, 768), 2)
    p1 = oracle.encode("iq1_s", w, workloads.iq1s_grid(16))
    p2 = oracle.encode("iq2_xs", w, workloads.iq2xs_grid(16))
    assert p1.shape == (1, 3, 3, 50) and p2.shape == (1, 3, 3, 74)
    assert 50 * 8 / 256 == 1.5625 and 74 * 8 / 256 == 2.3125


# --------------------------------------------------------------------------
# joint brute force on tiny grids: decomposition, objective and tie rule
# --------------------------------------------------------------------------


def _iq1s_brute_force_block(x, w, grid, d):
    """Enumerate every (choice, e0..e3) of each sub-block jointly; return the
    lexicographically first minimiser of the summed weighted error."""
    n = grid.shape[0]
    res = []
    for i in range(8):
        xs = x[32 * i: 32 * i + 32].astype(np.float64).reshape(4, 8)
        ws = w[32 * i: 32 * i + 32].astype(np.float64).reshape(4, 8)
        E = np.empty((16, 4, n))
        for c in range(16):
            s = d * (2 * (c & 7) + 1)
            delta = -0.125 if c >> 3 else 0.125
            xhat = s * (grid.astype(np.float64) + delta)          # [n, 8]
            E[c] = (ws[:, None, :] * (xs[:, None, :] - xhat[None]) ** 2).sum(axis=2)
        tot = (E[:, 0, :, None, None, None] + E[:, 1, None, :, None, None]
               + E[:, 2, None, None, :, None] + E[:, 3, None, None, None, :])
        flat = int(np.argmin(tot.reshape(-1)))        # first minimum in (c, e0..e3) order
        c, e0, e1, e2, e3 = np.unravel_index(flat, tot.shape)
        res.append((int(c), [int(e0), int(e1), int(e2), int(e3)]))
    return res


@pytest.mark.parametrize("n,dup", [(3, False), (5, False), (6, True)])
@pytest.mark.parametrize("weighted", [False, True])
def test_iq1s_matches_joint_brute_force(n, dup, weighted):
    grid = workloads.iq1s_grid(n, seed=n)
    if dup:
        grid[4] = grid[1]          # duplicate entry: the lower index must win
    w = workloads.normal_weight((1, 2, 256), 100 + n)
    imp = workloads.lognormal_importance((1, 256), 200 + n) if weighted else None
    p = oracle.encode("iq1_s", w, grid, imp)
    d, ent, k, sgn = iq1s_fields(p)
    wt = np.ones(256, np.float32) if imp is None else imp[0]
    for b in range(2):
        ref = _iq1s_brute_force_block(w[0, b], wt, grid, f16(int(d[b])))
        for i, (c, es) in enumerate(ref):
            assert int(k[b, i] + 8 * sgn[b, i]) == c
            assert list(ent[b, i]) == es
            if dup:
                assert 4 not in es


def _iq2xs_brute_force_scale_group(x, w, sigma, grid, d):
    n = grid.shape[0]
    x = x.astype(np.float64).reshape(2, 8)
    w = w.astype(np.float64).reshape(2, 8)
    E = np.empty((16, 2, n))
    for k in range(16):
        s = d * (2 * k + 1)
        xhat = s * sigma[:, None, :] * grid.astype(np.float64)[None]   # [2, n, 8]
        E[k] = (w[:, None, :] * (x[:, None, :] - xhat) ** 2).sum(axis=2)
    tot = E[:, 0, :, None] + E[:, 1, None, :]
    k, e0, e1 = np.unravel_index(int(np.argmin(tot.reshape(-1))), tot.shape)
    return int(k), [int(e0), int(e1)]


def _sigma_from_mask(mask7):
    bits = [(mask7 >> j) & 1 for j in range(7)]
    bits.append(sum(bits) & 1)
    return np.array([-1.0 if b else 1.0 for b in bits])


@pytest.mark.parametrize("n,dup", [(4, False), (7, True)])
@pytest.mark.parametrize("weighted", [False, True])
def test_iq2xs_matches_joint_brute_force(n, dup, weighted):
    grid = workloads.iq2xs_grid(n, seed=n)
    if dup:
        grid[5] = grid[2]
    w = workloads.student_t_weight((1, 2, 256), 300 + n)
    imp = workloads.lognormal_importance((1, 256), 400 + n) if weighted else None
    p = oracle.encode("iq2_xs", w, grid, imp)
    d, idx, masks, scales = iq2xs_fields(p)
    wt = np.ones(256, np.float32) if imp is None else imp[0]
    for b in range(2):
        x = w[0, b]
        for m in range(16):
            sig = np.stack([_sigma_from_mask(int(masks[b, 2 * m])),
                            _sigma_from_mask(int(masks[b, 2 * m + 1]))])
            k, es = _iq2xs_brute_force_scale_group(x[16 * m: 16 * m + 16], wt[16 * m: 16 * m + 16],
                                                   sig, grid, f16(int(d[b])))
            assert int(scales[b, m]) == k
            assert [int(idx[b, 2 * m]), int(idx[b, 2 * m + 1])] == es
            if dup:
                assert 5 not in es


def test_iq2xs_signs_follow_input_signs_and_flip_the_weakest():
    # #2525 / #2512 body: IQ2_XS takes the input signs and flips the weakest
    # element when the count of negatives is odd; masks worked out by hand.
    grid = workloads.iq2xs_grid(16)
    base = workloads.normal_weight((1, 1, 256), 5)
    g0 = np.array([0.3, -0.2, 0.5, 0.1, -0.4, 0.6, 0.2, -0.05], dtype=np.float32)
    w = base.copy()
    w[0, 0, :8] = g0
    p = oracle.encode("iq2_xs", w, grid)
    _, _, masks, _ = iq2xs_fields(p)
    assert masks[0, 0] == 0b0010010            # element 7 (|x| smallest) flipped to +
    imp = np.ones((1, 256), np.float32)
    imp[0, 3] = 0.01                            # now element 3 has the smallest w*x*x
    p = oracle.encode("iq2_xs", w, grid, imp)
    _, _, masks, _ = iq2xs_fields(p)
    assert masks[0, 0] == 0b0011010            # element 3 flipped to -, element 7 stays -
    # an even count keeps every input sign
    g1 = np.array([-0.3, -0.2, 0.5, 0.1, 0.4, 0.6, 0.2, 0.05], dtype=np.float32)
    w[0, 0, 8:16] = g1
    p = oracle.encode("iq2_xs", w, grid)
    _, _, masks, _ = iq2xs_fields(p)
    assert masks[0, 1] == 0b0000011


def test_iq2xs_sign_parity_is_even_and_matches_input_signs():
    w = workloads.student_t_weight((1, 32, 256), 21)
    grid = workloads.iq2xs_grid()
    p = oracle.encode("iq2_xs", w, grid)
    _, _, masks, _ = iq2xs_fields(p)
    xs = w.reshape(-1, 32, 8)
    for b in range(xs.shape[0]):
        for gi in range(32):
            sig = _sigma_from_mask(int(masks[b, gi]))
            assert (sig < 0).sum() % 2 == 0
            # at most one sign differs from the input's, and only if the input count is odd
            neg = xs[b, gi] < 0
            diff = (sig < 0) != neg
            assert diff.sum() == (neg.sum() % 2)


# --------------------------------------------------------------------------
# invariants stated on the pages
# --------------------------------------------------------------------------


@pytest.mark.parametrize("fmt", ["iq1_s", "iq2_xs", "iq1_m"])
def test_uniform_importance_reproduces_the_unweighted_payload(fmt):
    # #2723: uniform importance reproduces the unweighted payload exactly.
    grid = fmt_grid(fmt, 128 if fmt == "iq2_xs" else 256)
    w = workloads.normal_weight((1, 8, 512), 31)
    p0 = oracle.encode(fmt, w, grid)
    for c in (1.0, 4.0, 0.25):
        p = oracle.encode(fmt, w, grid, np.full((1, 512), c, np.float32))
        np.testing.assert_array_equal(p, p0)


@pytest.mark.parametrize("fmt", ["iq1_s", "iq2_xs", "iq1_m"])
def test_weighted_encode_lowers_the_weighted_error(fmt):
    grid = fmt_grid(fmt, 256 if fmt == "iq2_xs" else 512)
    w = workloads.normal_weight((1, 16, 512), 41)
    imp = workloads.lognormal_importance((1, 512), 42) ** 4
    pw = oracle.encode(fmt, w, grid, imp)
    pu = oracle.encode(fmt, w, grid)
    # same d on both (the predictor is unweighted)
    np.testing.assert_array_equal(payload_d(fmt, pw), payload_d(fmt, pu))
    ew = oracle.unit_errors(fmt, pw, w, grid, imp)
    eu = oracle.unit_errors(fmt, pu, w, grid, imp)
    if fmt == "iq2_xs":
        # the weakest-element flip depends on the importance, so the search is
        # only comparable where both encodes chose the same signs
        _, _, mw, _ = iq2xs_fields(pw)
        _, _, mu, _ = iq2xs_fields(pu)
        same = (mw == mu).reshape(-1, 16, 2).all(axis=2)
        assert same.mean() > 0.5
        ew, eu = ew[same], eu[same]
    assert np.all(ew <= eu * (1 + 1e-12))
    assert np.mean(ew < eu) > 0.5


def test_iq1s_payload_beats_random_single_code_perturbations():
    grid = workloads.iq1s_grid()
    w = workloads.normal_weight((1, 4, 256), 51)
    imp = workloads.lognormal_importance((1, 256), 52)
    p = oracle.encode("iq1_s", w, grid, imp)
    base = oracle.unit_errors("iq1_s", p, w, grid, imp)
    rng = np.random.default_rng(53)
    for _ in range(300):
        q = p.copy().reshape(-1, 50)
        b = rng.integers(0, q.shape[0])
        i = rng.integers(0, 8)
        if rng.random() < 0.5:
            q[b, 2 + 4 * i + rng.integers(0, 4)] = rng.integers(0, 256)   # low bits of an entry
        else:
            qh = int(q[b, 34 + 2 * i]) | (int(q[b, 35 + 2 * i]) << 8)
            qh ^= 1 << int(rng.integers(0, 16))                           # any qh bit
            q[b, 34 + 2 * i] = qh & 0xFF
            q[b, 35 + 2 * i] = qh >> 8
        e = oracle.unit_errors("iq1_s", q.reshape(p.shape), w, grid, imp)
        assert e[b, i] >= base[b, i] * (1 - 1e-12)


@pytest.mark.parametrize("fmt", ["iq1_s", "iq2_xs", "iq1_m"])
def test_decode_then_reencode_under_its_own_scales(fmt):
    # #3197: a decoding re-encodes exactly under its own pinned scales.
    grid = fmt_grid(fmt)
    w = workloads.normal_weight((1, 8, 512), 61)
    imp = workloads.lognormal_importance((1, 512), 62)
    p = oracle.encode(fmt, w, grid, imp)
    xhat = oracle.decode(fmt, p, grid).astype(np.float32)
    assert np.array_equal(xhat.astype(np.float64), oracle.decode(fmt, p, grid))  # exact in fp32
    d = payload_d(fmt, p).astype(np.uint16).reshape(1, 8, 2)
    p2 = oracle.encode(fmt, xhat, grid, imp, scales=d)
    # the re-encode reproduces the values exactly; bytes match unless another
    # code decodes to the very same values (then the lower choice index wins)
    np.testing.assert_array_equal(oracle.decode(fmt, p2, grid), oracle.decode(fmt, p, grid))
    same = np.all(p2.reshape(-1, p.shape[-1]) == p.reshape(-1, p.shape[-1]), axis=1)
    assert same.mean() >= 0.9
    # without pinning, d is re-predicted from the decoded amax and may move
    p3 = oracle.encode(fmt, xhat, grid, imp)
    assert p3.shape == p.shape


def test_decode_rejects_indices_beyond_the_grid():
    grid = workloads.iq1s_grid(1500)
    p = oracle.encode("iq1_s", workloads.normal_weight((1, 1, 256), 72), grid)
    p[0, 0, 0, 34 + 2 * 3 + 1] |= 0x0E           # qh bits 9-11 of sub-block 3 -> 7: index >= 1792
    with pytest.raises(oracle.OracleError):
        oracle.decode("iq1_s", p, grid)
    out = oracle.decode("iq1_s", p, grid, strict=False).reshape(256)
    assert not out[3 * 32 + 24: 3 * 32 + 32].any()


def test_range_checks_bite_with_truncated_grids():
    # #2450 review: index range checks only bite with a grid smaller than 2^bits.
    w = workloads.normal_weight((1, 16, 256), 71)
    g1 = workloads.iq1s_grid(1500)
    _, ent, k, sgn = iq1s_fields(oracle.encode("iq1_s", w, g1))
    assert ent.max() < 1500 and ent.max() > 1024
    assert len(np.unique(k)) > 1 and len(np.unique(sgn)) > 1
    g2 = workloads.iq2xs_grid(300)
    d, idx, _, sc = iq2xs_fields(oracle.encode("iq2_xs", w, g2))
    assert idx.max() < 300 and idx.max() > 256
    assert len(np.unique(sc)) > 1 and np.all(d > 0)


@pytest.mark.parametrize("fmt", ["iq1_s", "iq2_xs", "iq1_m"])
def test_zero_and_underflow_blocks_are_all_zero_bytes(fmt):
    grid = fmt_grid(fmt, 64)
    w = workloads.normal_weight((1, 3, 256), 81)
    w[0, 0] = 0.0
    w[0, 1] *= 1e-7                              # amax ~ 1e-8: d underflows to fp16 zero
    p = oracle.encode(fmt, w, grid)
    assert not p[0, 0].any() and not p[0, 1].any() and p[0, 2].any()


@pytest.mark.parametrize("fmt", ["iq1_s", "iq1_m"])
def test_zero_choice_group_in_a_live_block_takes_the_lowest_choice(fmt):
    # An all-zero choice group inside a block with a nonzero d: with the
    # all-zero grid entry, delta = +1/8 and -1/8 give exactly the same error
    # (s/8 per value either way), so the tie rule decides: the lowest choice
    # (IQ1_S c = 0: k = 0, delta bit 0; IQ1_M k = 0 and shift 0) and the
    # zero entry.
    grid = fmt_grid(fmt, 300)
    grid[7] = 0.0
    zero = int(np.nonzero(~grid.any(axis=1))[0][0])      # the first all-zero entry
    w = workloads.normal_weight((1, 2, 256), 83)
    L = 32 if fmt == "iq1_s" else 16
    w[0, 0, :L] = 0.0
    w[0, 1, 256 - L:] = 0.0
    imp = workloads.lognormal_importance((1, 256), 84)
    for im in (None, imp):
        p = oracle.encode(fmt, w, grid, im)
        ch = payload_choices(fmt, p).reshape(2, -1)
        assert ch[0, 0] == 0 and ch[1, -1] == 0
        if fmt == "iq1_s":
            ent = iq1s_fields(p)[1].reshape(2, 8, 4)
            assert np.all(ent[0, 0] == zero) and np.all(ent[1, -1] == zero)
        else:
            _, ent, shift, _ = iq1m_fields(p)
            ent, shift = ent.reshape(2, 32), shift.reshape(2, 32)
            assert np.all(ent[0, :2] == zero) and np.all(ent[1, -2:] == zero)
            assert not shift[0, :2].any() and not shift[1, -2:].any()


@pytest.mark.parametrize("fmt", ["iq1_s", "iq2_xs", "iq1_m"])
def test_rejects_bad_inputs(fmt):
    grid = fmt_grid(fmt, 64)
    w = workloads.normal_weight((1, 2, 256), 91)
    bad = w.copy()
    bad[0, 1, 7] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.encode(fmt, bad, grid)
    bad[0, 1, 7] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.encode(fmt, bad, grid)
    imp = np.ones((1, 256), np.float32)
    imp[0, 3] = -1.0
    with pytest.raises(oracle.OracleError):
        oracle.encode(fmt, w, grid, imp)
    imp[0, 3] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.encode(fmt, w, grid, imp)
    huge = w * 1e9                                # d beyond fp16 range
    with pytest.raises(oracle.OracleError):
        oracle.encode(fmt, huge, grid)
    with pytest.raises(oracle.OracleError):
        oracle.encode(fmt, w[:, :, :200], grid)


def test_sanity_bounds():
    # #2450 review: normalized MSE < 0.25 for IQ1_S; #2595: error falls with bit width.
    c = workloads.c1_iq1s_small()
    p = oracle.encode("iq1_s", c["w"], c["grid"])
    x = c["w"].reshape(-1).astype(np.float64)
    xh = oracle.decode("iq1_s", p, c["grid"]).reshape(-1)
    assert ((x - xh) ** 2).sum() / (x ** 2).sum() < 0.25
    p2 = oracle.encode("iq2_xs", c["w"], workloads.iq2xs_grid())
    xh2 = oracle.decode("iq2_xs", p2, workloads.iq2xs_grid()).reshape(-1)
    assert ((x - xh2) ** 2).sum() < ((x - xh) ** 2).sum()


@pytest.mark.parametrize("fmt", ["iq1_s", "iq2_xs", "iq1_m"])
def test_forced_choices_reproduce_the_free_encode(fmt):
    # #3157: a fixed choice reproduces, group by group, the payload encoded with
    # that choice; forcing the free encode's own picks reproduces it.
    grid = fmt_grid(fmt, 128 if fmt == "iq2_xs" else 256)
    w = workloads.normal_weight((1, 4, 512), 101)
    imp = workloads.lognormal_importance((1, 512), 102)
    p = oracle.encode(fmt, w, grid, imp)
    G = oracle.NUM_CHOICE_GROUPS[fmt]
    ch = payload_choices(fmt, p).reshape(1, 4, 2, G)
    np.testing.assert_array_equal(oracle.encode(fmt, w, grid, imp, choices=ch), p)
    # every group forced to one choice: each unit's error >= the free optimum
    for c in (0, 5, 7 if fmt == "iq1_m" else 11):
        pc = oracle.encode(fmt, w, grid, imp, choices=np.full_like(ch, c))
        assert np.all(payload_choices(fmt, pc) == c)
        assert np.all(oracle.unit_errors(fmt, pc, w, grid, imp)
                      >= oracle.unit_errors(fmt, p, w, grid, imp) * (1 - 1e-12))
    with pytest.raises(oracle.OracleError):
        oracle.encode(fmt, w, grid, imp, choices=np.full_like(ch, oracle.NUM_CHOICES[fmt]))


# --------------------------------------------------------------------------
# every-choice payloads and the decoded encode (fake quant)
# --------------------------------------------------------------------------


@pytest.mark.parametrize("fmt", ["iq1_s", "iq2_xs", "iq1_m"])
def test_every_choice_payloads_carry_their_choice_and_contain_the_free_encode(fmt):
    # #3159: packed[c] is the encode with every choice group forced to c.  So
    # every unit of packed[c] carries choice c, and per unit the least weighted
    # error over c is the free encode's, reached first at the free encode's
    # own choice (the free encode is pinned by brute force above).
    grid = fmt_grid(fmt, 96 if fmt == "iq2_xs" else 192)
    nc = oracle.NUM_CHOICES[fmt]
    w = workloads.normal_weight((2, 3, 256), 131)
    w[1, 2] = 0.0                                    # a zero block: all-zero in every payload
    imp = workloads.lognormal_importance((2, 256), 132)
    every = oracle.encode_every_choice(fmt, w, grid, imp)
    assert every.shape == (nc, 2, 3, 1, oracle.BLOCK_BYTES[fmt])
    free = oracle.encode(fmt, w, grid, imp)
    assert not every[:, 1, 2].any()
    live = np.ones((6,), bool)
    live[5] = False
    for c in range(nc):
        assert np.all(payload_choices(fmt, every[c])[live] == c)
        np.testing.assert_array_equal(payload_d(fmt, every[c]), payload_d(fmt, free))
    errs = np.stack([oracle.unit_errors(fmt, every[c], w, grid, imp) for c in range(nc)])
    e_free = oracle.unit_errors(fmt, free, w, grid, imp)
    np.testing.assert_allclose(errs.min(axis=0), e_free, rtol=1e-12, atol=0)
    c_free = payload_choices(fmt, free).reshape(e_free.shape)
    first = np.argmax(errs <= e_free[None] * (1 + 1e-12), axis=0)
    live_units = np.repeat(live, e_free.shape[-1]).reshape(c_free.shape)
    np.testing.assert_array_equal(first[live_units], c_free[live_units])


@pytest.mark.parametrize("fmt", ["iq1_s", "iq2_xs", "iq1_m"])
def test_fake_quant_is_the_decoded_encode(fmt):
    # The fake-quant weight is decode(encode(w)); decoding the printed worked
    # example is pinned above, so here its error must be the unit errors the
    # encode reports, and re-encoding it under its own scales is a fixed point.
    grid = fmt_grid(fmt, 128 if fmt == "iq2_xs" else 256)
    w = workloads.normal_weight((1, 4, 512), 141)
    imp = workloads.lognormal_importance((1, 512), 142)
    xh = oracle.fake_quant(fmt, w, grid, imp)
    p = oracle.encode(fmt, w, grid, imp)
    wt = np.broadcast_to(imp.astype(np.float64)[:, None, :], w.shape)
    e = (wt * (w.astype(np.float64) - xh) ** 2).reshape(-1, 256 // oracle.NUM_CHOICE_GROUPS[fmt]).sum(1)
    np.testing.assert_allclose(e, oracle.unit_errors(fmt, p, w, grid, imp).reshape(-1), rtol=1e-12)
    d = oracle.predict_scales(fmt, w).reshape(1, 4, 2)
    again = oracle.fake_quant(fmt, xh.astype(np.float32), grid, imp, scales=d)
    np.testing.assert_array_equal(again, xh)


# --------------------------------------------------------------------------
# candidates (top-C choices per IQ2_XS scale group)
# --------------------------------------------------------------------------


def test_candidates_are_the_sorted_choices_of_the_encode():
    grid = workloads.iq2xs_grid()
    w = workloads.student_t_weight((1, 6, 256), 111)
    imp = workloads.lognormal_importance((1, 256), 112)
    err, ch, codes = oracle.iq2xs_candidates(w, grid, imp, top_c=8)
    p = oracle.encode("iq2_xs", w, grid, imp)
    d, idx, masks, sc = iq2xs_fields(p)
    np.testing.assert_array_equal(ch[:, :, 0], sc)                 # top-1 = the encoder's pick
    np.testing.assert_array_equal(codes[:, :, 0, 0], idx[:, 0::2] | (masks[:, 0::2] << 9))
    np.testing.assert_array_equal(codes[:, :, 0, 1], idx[:, 1::2] | (masks[:, 1::2] << 9))
    xh = oracle.decode("iq2_xs", p, grid).reshape(-1, 16, 16)
    np.testing.assert_array_equal(err[:, :, 0, :], (xh - w.reshape(-1, 16, 16)).astype(np.float32))
    # weighted error of each candidate is non-decreasing with rank; choices distinct
    wt = imp.reshape(16, 16).astype(np.float64)
    e = (wt[None, :, None, :] * err.astype(np.float64) ** 2).sum(axis=3)
    assert np.all(np.diff(e, axis=2) >= -1e-9 * e[:, :, 1:])
    assert all(len(set(r)) == 8 for r in ch.reshape(-1, 8))
    # each candidate equals the forced encode with that local scale
    for r in (1, 5):
        pf = oracle.encode("iq2_xs", w, grid, imp, choices=ch[:, :, r].reshape(1, 6, 1, 16))
        xf = oracle.decode("iq2_xs", pf, grid).reshape(-1, 16, 16)
        np.testing.assert_array_equal(err[:, :, r, :], (xf - w.reshape(-1, 16, 16)).astype(np.float32))


def test_iq1s_candidates_are_the_sorted_choices_of_the_encode():
    grid = workloads.iq1s_grid(512)
    w = workloads.normal_weight((1, 5, 256), 113)
    w[0, 4] = 0.0                                       # zero block: c = 0, 1, ..., error -x
    imp = workloads.lognormal_importance((1, 256), 114)
    err, ch, codes = oracle.iq1s_candidates(w, grid, imp, top_c=6)
    assert err.shape == (5, 8, 6, 32) and codes.shape == (5, 8, 6, 4)
    p = oracle.encode("iq1_s", w, grid, imp)
    d, entries, k, sgn = iq1s_fields(p)
    np.testing.assert_array_equal(ch[:4, :, 0], (k + 8 * sgn)[:4])   # top-1 = the encoder's pick
    np.testing.assert_array_equal(codes[:4, :, 0, :], entries[:4])
    xh = oracle.decode("iq1_s", p, grid).reshape(-1, 8, 32)
    np.testing.assert_array_equal(err[:, :, 0, :], (xh - w.reshape(-1, 8, 32)).astype(np.float32))
    np.testing.assert_array_equal(ch[4], np.tile(np.arange(6), (8, 1)))
    np.testing.assert_array_equal(err[4], np.broadcast_to(-w.reshape(-1, 8, 1, 32)[4], (8, 6, 32)))
    wt = imp.reshape(8, 32).astype(np.float64)
    e = (wt[None, :, None, :] * err.astype(np.float64) ** 2).sum(axis=3)
    assert np.all(np.diff(e[:4], axis=2) >= -1e-9 * e[:4, :, 1:])
    assert all(len(set(r)) == 6 for r in ch.reshape(-1, 6))
    for r in (1, 5):                                    # = the forced encode with that choice
        pf = oracle.encode("iq1_s", w, grid, imp, choices=ch[:, :, r].reshape(1, 5, 1, 8))
        xf = oracle.decode("iq1_s", pf, grid).reshape(-1, 8, 32)
        np.testing.assert_array_equal(err[:, :, r, :], (xf - w.reshape(-1, 8, 32)).astype(np.float32))


# --------------------------------------------------------------------------
# choice search
# --------------------------------------------------------------------------


def _direct_search(H, cand, sweeps):
    """Each decision taken by evaluating the full e^T H e for every candidate."""
    H = H.astype(np.float64)
    G, C, L = cand.shape
    cand = cand.astype(np.float64)
    picks = []
    for g in range(G):
        Hg = H[g * L:(g + 1) * L, g * L:(g + 1) * L]
        q = np.einsum("ci,ij,cj->c", cand[g], Hg, cand[g])
        picks.append(int(np.argmin(q)))
    trace = [list(picks)]

    def J(p):
        e = np.concatenate([cand[g, p[g]] for g in range(G)])
        return e @ H @ e

    for _ in range(sweeps):
        for g in range(G):
            vals = []
            for c in range(C):
                p2 = list(picks)
                p2[g] = c
                vals.append(J(p2))
            best = int(np.argmin(vals))
            if vals[best] < vals[picks[g]]:
                picks[g] = best
        trace.append(list(picks))
    return picks, trace


def _random_cand(rows, G, C, seed, scale=0.01):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((rows, G, C, 256 // G))).astype(np.float32)


@pytest.mark.parametrize("G,C", [(16, 8), (8, 4)])
def test_choice_search_matches_direct_objective_decisions(G, C):
    H = workloads.block_hessian(256, 7)
    cand = _random_cand(6, G, C, 121)
    picks, trace = oracle.choice_search(H, cand, sweeps=2)
    for r in range(cand.shape[0]):
        p, t = _direct_search(H, cand[r], 2)
        assert list(picks[r]) == p
        assert [list(trace[s, r]) for s in range(3)] == t


def test_choice_search_sweeps_change_picks_and_lower_J():
    # #3218: the fused search's test fails if the refinement sweeps are skipped.
    H = workloads.block_hessian(256, 7)
    cand = _random_cand(64, 16, 8, 131)
    picks, trace = oracle.choice_search(H, cand, sweeps=2)
    J = [oracle.choice_objective(H, cand, trace[s]) for s in range(3)]
    assert np.all(J[1] <= J[0] * (1 + 1e-12)) and np.all(J[2] <= J[1] * (1 + 1e-12))
    assert np.any(trace[0] != trace[2])
    assert np.mean(J[2] < J[0]) > 0.5


def test_choice_search_keeps_the_pick_on_an_exact_tie():
    # #3158 step 3 moves a group only on a strict improvement.  Exact
    # arithmetic: H = I plus a coupling of 1/2 between element 0 of groups 0
    # and 1.  Step 2 gives group 0 candidate 1 (e^T e = 4 against 8) and
    # group 1 candidate 0 (4 against 9).  In the first sweep group 0 sees
    # rest = (1, 0, ...), so both its candidates score exactly 4: it keeps
    # candidate 1, though candidate 0 is the lower index of the least score.
    G, C, L = 16, 2, 16
    H = np.eye(256, dtype=np.float32)
    H[0, 16] = H[16, 0] = 0.5
    cand = np.zeros((1, G, C, L), np.float32)
    cand[0, 0, 0, :2] = (-2.0, 2.0)
    cand[0, 0, 1, :2] = (0.0, 2.0)
    cand[0, 1, 0, 0] = 2.0
    cand[0, 1, 1, 0] = 3.0
    picks, trace = oracle.choice_search(H, cand, sweeps=2)
    assert list(trace[0, 0, :2]) == [1, 0]
    assert list(picks[0, :2]) == [1, 0] and not picks[0, 2:].any()
    J = [oracle.choice_objective(H, cand, trace[s]) for s in range(3)]
    assert J[0][0] == J[2][0]


def test_identity_hessian_keeps_the_encoders_own_choices():
    # #3158: under H = I the search reproduces the encoder's own picks.
    grid = workloads.iq2xs_grid()
    w = workloads.student_t_weight((1, 16, 256), 141)
    err, ch, _ = oracle.iq2xs_candidates(w, grid, None, top_c=8)
    picks, trace = oracle.choice_search(np.eye(256, dtype=np.float32), err, sweeps=2)
    assert np.all(picks == 0)
    assert np.all(trace == 0)


def test_block_diagonal_hessian_reaches_the_brute_force_optimum():
    rng = np.random.default_rng(151)
    H = np.zeros((256, 256))
    for g in range(8):
        a = rng.standard_normal((32, 32))
        H[32 * g:32 * g + 32, 32 * g:32 * g + 32] = a @ a.T / 32 + np.eye(32)
    H = H.astype(np.float32)
    cand = _random_cand(3, 8, 3, 152)
    picks, trace = oracle.choice_search(H, cand, sweeps=2)
    assert np.array_equal(trace[0], trace[2])     # no cross terms: sweeps change nothing
    for r in range(3):
        best = min(itertools.product(range(3), repeat=8),
                   key=lambda p: oracle.choice_objective(H, cand[r:r + 1], np.array([p]))[0])
        Jb = oracle.choice_objective(H, cand[r:r + 1], np.array([best]))[0]
        Jp = oracle.choice_objective(H, cand[r:r + 1], picks[r:r + 1])[0]
        assert abs(Jp - Jb) <= 1e-12 * abs(Jb)


def test_choice_search_never_beats_the_global_optimum():
    H = workloads.block_hessian(256, 9)
    cand = _random_cand(2, 8, 3, 161)
    picks, _ = oracle.choice_search(H, cand, sweeps=2)
    for r in range(2):
        Jall = [oracle.choice_objective(H, cand[r:r + 1], np.array([p]))[0]
                for p in itertools.product(range(3), repeat=8)]
        Jp = oracle.choice_objective(H, cand[r:r + 1], picks[r:r + 1])[0]
        assert Jp >= min(Jall) * (1 - 1e-12)


def test_replay_accepts_the_oracles_trace_and_rejects_a_bad_one():
    H = workloads.block_hessian(256, 7)
    cand = _random_cand(8, 16, 8, 171)
    picks, trace = oracle.choice_search(H, cand, sweeps=2)
    for r in range(8):
        fail, worst = oracle.choice_replay(H, cand[r], trace[:, r, :], 1e-9)
        assert fail == 0 and worst <= 1e-12
    # move one step-2 pick to the worst choice of its group
    bad = trace[:, 0, :].copy()
    Hd = H.astype(np.float64)[0:16, 0:16]
    q = np.einsum("ci,ij,cj->c", cand[0, 0].astype(np.float64), Hd, cand[0, 0].astype(np.float64))
    bad[0, 0] = int(np.argmax(q))
    fail, _ = oracle.choice_replay(H, cand[0], bad, 1e-6)
    assert fail == 1


def test_replay_handles_32_column_groups():
    # G = 8 (IQ1_S sub-blocks): the replay's per-group vectors hold 32 values.
    H = workloads.block_hessian(256, 7)
    grid = workloads.iq1s_grid(512)
    w = workloads.normal_weight((1, 48, 256), 181)
    imp = np.sqrt(np.diag(H).astype(np.float64)).astype(np.float32)[None]
    err, _, _ = oracle.iq1s_candidates(w, grid, imp, top_c=8)
    for cand in (err, _random_cand(48, 8, 16, 182)):
        picks, trace = oracle.choice_search(H, cand, sweeps=2)
        for r in range(cand.shape[0]):
            fail, worst = oracle.choice_replay(H, cand[r], trace[:, r, :], 1e-9)
            assert fail == 0 and worst <= 1e-12, (r, fail, worst)


# --------------------------------------------------------------------------
# IQ1_M (#2525 IQ1_M commit bodies #2513, #2595)
# --------------------------------------------------------------------------


def test_iq1m_hand_block_decodes_as_worked_out():
    g = load("iq1m_hand_block.txt")
    grid = np.zeros((300, 8), np.float32)
    grid[1] = g["grid_row_1"]
    grid[257] = g["grid_row_257"]
    blk = np.zeros(56, np.uint8)
    blk[0] = blk[1] = blk[8] = blk[31] = 1
    blk[32] = 0x90
    blk[36] = 0x08
    blk[47] = 0x10
    for w_, v in enumerate(g["scale_words"]):
        blk[48 + 2 * w_] = int(v) & 0xFF
        blk[49 + 2 * w_] = int(v) >> 8
    d, ent, shift, k = iq1m_fields(blk)
    assert int(d[0]) == int(g["d_fp16_bits"]) and f16(int(d[0])) == 0.5
    out = oracle.decode("iq1_m", blk.reshape(1, 1, 1, 56), grid).reshape(32, 8)
    for grp in (0, 1, 2, 8, 31):
        np.testing.assert_array_equal(out[grp], g["expected_group%d" % grp])
    assert oracle.BLOCK_BYTES["iq1_m"] * 8 / 256 == 1.75


def test_iq1m_scale_anchor_follows_peak_to_rms():
    # #2513 "A scale-anchor correction": clamp(0.58 + 0.035 * peak_to_rms, 0.65,
    # 0.95).  Blocks of n equal spikes have peak-to-RMS sqrt(256/n) exactly:
    # 1, 4, 8, 16 reach both clamps and two points of the slope.
    for n_spk, ratio in ((256, 1.0), (16, 4.0), (4, 8.0), (1, 16.0)):
        x = np.zeros(256, np.float32)
        x[::256 // n_spk] = 0.5
        want = np.float32(0.58) + np.float32(np.float32(0.035) * np.float32(ratio))
        want = min(max(want, np.float32(0.65)), np.float32(0.95))
        assert oracle.iq1m_anchor(x) == want
        t = np.float32(np.float32(0.5) / np.float32(16.875)) * want
        bits = int(np.array([np.float32(t)]).astype(np.float16).view(np.uint16)[0])
        assert int(oracle.predict_scales("iq1_m", x)[0]) == bits
    assert oracle.iq1m_anchor(np.full(256, 0.25, np.float32)) == np.float32(0.65)
    # a Gaussian block sits on the slope, above IQ1_S's flat 0.61
    a = oracle.iq1m_anchor(workloads.normal_weight((256,), 151))
    assert 0.65 < a < 0.8


def _iq1m_brute_force_scale_group(x, w, grid, d):
    """Every (k, shift0, e0, shift1, e1) of a scale group jointly; the
    lexicographically first minimiser of the summed weighted error."""
    n = grid.shape[0]
    x = x.astype(np.float64).reshape(2, 8)
    w = w.astype(np.float64).reshape(2, 8)
    E = np.empty((8, 2, 2, n))                                   # [k, group, shift, entry]
    for k in range(8):
        s = d * (2 * k + 1)
        for sh in range(2):
            xhat = s * (grid.astype(np.float64) + (-0.125 if sh else 0.125))
            E[k, :, sh] = (w[:, None, :] * (x[:, None, :] - xhat[None]) ** 2).sum(axis=2)
    tot = E[:, 0, :, :, None, None] + E[:, 1, None, None, :, :]
    k, s0, e0, s1, e1 = np.unravel_index(int(np.argmin(tot.reshape(-1))), tot.shape)
    return int(k), [int(s0), int(s1)], [int(e0), int(e1)]


@pytest.mark.parametrize("n,dup", [(3, False), (6, True)])
@pytest.mark.parametrize("weighted", [False, True])
def test_iq1m_matches_joint_brute_force(n, dup, weighted):
    grid = workloads.iq1s_grid(n, seed=n + 20)
    if dup:
        grid[4] = grid[1]
    w = workloads.normal_weight((1, 2, 256), 500 + n)
    imp = workloads.lognormal_importance((1, 256), 600 + n) if weighted else None
    p = oracle.encode("iq1_m", w, grid, imp)
    d, ent, shift, k = iq1m_fields(p)
    wt = np.ones(256, np.float32) if imp is None else imp[0]
    for b in range(2):
        for m in range(16):
            kk, sh, es = _iq1m_brute_force_scale_group(w[0, b, 16 * m:16 * m + 16],
                                                       wt[16 * m:16 * m + 16], grid, f16(int(d[b])))
            assert int(k[b, m]) == kk
            assert [int(shift[b, 2 * m]), int(shift[b, 2 * m + 1])] == sh
            assert [int(ent[b, 2 * m]), int(ent[b, 2 * m + 1])] == es
            if dup:
                assert 4 not in es


def test_iq1m_candidates_are_the_sorted_choices_of_the_encode():
    grid = workloads.iq1s_grid(384)
    w = workloads.normal_weight((1, 5, 256), 161)
    w[0, 4] = 0.0
    imp = workloads.lognormal_importance((1, 256), 162)
    err, ch, codes = oracle.iq1m_candidates(w, grid, imp, top_c=5)
    assert err.shape == (5, 16, 5, 16) and codes.shape == (5, 16, 5, 2)
    p = oracle.encode("iq1_m", w, grid, imp)
    d, ent, shift, k = iq1m_fields(p)
    np.testing.assert_array_equal(ch[:4, :, 0], k[:4])
    np.testing.assert_array_equal(codes[:4, :, 0, 0], (ent | (shift << 11))[:4, 0::2])
    np.testing.assert_array_equal(codes[:4, :, 0, 1], (ent | (shift << 11))[:4, 1::2])
    xh = oracle.decode("iq1_m", p, grid).reshape(-1, 16, 16)
    np.testing.assert_array_equal(err[:, :, 0, :], (xh - w.reshape(-1, 16, 16)).astype(np.float32))
    np.testing.assert_array_equal(ch[4], np.tile(np.arange(5), (16, 1)))
    assert all(len(set(r)) == 5 for r in ch.reshape(-1, 5))
    for r in (1, 4):
        pf = oracle.encode("iq1_m", w, grid, imp, choices=ch[:, :, r].reshape(1, 5, 1, 16))
        xf = oracle.decode("iq1_m", pf, grid).reshape(-1, 16, 16)
        np.testing.assert_array_equal(err[:, :, r, :], (xf - w.reshape(-1, 16, 16)).astype(np.float32))


def test_iq1m_is_finer_than_iq1s_and_keeps_ranges():
    # 1.75 bits against 1.5625: a lower error on the same weight; the range
    # checks bite with a truncated grid; the shifts and scales vary.
    w = workloads.normal_weight((1, 16, 256), 171)
    x = w.reshape(-1).astype(np.float64)
    g = workloads.iq1s_grid()
    e_s = ((oracle.decode("iq1_s", oracle.encode("iq1_s", w, g), g).reshape(-1) - x) ** 2).sum()
    p = oracle.encode("iq1_m", w, g)
    e_m = ((oracle.decode("iq1_m", p, g).reshape(-1) - x) ** 2).sum()
    assert e_m < e_s and e_m / (x ** 2).sum() < 0.25
    _, ent, shift, k = iq1m_fields(oracle.encode("iq1_m", w, workloads.iq1s_grid(1500)))
    assert 1024 < ent.max() < 1500
    assert len(np.unique(k)) > 1 and 0 < shift.mean() < 1
