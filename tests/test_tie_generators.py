"""CPU checks of the near-tie input generators in tests/parity.py.

The GPU tests feed these blocks to the kernels to show that decisions whose
fp64 errors differ by just more than the 1e-6 tie bar are taken as the oracle
takes them.  That is only a test if the blocks really hold such near ties, so
here the oracle alone confirms it: the gaps it measures on its own encode of
the generated blocks lie in the band the generator aims at.
"""

import numpy as np
import pytest

import oracle
from tests.parity import entry_tie_blocks, set_entry, unit_choices, _pick


@pytest.mark.parametrize("fmt", ["iq1_s", "iq2_xs", "iq1_m"])
def test_entry_tie_blocks_hold_entry_level_near_ties(fmt):
    w, grid, imp, d, ch, groups, kinds, gap = entry_tie_blocks(fmt, 48, 1, True)
    band = (gap > 1e-6) & (gap < 1e-5)
    assert band.sum() >= 40, gap
    # the forced encode carries the forced choices, and the scaled group's
    # choice group is the only one whose free choice may have moved
    free = oracle.encode(fmt, w, grid, imp, scales=d)
    forced = oracle.encode(fmt, w, grid, imp, scales=d, choices=ch)
    np.testing.assert_array_equal(unit_choices(fmt, forced), ch.reshape(48, -1))
    moved = unit_choices(fmt, free) != ch.reshape(48, -1)
    unit = groups // (32 // oracle.NUM_CHOICE_GROUPS[fmt])
    moved[np.arange(48), unit] = False
    assert not moved.any()
    if fmt == "iq1_m":
        # both kinds: the runner-up with the same shift, and with the other one
        assert (kinds[band] == 1).sum() >= 10 and (kinds[band] == 0).sum() >= 5


def test_set_entry_and_pick_round_trip():
    # the layout helpers invert each other on every group of a real payload
    import workloads
    for fmt in ("iq1_s", "iq2_xs", "iq1_m"):
        grid = workloads.iq2xs_grid() if fmt == "iq2_xs" else workloads.iq1s_grid()
        p = oracle.encode(fmt, workloads.normal_weight((1, 1, 256), 3), grid).reshape(-1)
        for g in range(32):
            s, e = _pick(fmt, p, g)
            np.testing.assert_array_equal(set_entry(fmt, p, g, e, s), p)
            e2 = (e + 37) % grid.shape[0]
            q = set_entry(fmt, p, g, e2, None if s is None else 1 - s)
            assert _pick(fmt, q, g) == (None if s is None else 1 - s, e2)
            # only that group's fields moved
            x = oracle.decode(fmt, p.reshape(1, 1, -1), grid).reshape(256)
            y = oracle.decode(fmt, q.reshape(1, 1, -1), grid).reshape(256)
            moved = np.nonzero(x != y)[0]
            assert moved.size == 0 or (moved.min() >= 8 * g and moved.max() < 8 * g + 8)
