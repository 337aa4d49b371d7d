"""HIP candidate emission and local-Hessian choice search against the oracle.

Candidates: per IQ2_XS scale group, the top-C local scales in (cost, k) order
with their error vectors; the HIP and oracle lists must agree exactly except
where near-tied costs swap (then the float64 weighted errors agree within
1e-6 relative).  Choice search: the HIP and oracle searches consume the same
candidate array; rows whose decision traces differ must pass the oracle's
replay check (every HIP decision optimal within 1e-6 of the row's objective).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import ggml_iq_codebook_amd as iq  # noqa: E402

DEV = "cuda:0"
REPLAY_TOL = 1e-6


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write("\n[gpu] %s\n" % request.node.nodeid)
    sys.__stderr__.flush()
    yield


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _check_candidates(w, grid, imp, top_c, fmt="iq2_xs"):
    """w [rows, 256]: the GPU candidates of every row against the oracle's."""
    err, ch, codes = iq.encode_candidates(_dev(w), _dev(grid), None if imp is None else _dev(imp),
                                          fmt=fmt, top_c=top_c, codes=True)
    torch.cuda.synchronize()
    return _compare_candidates(err, ch, codes, w, grid, imp, top_c, fmt)


def _check_block_candidates(err, ch, w, grid, imp, top_c, fmt="iq2_xs"):
    """GPU candidates (without codes) of one 256-column block of many rows
    against the oracle's: same choices, bit-exact error vectors, except on
    ties of the choice group's weighted error."""
    G = iq.CHOICE_GROUPS[fmt]
    L = 256 // G
    err = err.cpu().numpy().reshape(-1, G, top_c, L)
    ch = ch.cpu().numpy().reshape(-1, G, top_c)
    rerr, rch, _ = oracle.candidates(fmt, w[None], grid, None if imp is None else imp[None],
                                     top_c=top_c)
    ok = (ch == rch) & np.all(err == rerr, axis=3)
    _judge_candidate_mismatches(ok, err, rerr, imp, G, L)


def _judge_candidate_mismatches(ok, err, rerr, imp, G, L):
    bad = ~ok
    if bad.any():
        wt = np.ones(256) if imp is None else imp.astype(np.float64).reshape(256)
        wt = wt.reshape(G, L)
        e_got = (wt[None, :, None, :] * err.astype(np.float64) ** 2).sum(axis=3)
        e_ref = (wt[None, :, None, :] * rerr.astype(np.float64) ** 2).sum(axis=3)
        rel = np.abs(e_got[bad] - e_ref[bad]) / np.maximum(e_ref[bad], 1e-300)
        assert rel.max() <= 1e-6, "candidate mismatch beyond ties: %g" % rel.max()
        assert bad.mean() < 0.01


def _compare_candidates(err, ch, codes, w, grid, imp, top_c, fmt):
    G = iq.CHOICE_GROUPS[fmt]
    L, nc = 256 // G, (4 if fmt == "iq1_s" else 2)
    err = err.cpu().numpy().reshape(-1, G, top_c, L)
    ch = ch.cpu().numpy().reshape(-1, G, top_c)
    codes = codes.cpu().numpy().view(np.uint16).reshape(-1, G, top_c, nc)
    rerr, rch, rcodes = oracle.candidates(fmt, w[None], grid, None if imp is None else imp[None],
                                          top_c=top_c)
    # where the choice agrees, codes and error vectors are bit-exact, or the
    # entries are a tie
    ok = (ch == rch) & np.all(codes == rcodes, axis=3)
    np.testing.assert_array_equal(err[ok], rerr[ok])
    _judge_candidate_mismatches(ok, err, rerr, imp, G, L)
    return err, ch


def test_candidates_small_rows():
    grid = workloads.iq2xs_grid()
    w = workloads.student_t_weight((40, 256), 31)
    imp = workloads.lognormal_importance((256,), 32)
    _check_candidates(w, grid, imp, 8)
    _check_candidates(w[:5], grid, None, 16)
    _check_candidates(w[:3], workloads.iq2xs_grid(77), imp, 1)


def test_candidates_with_grids_not_exact_in_bf16():
    # The fp32-operand sweep of the candidates kernel.
    w = workloads.student_t_weight((24, 256), 35)
    imp = workloads.lognormal_importance((256,), 36)
    _check_candidates(w, workloads.iq2xs_wide_grid(), imp, 8)
    _check_candidates(w[:6], workloads.iq2xs_real_grid(200, 3), imp, 16)
    _check_candidates(w[:4], workloads.iq2xs_real_grid(45, 4), None, 3)


def test_candidates_zero_block():
    grid = workloads.iq2xs_grid()
    w = workloads.student_t_weight((3, 256), 33)
    w[1] = 0.0
    err, ch = _check_candidates(w, grid, None, 8)
    assert ch.shape == (3, 16, 8) and np.all(ch[1] == np.arange(8))
    np.testing.assert_array_equal(err[1], np.broadcast_to(-w[1].reshape(16, 1, 16), (16, 8, 16)))


def _search_parity(H, cand, sweeps=2):
    picks, trace = iq.choice_search(_dev(H), _dev(cand), sweeps=sweeps, trace=True)
    torch.cuda.synchronize()
    picks = picks.cpu().numpy()
    trace = trace.cpu().numpy()
    np.testing.assert_array_equal(picks, trace[-1])
    rpicks, rtrace = oracle.choice_search(H, cand, sweeps=sweeps)
    differ = np.nonzero(np.any(trace != rtrace, axis=(0, 2)))[0]
    for r in differ:
        fail, worst = oracle.choice_replay(H, cand[r], trace[:, r, :], REPLAY_TOL)
        assert fail == 0, "row %d: decision %d off by %.3g of J" % (r, fail - 1, worst)
    assert len(differ) <= max(2, 0.01 * cand.shape[0])
    return trace, rtrace, len(differ)


@pytest.mark.parametrize("G,C,rows", [(16, 8, 37), (8, 4, 20), (16, 16, 9), (8, 16, 11), (16, 1, 5),
                                      (16, 3, 23), (8, 5, 13), (16, 12, 18)])
def test_choice_search_random_candidates(G, C, rows):
    H = workloads.block_hessian(256, 7)
    rng = np.random.default_rng(G * 100 + C)
    cand = (0.01 * rng.standard_normal((rows, G, C, 256 // G))).astype(np.float32)
    _search_parity(H, cand)
    _search_parity(H, cand, sweeps=0)
    _search_parity(H, cand, sweeps=3)


def test_identity_hessian_keeps_the_encoders_own_choices():
    grid = workloads.iq2xs_grid()
    w = workloads.student_t_weight((16, 256), 141)
    err, ch, _ = iq.encode_candidates(_dev(w), _dev(grid), None, top_c=8)
    picks, trace = iq.choice_search(torch.eye(256, device=DEV), err.reshape(16, 16, 8, 16).contiguous(),
                                    trace=True)
    torch.cuda.synchronize()
    assert int(trace.abs().sum().item()) == 0


def test_search_keeps_the_pick_on_an_exact_tie():
    # Exact arithmetic (the oracle pin of the same name): group 0's two
    # candidates tie at score 4 in the first sweep; the strict-improvement
    # rule keeps step 2's candidate 1.  Rows of the 16-row workgroup differ
    # only in which of the other groups carry nonzero, untied candidates.
    G, C, L = 16, 2, 16
    H = np.eye(256, dtype=np.float32)
    H[0, 16] = H[16, 0] = 0.5
    cand = np.zeros((20, G, C, L), np.float32)
    cand[:, 0, 0, :2] = (-2.0, 2.0)
    cand[:, 0, 1, :2] = (0.0, 2.0)
    cand[:, 1, 0, 0] = 2.0
    cand[:, 1, 1, 0] = 3.0
    for r in range(20):
        g = 2 + r % 14
        cand[r, g, 0, 3] = 1.0 + r           # candidate 1 (zero) is better in group g
    picks, trace = iq.choice_search(_dev(H), _dev(cand), sweeps=2, trace=True)
    torch.cuda.synchronize()
    picks = picks.cpu().numpy()
    assert np.all(picks[:, 0] == 1) and np.all(picks[:, 1] == 0)
    rpicks, rtrace = oracle.choice_search(H, cand, sweeps=2)
    np.testing.assert_array_equal(picks, rpicks)
    np.testing.assert_array_equal(trace.cpu().numpy(), rtrace)


def test_c5_choice_search_full():
    cfg = workloads.c5_choice_search()
    H, w, grid, imp = cfg["H"], cfg["w"][0], cfg["grid"], cfg["importance"][0]
    err, ch, _ = iq.encode_candidates(_dev(w), _dev(grid), _dev(imp), top_c=8)
    cand = err.reshape(4096, 16, 8, 16).contiguous()
    # the candidates of every row against the oracle
    _check_candidates(w, grid, imp, 8)
    cand_np = cand.cpu().numpy()
    trace, rtrace, nd = _search_parity(H, cand_np)
    # the sweeps change picks on this workload (a search that skipped them fails)
    assert np.any(trace[0] != trace[2])
    J = [oracle.choice_objective(H, cand_np, trace[s]) for s in range(3)]
    assert np.all(J[1] <= J[0] * (1 + 1e-6)) and np.all(J[2] <= J[1] * (1 + 1e-6))


def test_iq1s_candidates_small_rows():
    grid = workloads.iq1s_grid()
    w = workloads.normal_weight((24, 256), 34)
    imp = workloads.lognormal_importance((256,), 35)
    _check_candidates(w, grid, imp, 8, fmt="iq1_s")
    _check_candidates(w[:6], grid, None, 16, fmt="iq1_s")
    _check_candidates(w[:4], workloads.iq1s_grid(333), imp, 1, fmt="iq1_s")


@pytest.mark.parametrize("fmt,top_c", [("iq2_xs", 8), ("iq2_xs", 16), ("iq1_s", 8), ("iq1_s", 16),
                                       ("iq1_m", 8)])
def test_candidates_with_exactly_tied_choices(fmt, top_c):
    # A choice group of zero importance in a live block: every choice costs
    # exactly 0, so the (cost, choice) order is the choice order and the
    # kernel leaves its once-formed ranking for the per-round selection.
    grid = {"iq2_xs": workloads.iq2xs_grid, "iq1_s": workloads.iq1s_grid,
            "iq1_m": workloads.iq1s_grid}[fmt]()
    w = workloads.student_t_weight((12, 256), 41)
    imp = workloads.lognormal_importance((256,), 42)
    L = 256 // iq.CHOICE_GROUPS[fmt]
    imp[L:2 * L] = 0.0
    err, ch = _check_candidates(w, grid, imp, top_c, fmt=fmt)
    assert np.all(ch[:, 1] == np.arange(top_c))


def test_iq1s_candidates_zero_and_rejected_blocks():
    grid = workloads.iq1s_grid(256)
    w = workloads.normal_weight((3, 512), 36)
    w[1, :256] = 0.0
    err, ch = _check_candidates(w[:, :256], grid, None, 8, fmt="iq1_s")
    assert ch.shape == (3, 8, 8) and np.all(ch[1] == np.arange(8))
    np.testing.assert_array_equal(err[1], np.broadcast_to(-w[1, :256].reshape(8, 1, 32), (8, 8, 32)))
    bad = w.copy()
    bad[2, 300] = np.nan
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    e2, c2, k2 = iq.encode_candidates(_dev(bad), _dev(grid), fmt="iq1_s", top_c=4, codes=True,
                                      status=st, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == 5
    assert not e2[2, 1].abs().sum().item() and not k2[2, 1].abs().sum().item()


def test_iq1s_candidates_and_search():
    # IQ1_S: G = 8 sub-blocks of 32 columns, C = 8 and 16 candidates.
    H = workloads.block_hessian(256, 11)
    grid = workloads.iq1s_grid()
    w = workloads.normal_weight((1, 96, 256), 37)[0]
    imp = np.sqrt(np.diag(H).astype(np.float64)).astype(np.float32)
    for top_c in (8, 16):
        err, ch = _check_candidates(w, grid, imp, top_c, fmt="iq1_s")
        cand = np.ascontiguousarray(err.reshape(96, 8, top_c, 32))
        trace, rtrace, nd = _search_parity(H, cand)
        J = [oracle.choice_objective(H, cand, trace[s]) for s in range(3)]
        assert np.all(J[1] <= J[0] * (1 + 1e-6)) and np.all(J[2] <= J[1] * (1 + 1e-6))


@pytest.mark.parametrize("fmt", ["iq2_xs", "iq1_s"])
def test_batched_block_search_equals_per_block_searches(fmt):
    # Three 256-column blocks of one weight, each with its own H, in one launch.
    G = 16 if fmt == "iq2_xs" else 8
    grid = workloads.iq2xs_grid() if fmt == "iq2_xs" else workloads.iq1s_grid()
    Hs = np.stack([workloads.block_hessian(256, s) for s in (7, 8, 9)])
    w = workloads.student_t_weight((1, 70, 768), 38)[0]
    imp = np.sqrt(np.concatenate([np.diag(h) for h in Hs]).astype(np.float64)).astype(np.float32)
    err, ch, _ = iq.encode_candidates(_dev(w), _dev(grid), _dev(imp), fmt=fmt, top_c=6)
    cand = err.reshape(70, 3, G, 6, 256 // G).contiguous()
    picks, trace = iq.choice_search(_dev(Hs), cand, trace=True)
    torch.cuda.synchronize()
    assert picks.shape == (70, 3, G) and trace.shape == (3, 70, 3, G)
    cand_np = cand.cpu().numpy()
    for b in range(3):
        cb = np.ascontiguousarray(cand_np[:, b])
        p1, t1 = iq.choice_search(_dev(Hs[b]), _dev(cb), trace=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(picks[:, b].cpu().numpy(), p1.cpu().numpy())
        np.testing.assert_array_equal(trace[:, :, b].cpu().numpy(), t1.cpu().numpy())
        _search_parity(Hs[b], cb)


def test_c5_iq1s_choice_search_full():
    cfg = workloads.c5_iq1s_choice_search()
    H, w, grid, imp = cfg["H"], cfg["w"][0], cfg["grid"], cfg["importance"][0]
    err, ch, _ = iq.encode_candidates(_dev(w), _dev(grid), _dev(imp), fmt="iq1_s", top_c=8)
    cand = err.reshape(4096, 8, 8, 32).contiguous()
    _check_candidates(w, grid, imp, 8, fmt="iq1_s")
    cand_np = cand.cpu().numpy()
    trace, rtrace, nd = _search_parity(H, cand_np)
    assert np.any(trace[0] != trace[2])


def test_c5_weight_batched_search_full():
    # The whole 4096x4096 IQ2_XS weight: candidates of all 16 blocks in one
    # launch, the 16 blocks searched in one launch; every row of every block
    # against the oracle (candidates, and the search by trace replay).
    cfg = workloads.c5_weight_choice_search()
    Hs, w, grid, imp = cfg["H"], cfg["w"][0], cfg["grid"], cfg["importance"][0]
    err, ch, _ = iq.encode_candidates(_dev(w), _dev(grid), _dev(imp), top_c=8)
    cand = err.reshape(4096, 16, 16, 8, 16)
    picks, trace = iq.choice_search(_dev(Hs), cand, trace=True)
    torch.cuda.synchronize()
    cand_np = cand.cpu().numpy()
    tr = trace.cpu().numpy()
    for b in range(16):
        cb = np.ascontiguousarray(cand_np[:, b])
        rpicks, rtrace = oracle.choice_search(Hs[b], cb, sweeps=2)
        differ = np.nonzero(np.any(tr[:, :, b] != rtrace, axis=(0, 2)))[0]
        for r in differ:
            fail, worst = oracle.choice_replay(Hs[b], cb[r], tr[:, r, b, :], REPLAY_TOL)
            assert fail == 0, "block %d row %d: decision %d off by %.3g" % (b, r, fail - 1, worst)
        assert len(differ) <= max(2, 0.01 * 4096)
        # the candidates of every row of this block against the oracle's
        _check_block_candidates(err.reshape(4096, 16, 16, 8, 16)[:, b], ch.reshape(4096, 16, 16, 8)[:, b],
                                np.ascontiguousarray(w[:, 256 * b:256 * (b + 1)]), grid,
                                np.ascontiguousarray(imp[256 * b:256 * (b + 1)]), 8)


def test_iq1m_candidates_and_search():
    # IQ1_M: 16 scale groups of 16 columns, 8 local scales (the shift is free
    # per group); candidates against the oracle, then the G = 16 search.
    H = workloads.block_hessian(256, 12)
    grid = workloads.iq1s_grid()
    w = workloads.normal_weight((1, 80, 256), 39)[0]
    w[3] = 0.0
    imp = np.sqrt(np.diag(H).astype(np.float64)).astype(np.float32)
    err, ch = _check_candidates(w, grid, imp, 8, fmt="iq1_m")
    assert np.all(ch[3] == np.arange(8))
    _check_candidates(w[:7], workloads.iq1s_grid(999), None, 3, fmt="iq1_m")
    cand = np.ascontiguousarray(err.reshape(80, 16, 8, 16))
    trace, rtrace, nd = _search_parity(H, cand)
    J = [oracle.choice_objective(H, cand, trace[s]) for s in range(3)]
    assert np.all(J[1] <= J[0] * (1 + 1e-6)) and np.all(J[2] <= J[1] * (1 + 1e-6))
    with pytest.raises(iq.IQError) as ei:
        iq.encode_candidates(_dev(w), _dev(grid), fmt="iq1_m", top_c=9)
    assert ei.value.code == 8
