"""HIP encode / decode parity against the oracle, through the C-ABI.

Every test runs the HIP kernels of libiqcodec.so on a gfx950 GPU and compares
with the CPU oracle on the same seeded inputs: bit-exact scales, bit-exact
codes except on floating-point ties (then the float64 weighted errors agree
within 1e-6 relative), bit-exact decoded values.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import compare_payloads, grid_for, oracle_cached, scale_bits, unit_codes

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the CPU suite deselects these with -m "not gpu"
    pytest.skip("no GPU", allow_module_level=True)

import ggml_iq_codebook_amd as iq  # noqa: E402

DEV = "cuda:0"
FMTS = ["iq1_s", "iq2_xs", "iq1_m"]


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write("\n[gpu] %s\n" % request.node.nodeid)
    sys.__stderr__.flush()
    yield


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _block_imp(imp, B, R, C):
    if imp is None:
        return None
    imp = np.asarray(imp, np.float32).reshape(B, C)
    return np.broadcast_to(imp[:, None, :], (B, R, C)).reshape(-1, 256)


def _gpu_encode(fmt, w, grid, imp=None, **kw):
    out = iq.encode(_dev(w), _dev(grid), None if imp is None else _dev(imp), fmt=fmt, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_full(fmt, w, grid, imp=None):
    B, R, C = w.shape
    got = _gpu_encode(fmt, w, grid, imp)
    ref = oracle.encode(fmt, w, grid, imp)
    return compare_payloads(fmt, got, ref, w.reshape(-1, 256), grid, _block_imp(imp, B, R, C))


def test_library_is_the_hip_build():
    L = iq.load(build_if_missing=False)
    assert L._name.endswith("libiqcodec.so")
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")


@pytest.mark.parametrize("uniform", [None, "ones"])
def test_c1_iq1s_small_matches_oracle(uniform):
    c = workloads.c1_iq1s_small()
    imp = None if uniform is None else np.ones((1, 256), np.float32)
    _check_full("iq1_s", c["w"], c["grid"], imp)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape,n", [((2, 13, 768), None), ((1, 5, 256), 1000), ((1, 3, 512), 37),
                                     ((1, 2, 256), 1), ((3, 1, 1024), 33)])
def test_ragged_shapes_and_grid_sizes(fmt, shape, n):
    grid = grid_for(fmt, n, seed=3)
    w = workloads.student_t_weight(shape, 17)
    imp = workloads.lognormal_importance((shape[0], shape[2]), 18)
    _check_full(fmt, w, grid, imp)


def _iq2xs_grid_kind(kind, n, seed):
    if kind == "wide":
        return workloads.iq2xs_wide_grid(n, seed)
    if kind == "real":
        return workloads.iq2xs_real_grid(n, seed)
    grid = workloads.iq2xs_grid(n, seed)          # "one_off": one value off bf16
    grid[-1, 7] = np.float32(5.0 + 2.0 ** -18)
    return grid


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n", [None, 37, 300])
def test_full_sets_then_a_short_set(fmt, n):
    # 4101 blocks: 257 sets of 16 blocks for 256 persistent workgroups, so one
    # workgroup takes a full set and then a set of 5.  The waves of a full set
    # meet at workgroup barriers during the sweep (one per tracking chunk: a
    # truncated grid has one or a few chunks); a short set takes none (its
    # idle waves never reach them).
    w = workloads.normal_weight((1, 4101, 256), 61)
    imp = workloads.lognormal_importance((1, 256), 62)
    _check_full(fmt, w, grid_for(fmt, n), imp)


@pytest.mark.parametrize("fmt,mode", [("iq1_s", "encode"), ("iq1_s", "fake"), ("iq1_m", "encode"),
                                      ("iq2_xs", "encode"), ("iq2_xs", "fake")])
def test_repeated_full_size_launches_are_identical(fmt, mode):
    # The 4096x4096 workload launched again and again: every output byte the
    # same each time (the sweeps' workgroup barriers and LDS staging leave no
    # room for a race to show as a changed code or value).
    cfg = workloads.c3_iq2xs_4096() if fmt == "iq2_xs" else workloads.c2_iq1s_4096()
    w, grid, imp = _dev(cfg["w"]), _dev(cfg["grid"]), _dev(cfg["importance"])
    fn = iq.encode if mode == "encode" else iq.fake_quant
    ref = fn(w, grid, imp, fmt=fmt)
    for _ in range(6):
        assert torch.equal(fn(w, grid, imp, fmt=fmt), ref)


@pytest.mark.parametrize("kind", ["wide", "real", "one_off"])
@pytest.mark.parametrize("shape,n", [((2, 5, 768), 512), ((1, 3, 512), 37), ((1, 4, 256), 100)])
def test_iq2xs_grids_not_exact_in_bf16(kind, shape, n):
    # Grids whose values or squares bf16 cannot hold take the fp32-operand
    # sweep; the payload must match the oracle as for the {1,3,5} grids.
    grid = _iq2xs_grid_kind(kind, n, 41)
    w = workloads.student_t_weight(shape, 42)
    imp = workloads.lognormal_importance((shape[0], shape[2]), 43)
    _check_full("iq2_xs", w, grid, imp)
    _check_full("iq2_xs", w, grid, None)


@pytest.mark.parametrize("fmt", ["iq1_s", "iq1_m"])
def test_zero_choice_group_in_a_live_block_takes_the_lowest_choice(fmt):
    # delta = +1/8 and -1/8 tie exactly on an all-zero choice group when the
    # grid holds the all-zero entry: the lowest choice and the zero entry win,
    # as in the oracle (the pin of the same name).
    grid = grid_for(fmt, 300)
    grid[7] = 0.0
    w = workloads.normal_weight((1, 2, 256), 83)
    L = 32 if fmt == "iq1_s" else 16
    w[0, 0, :L] = 0.0
    w[0, 1, 256 - L:] = 0.0
    imp = workloads.lognormal_importance((1, 256), 84)
    G = 8 if fmt == "iq1_s" else 16
    for im in (None, imp):
        got = _gpu_encode(fmt, w, grid, im)
        ref = oracle.encode(fmt, w, grid, im)
        compare_payloads(fmt, got, ref, w.reshape(-1, 256), grid, _block_imp(im, 1, 2, 256))
        u_got = unit_codes(fmt, got).reshape(2, G, -1)
        u_ref = unit_codes(fmt, ref).reshape(2, G, -1)
        np.testing.assert_array_equal(u_got[0, 0], u_ref[0, 0])
        np.testing.assert_array_equal(u_got[1, -1], u_ref[1, -1])


def test_c3_iq2xs_rows_match_oracle():
    c = workloads.c3_iq2xs_4096()
    w = c["w"][:, :24, :]
    _check_full("iq2_xs", w, c["grid"], c["importance"])


@pytest.mark.parametrize("fmt", FMTS)
def test_uniform_importance_reproduces_unweighted_payload(fmt):
    grid = grid_for(fmt)
    w = workloads.normal_weight((1, 32, 512), 5)
    p0 = _gpu_encode(fmt, w, grid)
    for c in (1.0, 4.0, 0.125):
        p = _gpu_encode(fmt, w, grid, np.full((1, 512), c, np.float32))
        np.testing.assert_array_equal(p, p0)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_is_exact(fmt):
    grid = grid_for(fmt)
    w = workloads.normal_weight((2, 7, 512), 6)
    p = oracle.encode(fmt, w, grid)
    out = iq.dequant(_dev(p), _dev(grid), fmt=fmt)
    torch.cuda.synchronize()
    want = oracle.decode(fmt, p, grid)
    np.testing.assert_array_equal(out.cpu().numpy().astype(np.float64), want)


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_reencode_round_trip_under_pinned_scales(fmt):
    grid = grid_for(fmt)
    w = workloads.normal_weight((1, 16, 512), 7)
    imp = workloads.lognormal_importance((1, 512), 8)
    p = _gpu_encode(fmt, w, grid, imp)
    xhat = iq.dequant(_dev(p), _dev(grid), fmt=fmt)
    d = torch.from_numpy(scale_bits(fmt, p).astype(np.uint16).view(np.int16).reshape(1, 16, 2)).to(DEV)
    p2 = iq.encode(xhat, _dev(grid), _dev(imp), fmt=fmt, scales=d.contiguous())
    x2 = iq.dequant(p2, _dev(grid), fmt=fmt)
    torch.cuda.synchronize()
    assert torch.equal(x2, xhat)
    same = (p2.cpu().numpy().reshape(-1, p.shape[-1]) == p.reshape(-1, p.shape[-1])).all(axis=1)
    assert same.mean() >= 0.9
    # pinned scales match the oracle's pinned encode
    ref = oracle.encode(fmt, xhat.cpu().numpy(), grid, imp, scales=d.cpu().numpy().view(np.uint16))
    compare_payloads(fmt, p2.cpu().numpy(), ref, xhat.cpu().numpy().reshape(-1, 256), grid,
                     _block_imp(imp, 1, 16, 512))


@pytest.mark.parametrize("fmt", FMTS)
def test_forced_choices_match_oracle(fmt):
    grid = grid_for(fmt, 256 if fmt == "iq2_xs" else 512)
    w = workloads.normal_weight((1, 6, 512), 9)
    imp = workloads.lognormal_importance((1, 512), 10)
    G = iq.CHOICE_GROUPS[fmt]
    ch = np.random.default_rng(11).integers(0, iq.NUM_CHOICES[fmt], (1, 6, 2, G)).astype(np.int32)
    got = _gpu_encode(fmt, w, grid, imp, choices=_dev(ch))
    ref = oracle.encode(fmt, w, grid, imp, choices=ch)
    compare_payloads(fmt, got, ref, w.reshape(-1, 256), grid, _block_imp(imp, 1, 6, 512))


@pytest.mark.parametrize("fmt", FMTS)
def test_determinism_and_launch_partition_invariance(fmt):
    grid = grid_for(fmt)
    w = workloads.normal_weight((1, 40, 1024), 12)
    imp = workloads.lognormal_importance((1, 1024), 13)
    a = _gpu_encode(fmt, w, grid, imp)
    b = _gpu_encode(fmt, w, grid, imp)
    np.testing.assert_array_equal(a, b)
    parts = [_gpu_encode(fmt, w[:, r0:r0 + 7], grid, imp) for r0 in range(0, 40, 7)]
    np.testing.assert_array_equal(np.concatenate(parts, axis=1), a)


def test_zero_and_underflow_blocks():
    for fmt in FMTS:
        grid = grid_for(fmt, 64)
        w = workloads.normal_weight((1, 3, 256), 81)
        w[0, 0] = 0.0
        w[0, 1] *= 1e-7
        got = _gpu_encode(fmt, w, grid)
        np.testing.assert_array_equal(got, oracle.encode(fmt, w, grid))
        assert not got[0, 0].any() and not got[0, 1].any()


def _status_of(fn):
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    fn(st)
    torch.cuda.synchronize()
    return int(st.item())


@pytest.mark.parametrize("fmt", FMTS)
def test_device_data_errors_are_reported(fmt):
    grid = grid_for(fmt, 64)
    w = workloads.normal_weight((1, 4, 512), 91)
    bad = w.copy()
    bad[0, 2, 300] = np.nan
    out = torch.full((1, 4, 2, iq.BLOCK_BYTES[fmt]), 7, dtype=torch.uint8, device=DEV)
    st = _status_of(lambda s: iq.encode(_dev(bad), _dev(grid), fmt=fmt, out=out, status=s, check=False))
    assert st == 5                                   # IQ_ERR_NONFINITE
    o = out.cpu().numpy()
    assert not o[0, 2, 1].any()                      # the bad block is zeroed
    np.testing.assert_array_equal(np.delete(o.reshape(8, -1), 5, axis=0),
                                  np.delete(oracle.encode(fmt, w, grid).reshape(8, -1), 5, axis=0))
    imp = np.ones((1, 512), np.float32)
    imp[0, 17] = -1.0
    st = _status_of(lambda s: iq.encode(_dev(w), _dev(grid), _dev(imp), fmt=fmt, status=s, check=False))
    assert st == 6                                   # IQ_ERR_IMPORTANCE
    st = _status_of(lambda s: iq.encode(_dev(w * 1e9), _dev(grid), fmt=fmt, status=s, check=False))
    assert st == 7                                   # IQ_ERR_SCALE_RANGE
    g2 = grid.copy()
    g2[3, 4] = -1.0 if fmt == "iq2_xs" else 2.0
    st = _status_of(lambda s: iq.encode(_dev(w), _dev(g2), fmt=fmt, status=s, check=False))
    assert st == 4                                   # IQ_ERR_GRID
    with pytest.raises(iq.IQError) as ei:
        iq.encode(_dev(bad), _dev(grid), fmt=fmt)
    assert ei.value.code == 5


def test_null_status_synchronizes_and_returns_the_data_error():
    # The C-ABI with status = NULL: the call waits for its stream and returns
    # the first data error itself (IQ_OK when there is none); the output is
    # that of the call with a status word.
    import ctypes
    L = iq.load(build_if_missing=False)
    P = ctypes.c_void_p
    stream = P(torch.cuda.current_stream().cuda_stream)
    grid = _dev(grid_for("iq1_s", 256))
    w = workloads.normal_weight((1, 4, 512), 95)
    bad = w.copy()
    bad[0, 1, 7] = np.inf
    ref = _gpu_encode("iq1_s", w, grid.cpu().numpy())
    for x, want in ((w, 0), (bad, 5), (w, 0)):
        out = torch.full((1, 4, 2, 50), 3, dtype=torch.uint8, device=DEV)
        xd = _dev(x)
        code = L.iq_encode(0, 0, P(xd.data_ptr()), 1, 4, 512, None, P(grid.data_ptr()), 256,
                           None, None, P(out.data_ptr()), None, stream)
        assert code == want
        o = out.cpu().numpy()
        if want == 0:
            np.testing.assert_array_equal(o, ref)
        else:
            assert not o[0, 1, 0].any()
            np.testing.assert_array_equal(np.delete(o.reshape(8, 50), 2, axis=0),
                                          np.delete(ref.reshape(8, 50), 2, axis=0))
    imp = torch.ones(512, dtype=torch.float32, device=DEV)
    imp[3] = float("nan")
    err = torch.empty((4, 2, 8, 4, 32), dtype=torch.float32, device=DEV)
    ch = torch.empty((4, 2, 8, 4), dtype=torch.int32, device=DEV)
    xd = _dev(w[0])
    assert L.iq_encode_candidates(0, 0, P(xd.data_ptr()), 4, 512, P(imp.data_ptr()),
                                  P(grid.data_ptr()), 256, 4, P(err.data_ptr()),
                                  P(ch.data_ptr()), None, None, stream) == 6
    p = oracle.encode("iq1_s", w, grid.cpu().numpy())
    p[0, 2, 1, 2] = 255
    p[0, 2, 1, 34] |= 0x07                            # entry 2047 >= grid_size 256
    pd = _dev(p)
    xo = torch.empty((1, 4, 512), dtype=torch.float32, device=DEV)
    assert L.iq_dequant(0, P(pd.data_ptr()), 1, 4, 512, P(grid.data_ptr()), 256,
                        P(xo.data_ptr()), None, stream) == 9
    # the binding's default (status=None, check=True) is this path
    with pytest.raises(iq.IQError) as ei:
        iq.dequant(pd, grid, fmt="iq1_s")
    assert ei.value.code == 9


def test_synchronous_argument_errors():
    grid = _dev(workloads.iq1s_grid(64))
    w = _dev(workloads.normal_weight((1, 4, 256), 1))
    with pytest.raises(iq.IQError) as ei:
        iq.encode(_dev(workloads.normal_weight((1, 4, 200), 1)), grid)
    assert ei.value.code == 3                        # IQ_ERR_SHAPE
    big = np.concatenate([workloads.iq1s_grid(2048), workloads.iq1s_grid(1)])
    with pytest.raises(iq.IQError) as ei:
        iq.encode(w, _dev(big))
    assert ei.value.code == 4                        # IQ_ERR_GRID
    with pytest.raises(iq.IQError) as ei:
        iq.encode_candidates(w[0], grid, fmt="iq1_s", top_c=17)
    assert ei.value.code == 8                        # IQ_ERR_ARG


def test_dequant_reports_indices_beyond_the_grid():
    grid = workloads.iq1s_grid(1500)
    p = oracle.encode("iq1_s", workloads.normal_weight((1, 1, 256), 72), grid)
    p[0, 0, 0, 34 + 2 * 3 + 1] |= 0x0E
    out = torch.empty((1, 1, 256), dtype=torch.float32, device=DEV)
    st = _status_of(lambda s: iq.dequant(_dev(p), _dev(grid), fmt="iq1_s", out=out, status=s,
                                         check=False))
    assert st == 9                                   # IQ_ERR_CODE
    want = oracle.decode("iq1_s", p, grid, strict=False).reshape(256)
    np.testing.assert_array_equal(out.cpu().numpy().reshape(256).astype(np.float64), want)


# ---------------------------------------------------------------------------
# full-size workloads against the oracle, every block
# ---------------------------------------------------------------------------


def _full(fmt, cfg, name):
    # every block of the workload, in the launch bench.py times, against the
    # oracle's encode of the whole weight
    w, grid, imp = cfg["w"], cfg["grid"], cfg["importance"]
    B, R, C = w.shape
    got = _gpu_encode(fmt, w, grid, imp)
    ref = oracle_cached((name, fmt, "encode"), lambda: oracle.encode(fmt, w, grid, imp))
    return compare_payloads(fmt, got, ref, w.reshape(-1, 256), grid, _block_imp(imp, B, R, C))


def test_c2_iq1s_4096_full():
    _full("iq1_s", workloads.c2_iq1s_4096(), "c2")


def test_c3_iq2xs_4096_full():
    _full("iq2_xs", workloads.c3_iq2xs_4096(), "c3")


def test_iq1m_4096_full():
    # IQ1_M on the IQ1_S workload's 4096x4096 weight, every block
    _full("iq1_m", dict(workloads.c2_iq1s_4096(), fmt="iq1_m"), "c2")


_C4 = {}


def _c4_gpu():
    # The MoE batch (16 experts of 1536x4096) in one batched call, as bench.py
    # times it; encoded once per test process.
    if not _C4:
        cfg = workloads.c4_moe_batch()
        _C4["cfg"] = cfg
        _C4["got"] = _gpu_encode("iq1_s", cfg["w"], cfg["grid"], cfg["importance"])
    return _C4["cfg"], _C4["got"]


@pytest.mark.parametrize("e0", [0, 4, 8, 12])
def test_c4_moe_batch_full(e0):
    # every block of four experts of the batched call against the oracle
    # (the four parts together cover all 16 experts)
    cfg, got = _c4_gpu()
    w, grid, imp = cfg["w"][e0:e0 + 4], cfg["grid"], cfg["importance"][e0:e0 + 4]
    ref = oracle.encode("iq1_s", w, grid, imp)
    compare_payloads("iq1_s", got[e0:e0 + 4], ref, w.reshape(-1, 256), grid,
                     _block_imp(imp, *w.shape))


def test_c4_moe_batch_equals_per_expert_calls():
    cfg, got = _c4_gpu()
    for e in (0, 7, 15):
        one = _gpu_encode("iq1_s", cfg["w"][e:e + 1], cfg["grid"], cfg["importance"][e:e + 1])
        np.testing.assert_array_equal(one[0], got[e])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("weighted", [True, False])
def test_near_tied_choices_follow_the_oracle(fmt, weighted):
    # One choice group per block whose two best choices differ by 1.1e-6 to
    # 4e-6 of its error: above the tie bar, so the kernel must pick the better
    # one, though fp32 rounding of the costs alone could order them either way.
    from tests.parity import near_tie_blocks
    w, grid, imp, d, unit, gap = near_tie_blocks(fmt, 64, 1, weighted)
    assert ((gap > 1e-6) & (gap < 1e-5)).sum() >= 40
    sc = torch.from_numpy(d.view(np.int16)).to(DEV)
    wi = None if imp is None else _dev(imp)
    got = iq.encode(_dev(w), _dev(grid), wi, fmt=fmt, scales=sc)
    xh, pk = iq.fake_quant(_dev(w), _dev(grid), wi, fmt=fmt, scales=sc, packed=True)
    torch.cuda.synchronize()
    ref = oracle.encode(fmt, w, grid, imp, scales=d)
    ib = _block_imp(imp, 1, 64, 256)
    compare_payloads(fmt, got.cpu().numpy(), ref, w.reshape(-1, 256), grid, ib, max_tie_frac=1.0)
    np.testing.assert_array_equal(pk.cpu().numpy(), got.cpu().numpy())


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("weighted", [True, False])
def test_near_tied_entries_follow_the_oracle(fmt, weighted):
    # One group per block whose two best grid entries (IQ1_M: (shift, entry)
    # pairs) differ by 1.1e-6 to 4e-6 of its choice group's error, under a
    # forced choice and a pinned scale: above the tie bar, so the kernel must
    # take the better entry, though fp32 keys alone could order them either
    # way.  Checked in the payload (forced and free choice), the fused
    # fake-quant payload and the candidates.
    from tests.parity import entry_tie_blocks
    w, grid, imp, d, ch, groups, kinds, gap = entry_tie_blocks(fmt, 64, 2, weighted)
    assert ((gap > 1e-6) & (gap < 1e-5)).sum() >= 40
    sc = torch.from_numpy(d.view(np.int16)).to(DEV)
    wi = None if imp is None else _dev(imp)
    ib = _block_imp(imp, 1, 64, 256)
    got = iq.encode(_dev(w), _dev(grid), wi, fmt=fmt, scales=sc, choices=_dev(ch))
    _, pk = iq.fake_quant(_dev(w), _dev(grid), wi, fmt=fmt, scales=sc, choices=_dev(ch),
                          packed=True)
    free = iq.encode(_dev(w), _dev(grid), wi, fmt=fmt, scales=sc)
    torch.cuda.synchronize()
    ref = oracle.encode(fmt, w, grid, imp, scales=d, choices=ch)
    compare_payloads(fmt, got.cpu().numpy(), ref, w.reshape(-1, 256), grid, ib, max_tie_frac=1.0)
    compare_payloads(fmt, pk.cpu().numpy(), ref, w.reshape(-1, 256), grid, ib, max_tie_frac=1.0)
    compare_payloads(fmt, free.cpu().numpy(), oracle.encode(fmt, w, grid, imp, scales=d),
                     w.reshape(-1, 256), grid, ib, max_tie_frac=1.0)
    # the candidates decide entries under every choice with the same sweep
    # (they predict the scale, which the generator kept at the pinned one for
    # IQ1_S and IQ2_XS; IQ1_M's anchor follows the block's RMS, which moved)
    from tests.test_gpu_search import _check_candidates
    _check_candidates(np.ascontiguousarray(w[0]), grid, None if imp is None else imp[0], 8,
                      fmt=fmt)
