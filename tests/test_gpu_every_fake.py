"""Every-choice payloads and the fused encode-decode (fake quant), through the
C-ABI, against the GPU's own forced encodes and decode and against the oracle.

Every-choice ("[2/4] Encode every GGML IQ choice in one pass" #3159): entry c
must equal, byte for byte, the encode with every choice group forced to c.
Fake quant: the decoded values must equal, bit for bit, iq_dequant of the
payload iq_encode writes with the same arguments, and the oracle's decode of
that payload.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import compare_payloads, grid_for, oracle_cached

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the CPU suite deselects these with -m "not gpu"
    pytest.skip("no GPU", allow_module_level=True)

import ggml_iq_codebook_amd as iq  # noqa: E402

DEV = "cuda:0"
G = {"iq1_s": 8, "iq2_xs": 16, "iq1_m": 16}
FMTS = ["iq1_s", "iq2_xs", "iq1_m"]


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write("\n[gpu] %s\n" % request.node.nodeid)
    sys.__stderr__.flush()
    yield


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _block_imp(imp, B, R, C):
    imp = np.asarray(imp, np.float32).reshape(B, C)
    return np.broadcast_to(imp[:, None, :], (B, R, C)).reshape(-1, 256)


def _scales_of(p):
    return (p[..., 0].astype(np.uint16) | (p[..., 1].astype(np.uint16) << 8))


def _bits(t):
    return t.contiguous().view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape,n", [((2, 5, 512), None), ((1, 3, 768), 301)])
def test_every_choice_equals_the_forced_encodes(fmt, shape, n):
    grid = grid_for(fmt, n, seed=5)
    w = workloads.student_t_weight(shape, 201)
    w[0, 1, :256] = 0.0                              # a zero block
    imp = workloads.lognormal_importance((shape[0], shape[2]), 202)
    B, R, C = shape
    every = iq.encode_every_choice(_dev(w), _dev(grid), _dev(imp), fmt=fmt)
    torch.cuda.synchronize()
    nc = iq.NUM_CHOICES[fmt]
    assert every.shape == (nc, B, R, C // 256, iq.BLOCK_BYTES[fmt])
    ev = every.cpu().numpy()
    ref = oracle.encode_every_choice(fmt, w, grid, imp)
    for c in range(nc):
        full = torch.full((B, R, C // 256, G[fmt]), c, dtype=torch.int32, device=DEV)
        forced = iq.encode(_dev(w), _dev(grid), _dev(imp), fmt=fmt, choices=full)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ev[c], forced.cpu().numpy(), err_msg="choice %d" % c)
        compare_payloads(fmt, ev[c], ref[c], w.reshape(-1, 256), grid, _block_imp(imp, B, R, C))


@pytest.mark.parametrize("fmt", FMTS)
def test_every_choice_under_pinned_scales_and_without_importance(fmt):
    grid = grid_for(fmt)
    w = workloads.normal_weight((1, 4, 512), 203)
    d = oracle.predict_scales(fmt, w * np.float32(0.75)).reshape(1, 4, 2)
    sc = torch.from_numpy(d.view(np.int16)).to(DEV)
    every = iq.encode_every_choice(_dev(w), _dev(grid), fmt=fmt, scales=sc)
    torch.cuda.synchronize()
    ref = oracle.encode_every_choice(fmt, w, grid, None, scales=d)
    for c in range(iq.NUM_CHOICES[fmt]):
        compare_payloads(fmt, every[c].cpu().numpy(), ref[c], w.reshape(-1, 256), grid)


@pytest.mark.parametrize("fmt", FMTS)
def test_every_choice_zeroes_rejected_blocks_in_every_payload(fmt):
    grid = grid_for(fmt, 64)
    w = workloads.normal_weight((1, 3, 512), 204)
    w[0, 1, 260] = np.inf
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    every = iq.encode_every_choice(_dev(w), _dev(grid), fmt=fmt, status=st, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == 5                       # IQ_ERR_NONFINITE
    ev = every.cpu().numpy()
    assert not ev[:, 0, 1, 1].any()
    ok = w.copy()
    ok[0, 1, 256:] = 0.0
    ref = oracle.encode_every_choice(fmt, ok, grid)
    keep = [0, 1, 2, 4, 5]                           # blocks other than the rejected one
    nc = iq.NUM_CHOICES[fmt]
    np.testing.assert_array_equal(ev.reshape(nc, 6, -1)[:, keep], ref.reshape(nc, 6, -1)[:, keep])


def test_every_choice_c2_full():
    # The full IQ1_S 4096x4096 weighted workload in one launch; all 16
    # payloads, every block, against the oracle's forced encodes.
    cfg = workloads.c2_iq1s_4096()
    w, grid, imp = cfg["w"], cfg["grid"], cfg["importance"]
    B, R, C = w.shape
    every = iq.encode_every_choice(_dev(w), _dev(grid), _dev(imp), fmt="iq1_s")
    torch.cuda.synchronize()
    ev = every.cpu().numpy().reshape(16, -1, 50)
    ref = oracle.encode_every_choice("iq1_s", w, grid, imp).reshape(16, -1, 50)
    ib = _block_imp(imp, B, R, C)
    for c in range(16):
        compare_payloads("iq1_s", ev[c], ref[c], w.reshape(-1, 256), grid, ib)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mode", ["free", "pinned", "forced", "uniform"])
def test_fake_quant_is_bitwise_the_decoded_payload(fmt, mode):
    grid = grid_for(fmt, 300 if fmt == "iq2_xs" else 1200)
    w = workloads.normal_weight((2, 6, 512), 211)
    w[1, 3, 256:] = 0.0                              # a zero block (decodes to signed zeros)
    imp = None if mode == "uniform" else workloads.lognormal_importance((2, 512), 212)
    kw = {}
    if mode == "pinned":
        kw["scales"] = torch.from_numpy(oracle.predict_scales(fmt, w * np.float32(1.3))
                                        .reshape(2, 6, 2).view(np.int16)).to(DEV)
    if mode == "forced":
        kw["choices"] = _dev(np.random.default_rng(213).integers(0, iq.NUM_CHOICES[fmt],
                                                                 (2, 6, 2, G[fmt])).astype(np.int32))
    wi = None if imp is None else _dev(imp)
    xh, pk = iq.fake_quant(_dev(w), _dev(grid), wi, fmt=fmt, packed=True, **kw)
    p = iq.encode(_dev(w), _dev(grid), wi, fmt=fmt, **kw)
    xd = iq.dequant(p, _dev(grid), fmt=fmt)
    torch.cuda.synchronize()
    assert torch.equal(pk, p)
    np.testing.assert_array_equal(_bits(xh), _bits(xd))
    np.testing.assert_array_equal(xh.cpu().numpy().astype(np.float64),
                                  oracle.decode(fmt, p.cpu().numpy(), grid))
    # the payload behind it against the oracle's encode
    sc = kw["scales"].cpu().numpy().view(np.uint16) if "scales" in kw else None
    ch = kw["choices"].cpu().numpy() if "choices" in kw else None
    ref = oracle.encode(fmt, w, grid, imp, scales=sc, choices=ch)
    compare_payloads(fmt, p.cpu().numpy(), ref, w.reshape(-1, 256), grid,
                     None if imp is None else _block_imp(imp, 2, 6, 512))


@pytest.mark.parametrize("fmt", FMTS)
def test_fake_quant_writes_zeros_for_rejected_blocks(fmt):
    grid = grid_for(fmt, 128)
    w = workloads.normal_weight((1, 2, 512), 214)
    w[0, 1, 3] = np.nan
    out = torch.full((1, 2, 512), 5.0, dtype=torch.float32, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    iq.fake_quant(_dev(w), _dev(grid), fmt=fmt, out=out, status=st, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == 5
    o = out.cpu().numpy()
    assert np.all(o[0, 1, :256] == 0.0) and not np.signbit(o[0, 1, :256]).any()
    ok = np.delete(w.reshape(4, 256), 2, axis=0).reshape(1, 3, 256)
    want = oracle.fake_quant(fmt, ok, grid).reshape(3, 256)
    np.testing.assert_array_equal(np.delete(o.reshape(4, 256), 2, axis=0).astype(np.float64), want)


@pytest.mark.parametrize("kind", ["wide", "real"])
def test_iq2xs_every_choice_and_fake_quant_with_grids_not_exact_in_bf16(kind):
    # The fp32-operand sweep: every-choice payloads equal the forced encodes
    # and the oracle; the fused decode is bitwise the decode of the payload.
    grid = (workloads.iq2xs_wide_grid if kind == "wide" else workloads.iq2xs_real_grid)(300, 6)
    w = workloads.student_t_weight((1, 4, 512), 216)
    imp = workloads.lognormal_importance((1, 512), 217)
    every = iq.encode_every_choice(_dev(w), _dev(grid), _dev(imp), fmt="iq2_xs")
    xh, pk = iq.fake_quant(_dev(w), _dev(grid), _dev(imp), fmt="iq2_xs", packed=True)
    xd = iq.dequant(pk, _dev(grid), fmt="iq2_xs")
    torch.cuda.synchronize()
    ev = every.cpu().numpy()
    ref = oracle.encode_every_choice("iq2_xs", w, grid, imp)
    for c in range(16):
        full = torch.full((1, 4, 2, 16), c, dtype=torch.int32, device=DEV)
        forced = iq.encode(_dev(w), _dev(grid), _dev(imp), fmt="iq2_xs", choices=full)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ev[c], forced.cpu().numpy(), err_msg="choice %d" % c)
        compare_payloads("iq2_xs", ev[c], ref[c], w.reshape(-1, 256), grid, _block_imp(imp, 1, 4, 512))
    np.testing.assert_array_equal(_bits(xh), _bits(xd))
    compare_payloads("iq2_xs", pk.cpu().numpy(), oracle.encode("iq2_xs", w, grid, imp),
                     w.reshape(-1, 256), grid, _block_imp(imp, 1, 4, 512))


def test_fake_quant_rejects_output_overlapping_the_weight():
    grid = _dev(workloads.iq1s_grid(64))
    w = _dev(workloads.normal_weight((1, 4, 256), 215))
    with pytest.raises(iq.IQError) as ei:
        iq.fake_quant(w, grid, out=w)
    assert ei.value.code == 8                        # IQ_ERR_ARG


def test_fake_quant_c2_full_size():
    # The fused path at the full IQ1_S 4096x4096 weighted workload: bitwise the
    # decode of its own payload; the payload, every block, against the
    # oracle's encode, and the values against the oracle's decode.
    cfg = workloads.c2_iq1s_4096()
    w, grid, imp = cfg["w"], cfg["grid"], cfg["importance"]
    xh, pk = iq.fake_quant(_dev(w), _dev(grid), _dev(imp), fmt="iq1_s", packed=True)
    xd = iq.dequant(pk, _dev(grid), fmt="iq1_s")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(xh), _bits(xd))
    p = pk.cpu().numpy()
    ref = oracle_cached(("c2", "iq1_s", "encode"), lambda: oracle.encode("iq1_s", w, grid, imp))
    compare_payloads("iq1_s", p, ref, w.reshape(-1, 256), grid, _block_imp(imp, *w.shape))
    np.testing.assert_array_equal(xh.cpu().numpy().astype(np.float64),
                                  oracle.decode("iq1_s", p, grid))
