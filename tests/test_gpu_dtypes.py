"""Weights stored as bf16, fp16 or fp64 (the #2450 code review: the encoders
take float32, float64, float16 and bfloat16 weights), through the C-ABI.

The kernels read every value as fp32: bf16 and fp16 exactly, fp64 rounded to
nearest even.  So the payload, every-choice payloads, fused decode and
candidates of a typed weight must equal, byte for byte, those of its fp32
conversion (numpy's round-to-nearest-even cast for fp64), and the payload
must match the oracle's encode of those fp32 values.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import compare_payloads, grid_for

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the CPU suite deselects these with -m "not gpu"
    pytest.skip("no GPU", allow_module_level=True)

import ggml_iq_codebook_amd as iq  # noqa: E402

DEV = "cuda:0"
FMTS = ["iq1_s", "iq2_xs", "iq1_m"]
DTYPES = [torch.bfloat16, torch.float16, torch.float64]


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write("\n[gpu] %s\n" % request.node.nodeid)
    sys.__stderr__.flush()
    yield


def _typed(shape, dt, seed):
    """A weight in dt and its fp32 values (the conversion the kernels apply)."""
    x = workloads.student_t_weight(shape, seed).astype(np.float64)
    if dt == torch.float64:
        # values fp32 cannot hold exactly: the cast rounds
        x = x * (1.0 + 1e-9 * np.random.default_rng(seed + 1).standard_normal(shape))
        wt = torch.from_numpy(x)
        w32 = x.astype(np.float32)
    else:
        wt = torch.from_numpy(x.astype(np.float32)).to(dt)
        w32 = wt.float().numpy()
    return wt.to(DEV), w32


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _block_imp(imp, B, R, C):
    return np.broadcast_to(np.asarray(imp, np.float32).reshape(B, 1, C), (B, R, C)).reshape(-1, 256)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dt", DTYPES, ids=["bf16", "f16", "f64"])
def test_typed_weights_encode_like_their_fp32_values(fmt, dt):
    shape = (2, 5, 512)
    wt, w32 = _typed(shape, dt, 301)
    if dt == torch.float64:
        assert not np.array_equal(w32.astype(np.float64), wt.cpu().numpy())
    grid = grid_for(fmt, 700 if fmt != "iq2_xs" else 300, seed=7)
    imp = workloads.lognormal_importance((2, 512), 302)
    g, i, wf = _dev(grid), _dev(imp), _dev(w32)
    p = iq.encode(wt, g, i, fmt=fmt)
    p32 = iq.encode(wf, g, i, fmt=fmt)
    ev = iq.encode_every_choice(wt, g, i, fmt=fmt)
    ev32 = iq.encode_every_choice(wf, g, i, fmt=fmt)
    xh, pk = iq.fake_quant(wt, g, i, fmt=fmt, packed=True)
    xh32 = iq.fake_quant(wf, g, i, fmt=fmt)
    torch.cuda.synchronize()
    assert torch.equal(p, p32)
    assert torch.equal(ev, ev32)
    assert torch.equal(pk, p)
    assert torch.equal(xh.view(torch.int32), xh32.view(torch.int32))
    compare_payloads(fmt, p.cpu().numpy(), oracle.encode(fmt, w32, grid, imp),
                     w32.reshape(-1, 256), grid, _block_imp(imp, *shape))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dt", DTYPES, ids=["bf16", "f16", "f64"])
def test_typed_weights_candidates_like_their_fp32_values(fmt, dt):
    wt, w32 = _typed((1, 24, 512), dt, 303)
    grid = grid_for(fmt, None, seed=8)
    imp = workloads.lognormal_importance((512,), 304)
    g, i = _dev(grid), _dev(imp)
    a = iq.encode_candidates(wt[0], g, i, fmt=fmt, top_c=5, codes=True)
    b = iq.encode_candidates(_dev(w32[0]), g, i, fmt=fmt, top_c=5, codes=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int32) if u.dtype == torch.float32 else u,
                           v.view(torch.int32) if v.dtype == torch.float32 else v)


def test_typed_weights_reject_values_fp32_cannot_hold():
    # A finite fp64 weight beyond fp32's range reads as infinite: its block is
    # rejected as non-finite and written as zeros; a bf16 infinity likewise.
    grid = _dev(workloads.iq1s_grid(256))
    x = workloads.normal_weight((1, 3, 256), 305).astype(np.float64)
    x[0, 1, 17] = 1e300
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    p = iq.encode(_dev(x), grid, fmt="iq1_s", status=st, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == 5                       # IQ_ERR_NONFINITE
    p = p.cpu().numpy()
    assert not p[0, 1].any() and p[0, 0].any() and p[0, 2].any()
    xb = torch.from_numpy(workloads.normal_weight((1, 2, 256), 306)).to(torch.bfloat16)
    xb[0, 0, 3] = float("inf")
    st.zero_()
    p = iq.encode(xb.to(DEV), grid, fmt="iq1_s", status=st, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == 5
    assert not p[0, 0].any()


def test_unsupported_weight_dtype_is_refused():
    grid = _dev(workloads.iq1s_grid(64))
    with pytest.raises(TypeError):
        iq.encode(torch.zeros((1, 2, 256), dtype=torch.int32, device=DEV), grid)
