"""CPU checks of the C-ABI library: it loads, exports every function that
include/iq_codec.h declares, reports format geometry, and rejects bad
arguments synchronously before any device work (no GPU needed for those)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "iq_codec.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(iq_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import ggml_iq_codebook_amd as iq
    return iq.load(build_if_missing=True)


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "iq_choice_search", "iq_choice_search_blocks", "iq_dequant", "iq_encode",
        "iq_encode_candidates",
        "iq_encode_every_choice", "iq_fake_quant", "iq_format_info", "iq_status_str"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_format_info(lib):
    import ggml_iq_codebook_amd as iq
    assert iq.format_info("iq1_s") == dict(block_elems=256, block_bytes=50, group=8, index_bits=11,
                                           grid_max=2048, choice_groups=8, num_choices=16)
    assert iq.format_info("iq2_xs") == dict(block_elems=256, block_bytes=74, group=8, index_bits=9,
                                            grid_max=512, choice_groups=16, num_choices=16)
    info = iq._FormatInfo()
    assert lib.iq_format_info(7, ctypes.byref(info)) == 2          # IQ_ERR_FORMAT
    assert lib.iq_format_info(0, None) == 1                         # IQ_ERR_NULL


def test_status_strings(lib):
    for code in range(12):
        assert lib.iq_status_str(code)
    assert lib.iq_status_str(99) == b"unknown status"


P = ctypes.c_void_p
FAKE = P(0x100000)      # never dereferenced: validation fails before any device access


def test_encode_argument_errors_need_no_gpu(lib):
    enc = lib.iq_encode
    # fmt, wdtype, w, batch, rows, cols, imp, grid, grid_size, scales, choices, out, status,
    # stream
    assert enc(5, 0, FAKE, 1, 1, 256, None, FAKE, 16, None, None, FAKE, FAKE, None) == 2
    assert enc(0, 0, None, 1, 1, 256, None, FAKE, 16, None, None, FAKE, FAKE, None) == 1
    assert enc(0, 0, FAKE, 1, 1, 200, None, FAKE, 16, None, None, FAKE, FAKE, None) == 3
    assert enc(0, 0, FAKE, 1, 0, 256, None, FAKE, 16, None, None, FAKE, FAKE, None) == 3
    assert enc(0, 0, FAKE, 0, 1, 256, None, FAKE, 16, None, None, FAKE, FAKE, None) == 3
    assert enc(0, 0, FAKE, 1, 1 << 40, 1 << 20, None, FAKE, 16, None, None, FAKE, FAKE, None) == 3
    assert enc(0, 0, FAKE, 1, 1, 256, None, FAKE, 0, None, None, FAKE, FAKE, None) == 4
    assert enc(0, 0, FAKE, 1, 1, 256, None, FAKE, 2049, None, None, FAKE, FAKE, None) == 4
    assert enc(1, 0, FAKE, 1, 1, 256, None, FAKE, 513, None, None, FAKE, FAKE, None) == 4
    assert enc(0, 0, P(0x100004), 1, 1, 256, None, FAKE, 16, None, None, FAKE, FAKE, None) == 8
    # weight storage types: 0 fp32, 1 bf16, 2 fp16, 3 fp64; anything else is IQ_ERR_ARG,
    # and bf16 weights still need 16-byte alignment
    assert enc(0, 4, FAKE, 1, 1, 256, None, FAKE, 16, None, None, FAKE, FAKE, None) == 8
    assert enc(1, -1, FAKE, 1, 1, 256, None, FAKE, 16, None, None, FAKE, FAKE, None) == 8
    assert enc(0, 1, P(0x100008), 1, 1, 256, None, FAKE, 16, None, None, FAKE, FAKE, None) == 8


def test_other_entry_points_argument_errors_need_no_gpu(lib):
    deq = lib.iq_dequant
    assert deq(0, None, 1, 1, 256, FAKE, 16, FAKE, FAKE, None) == 1
    assert deq(0, FAKE, 1, 1, 100, FAKE, 16, FAKE, FAKE, None) == 3
    assert deq(1, FAKE, 1, 1, 256, FAKE, 600, FAKE, FAKE, None) == 4
    cand = lib.iq_encode_candidates
    assert cand(7, 0, FAKE, 1, 256, None, FAKE, 16, 8, FAKE, FAKE, None, FAKE, None) == 2
    assert cand(0, 0, FAKE, 1, 256, None, FAKE, 2049, 8, FAKE, FAKE, None, FAKE, None) == 4
    assert cand(0, 0, FAKE, 1, 256, None, FAKE, 16, 17, FAKE, FAKE, None, FAKE, None) == 8
    assert cand(1, 0, FAKE, 1, 256, None, FAKE, 16, 0, FAKE, FAKE, None, FAKE, None) == 8
    assert cand(1, 0, FAKE, 1, 256, None, FAKE, 16, 17, FAKE, FAKE, None, FAKE, None) == 8
    assert cand(1, 0, FAKE, 1, 250, None, FAKE, 16, 8, FAKE, FAKE, None, FAKE, None) == 3
    assert cand(1, 5, FAKE, 1, 256, None, FAKE, 16, 8, FAKE, FAKE, None, FAKE, None) == 8
    cs = lib.iq_choice_search
    assert cs(FAKE, FAKE, 4, 12, 8, 2, FAKE, None, None) == 8
    assert cs(FAKE, FAKE, 4, 16, 0, 2, FAKE, None, None) == 8
    assert cs(FAKE, FAKE, 4, 16, 17, 2, FAKE, None, None) == 8
    assert cs(FAKE, FAKE, 4, 16, 8, 9, FAKE, None, None) == 8
    assert cs(FAKE, FAKE, 0, 16, 8, 2, FAKE, None, None) == 3
    assert cs(None, FAKE, 4, 16, 8, 2, FAKE, None, None) == 1


def test_every_choice_and_fake_quant_argument_errors_need_no_gpu(lib):
    ev = lib.iq_encode_every_choice
    # fmt, wdtype, w, batch, rows, cols, imp, grid, grid_size, scales, out, status, stream
    assert ev(7, 0, FAKE, 1, 1, 256, None, FAKE, 16, None, FAKE, FAKE, None) == 2
    assert ev(0, 0, FAKE, 1, 1, 300, None, FAKE, 16, None, FAKE, FAKE, None) == 3
    assert ev(1, 0, FAKE, 1, 1, 256, None, FAKE, 16, None, None, FAKE, None) == 1
    assert ev(1, 0, FAKE, 1, 1, 256, None, FAKE, 513, None, FAKE, FAKE, None) == 4
    fq = lib.iq_fake_quant
    # fmt, wdtype, w, batch, rows, cols, imp, grid, grid_size, scales, choices, xhat, out,
    # status, stream
    assert fq(0, 0, FAKE, 1, 1, 256, None, FAKE, 16, None, None, None, None, FAKE, None) == 1
    assert fq(0, 0, FAKE, 1, 1, 0, None, FAKE, 16, None, None, P(0x200000), None, FAKE, None) == 3
    assert fq(0, 0, FAKE, 1, 1, 256, None, FAKE, 16, None, None, P(0x200008), None, FAKE, None) == 8
    # the decoded values may not overlap the weights (checked before any device access)
    assert fq(0, 0, FAKE, 1, 2, 256, None, FAKE, 16, None, None, P(0x100400), None, FAKE, None) == 8
    assert fq(0, 0, FAKE, 1, 1, 256, None, FAKE, 16, None, None, FAKE, None, FAKE, None) == 8
    # overlap is judged on the weight's own size: one fp64 row spans 2 KiB
    assert fq(0, 3, FAKE, 1, 1, 256, None, FAKE, 16, None, None, P(0x100400), None, FAKE, None) == 8
    assert fq(2, 9, FAKE, 1, 1, 256, None, FAKE, 16, None, None, P(0x200000), None, FAKE, None) == 8


def test_batched_search_argument_errors_need_no_gpu(lib):
    cs = lib.iq_choice_search_blocks
    # H, cand, rows, nblk, G, C, sweeps, picks, trace, stream
    assert cs(FAKE, FAKE, 4, 0, 16, 8, 2, FAKE, None, None) == 3
    assert cs(FAKE, FAKE, 4, 65536, 16, 8, 2, FAKE, None, None) == 3
    assert cs(FAKE, FAKE, 0, 3, 16, 8, 2, FAKE, None, None) == 3
    assert cs(FAKE, FAKE, 4, 3, 4, 8, 2, FAKE, None, None) == 8
    assert cs(FAKE, None, 4, 3, 8, 8, 2, FAKE, None, None) == 1
    # the candidate vectors are read as 16-byte words
    assert cs(FAKE, P(0x100004), 4, 3, 16, 8, 2, FAKE, None, None) == 8


def _no_device_visible():
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_device_visible(),
                    reason="reaches the device check; with a GPU present it would launch on "
                           "placeholder pointers")
def test_null_status_is_an_argument_the_calls_accept(lib):
    # A NULL status asks the call to synchronize and return the data error
    # itself, so it is not IQ_ERR_NULL: argument errors still come first, and a
    # call with valid arguments goes on to the device check, which fails here
    # for want of a GPU (IQ_ERR_HIP or IQ_ERR_DEVICE), before any launch.
    enc = lib.iq_encode
    assert enc(0, 0, FAKE, 1, 1, 200, None, FAKE, 16, None, None, FAKE, None, None) == 3
    assert enc(0, 0, FAKE, 1, 1, 256, None, FAKE, 16, None, None, None, None, None) == 1
    assert enc(0, 0, FAKE, 1, 1, 256, None, FAKE, 16, None, None, FAKE, None, None) in (10, 11)
    ev = lib.iq_encode_every_choice
    assert ev(0, 0, FAKE, 1, 1, 256, None, FAKE, 16, None, FAKE, None, None) in (10, 11)
    fq = lib.iq_fake_quant
    assert fq(0, 0, FAKE, 1, 1, 256, None, FAKE, 16, None, None, P(0x200000), None, None,
              None) in (10, 11)
    assert lib.iq_dequant(0, FAKE, 1, 1, 256, FAKE, 16, FAKE, None, None) in (10, 11)
    assert lib.iq_dequant(0, FAKE, 1, 1, 256, FAKE, 16, P(0x200008), None, None) == 8
    cand = lib.iq_encode_candidates
    assert cand(1, 0, FAKE, 1, 256, None, FAKE, 16, 8, FAKE, FAKE, None, None, None) in (10, 11)
    # a misaligned status word is still rejected
    assert enc(0, 0, FAKE, 1, 1, 256, None, FAKE, 16, None, None, FAKE, P(0x300002), None) == 8
