"""Mutation check of the oracle's pins: each case plants one plausible mistake
in a copy of oracle/iq_oracle.c (a dropped term, a flipped sign, a wrong
index or constant, a reversed comparison), builds it, and runs the pin suite
(tests/test_oracle_pins.py) against it in a subprocess; some pin must fail.
An unmodified copy built the same way must pass every pin.  CPU only."""

import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "iq_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# name: (text in iq_oracle.c, which occurrence (0-based), replacement)
MUTANTS = {
    "iq1s_error_drops_importance": ("e += (w ? (double)w[j] : 1.0) * r * r;", 0, "e += r * r;"),
    "iq2xs_error_drops_importance": ("e += (w ? (double)w[j] : 1.0) * r * r;", 1, "e += r * r;"),
    "iq1s_delta_sign_flipped": ("double delta = dbit ? -0.125 : 0.125;", 0,
                                "double delta = dbit ? 0.125 : -0.125;"),
    "iq1s_local_scale_even": ("double s = d * (double)(2 * k + 1);", 0,
                              "double s = d * (double)(2 * k + 2);"),
    "iq1s_entry_tie_to_highest": ("if (v < be) { be = v; best = e; }", 0,
                                  "if (v <= be) { be = v; best = e; }"),
    "iq1s_choice_tie_to_highest": ("if (cost < best_cost) {", 0, "if (cost <= best_cost) {"),
    "iq2xs_weakest_is_strongest": ("if (weak < best) { best = weak; jw = j; }", 0,
                                   "if (weak > best || j == 0) { best = weak; jw = j; }"),
    "iq2xs_flip_on_even_count": ("if (cnt & 1) {", 0, "if (!(cnt & 1)) {"),
    "iq2xs_mask_shifted": ("if (j < 7 && neg[j]) mask |= 1 << j;", 0,
                           "if (j < 7 && neg[j]) mask |= 1 << (6 - j);"),
    "scale_anchor_changed": ("#define SCALE_ANCHOR 0.61f", 0, "#define SCALE_ANCHOR 0.6f"),
    "iq2xs_divisor_changed": ("#define IQ2XS_DIVISOR 155.0f", 0, "#define IQ2XS_DIVISOR 150.0f"),
    "iq1s_decode_high_bits_misplaced": ("(((qh >> (3 * l)) & 7) << 8)", 0, "(((qh >> (3 * l)) & 7) << 7)"),
    "iq2xs_decode_nibbles_swapped": ("int k = (m & 1) ? (blk[66 + m / 2] >> 4) : (blk[66 + m / 2] & 15);", 0,
                                     "int k = (m & 1) ? (blk[66 + m / 2] & 15) : (blk[66 + m / 2] >> 4);"),
    "iq1m_anchor_offset_changed": ("volatile float a = 0.58f + t;", 0, "volatile float a = 0.6f + t;"),
    "iq1m_d_nibbles_reversed": ("((sc[wd] >> 12) << (4 * wd))", 0, "((sc[wd] >> 12) << (4 * (3 - wd)))"),
    "iq2xs_candidates_reverse_order": ("if (kb < 0 || cost[k] < cost[kb]) kb = k;", 1,
                                       "if (kb < 0 || cost[k] > cost[kb]) kb = k;"),
    "search_score_drops_factor_two": ("score[c] = Q[g * C + c] + 2.0 * dot;", 0,
                                      "score[c] = Q[g * C + c] + dot;"),
    "search_moves_on_ties": ("if (score[best] < score[p[g]]) {", 0, "if (score[best] <= score[p[g]]) {"),
}


def _mutated(text, occ, new):
    src = open(SRC).read()
    at = -1
    for _ in range(occ + 1):
        at = src.index(text, at + 1)
    return src[:at] + new + src[at + len(text):]


def _build(src_text, tmp_path, name):
    c = tmp_path / (name + ".c")
    so = tmp_path / (name + ".so")
    c.write_text(src_text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                           "-fno-fast-math", "-fPIC", "-shared", str(c), "-o", str(so), "-lm"])
    return str(so)


def _run_pins(so):
    env = dict(os.environ, IQ_ORACLE_LIB=so, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    return r.returncode, r.stdout[-2000:]


def test_every_mutant_is_caught_and_the_control_passes(tmp_path):
    for name, (text, occ, new) in MUTANTS.items():
        assert open(SRC).read().count(text) > occ, "mutation target missing: %s" % name
    jobs = {"control": _build(open(SRC).read(), tmp_path, "control")}
    for name, (text, occ, new) in MUTANTS.items():
        jobs[name] = _build(_mutated(text, occ, new), tmp_path, name)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        res = dict(zip(jobs, ex.map(_run_pins, jobs.values())))
    rc, out = res.pop("control")
    assert rc == 0, "the unmodified oracle fails its pins:\n" + out
    missed = [n for n, (rc, _) in res.items() if rc == 0]
    assert not missed, "mutants no pin catches: %s" % missed
