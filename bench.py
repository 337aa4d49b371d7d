#!/usr/bin/env python3
"""Benchmark of the importance-weighted IQ1_S encode on one MI355X.

A step is one call of the encode (scale prediction, grid staging, the
exhaustive candidate scoring over the 2048-entry grid, the argmin reductions
and the bit-packing, all in one kernel) over the 4096 x 4096 fp32 weight with
per-column lognormal importance.  Inputs are resident in HBM before the timed
region.  The JSON line carries:

* value: fp32 input bytes encoded per second (GB/s), whole job;
* roofline: for the encode kernel, its average launch time (HIP events on the
  launch stream) against the two bounds of the search's arithmetic -- the
  elementwise part (the 16 choice keys and the shift terms, fp32) at the
  MI355X FP32 vector peak, and the dot products (a contraction) at the bf16
  matrix-core peak -- whose larger time is the kernel's bound; `frac` is the
  elementwise part's achieved rate over the FP32 vector peak (that part sets
  the bound), `mfma` the contraction's over the matrix-core peak.  The VALU
  issue and matrix-core busy fractions, and the HBM traffic, come from the
  committed rocprofv3 counter summaries when they were taken on the current
  kernel source;
* cpu_baseline: the CPU oracle timed on the whole workload on this host's
  cores (with the host's CPU model and core count).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2|c1|c3|...]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Algorithmic work of the exhaustive search per (8-value group, grid entry),
# counted once (FMA = 2 flops, compares excluded), split into the contraction
# (the weighted dot products over the group's 8 values, a [entries x 8] by
# [8 x groups] product) and the elementwise rest (the shift terms that turn
# the dot products into U(+-1/8) and V(+-1/8), and the 16 choice keys, one FMA
# each):
#   IQ1_S weighted: 3 dot products of 8 (48) + shift terms (10) + 16 keys (32) = 90;
#   IQ1_S unweighted: the entry norms do not depend on the group: 1 dot product
#   (16) + 10 + 32 = 58;
#   IQ2_XS weighted: 2 dot products (32) + 1 + 16 keys (32) = 65;
#   IQ1_M: the IQ1_S search (16 (k, shift) keys per group and entry).
CONTRACTION_FLOPS = {("iq1_s", True): 48, ("iq1_s", False): 16, ("iq2_xs", True): 32,
                     ("iq2_xs", False): 32, ("iq1_m", True): 48, ("iq1_m", False): 16}
ELEMENTWISE_FLOPS = {("iq1_s", True): 42, ("iq1_s", False): 42, ("iq2_xs", True): 33,
                     ("iq2_xs", False): 33, ("iq1_m", True): 42, ("iq1_m", False): 42}
FLOPS_PER_GROUP_ENTRY = {k: CONTRACTION_FLOPS[k] + ELEMENTWISE_FLOPS[k] for k in CONTRACTION_FLOPS}

# MI355X published peaks.  FP32 vector: 256 CU x 4 SIMD x 16 lanes x 2 (FMA) x 2
# x 2.4 GHz; the last factor 2 is packed FP32 or the dual issue of two VALU
# instructions from different waves; this library is built without packed
# FP32, so dual issue is the only way to it.  bf16 dense matrix cores:
# 2.5 PFLOP/s.  HBM3E: 8 TB/s.
PEAK_FP32_VECTOR_TFLOPS = 157.3
PEAK_BF16_MFMA_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0

WORKLOADS = {
    "c1": ("c1_iq1s_small", "IQ1_S encode of one 64x256 fp32 weight, uniform importance, "
                            "seeded 2048x8 ternary grid"),
    "c2": ("c2_iq1s_4096", "IQ1_S weighted encode of a 4096x4096 fp32 weight, N(0,0.02), "
                           "per-column sqrt-lognormal importance, seeded 2048x8 ternary grid"),
    "c3": ("c3_iq2xs_4096", "IQ2_XS weighted encode of a 4096x4096 fp32 weight, 0.02*t5, "
                            "per-column sqrt-lognormal importance, seeded 512x8 {1,3,5} grid"),
    "c4": ("c4_moe_batch", "IQ1_S weighted encode of 16 expert weights of 1536x4096 fp32 in one "
                           "batched call, per-expert importance"),
    "c5": ("c5_choice_search", "IQ2_XS top-8 candidate encode + local-Hessian choice search, "
                               "4096 rows x one 256-column block, 2 sweeps"),
    "c5_iq1s": ("c5_iq1s_choice_search", "IQ1_S top-8 candidate encode + local-Hessian choice "
                                         "search (G=8), 4096 rows x one 256-column block, 2 sweeps"),
    "c5_weight": ("c5_weight_choice_search", "IQ2_XS top-8 candidate encode + local-Hessian choice "
                                             "search of a whole 4096x4096 weight: 16 blocks, one H "
                                             "each, searched in one launch, 2 sweeps"),
    # The same IQ1_S 4096x4096 weighted workload through the other encode outputs.
    "c2_every": ("c2_iq1s_4096", "IQ1_S weighted every-choice encode (16 payloads from one sweep) "
                                 "of a 4096x4096 fp32 weight"),
    "c2_fake": ("c2_iq1s_4096", "IQ1_S weighted fused encode+decode (fake quant, fp32 out) of a "
                                "4096x4096 fp32 weight"),
    "c2_pinned": ("c2_iq1s_4096", "IQ1_S weighted re-encode of a 4096x4096 fp32 weight under "
                                  "pinned super-block scales"),
    "c2_iq1m": ("c2_iq1m_4096", "IQ1_M weighted encode of a 4096x4096 fp32 weight, N(0,0.02), "
                                "per-column sqrt-lognormal importance, seeded 2048x8 ternary grid"),
    # Decode of the payloads the c2 and c3 encodes write (HBM-bound).
    "c2_dequant": ("c2_iq1s_4096", "IQ1_S decode of the 4096x4096 weighted encode's payload "
                                   "(3.28 MB) to fp32 (67.1 MB)"),
    "c3_dequant": ("c3_iq2xs_4096", "IQ2_XS decode of the 4096x4096 weighted encode's payload "
                                    "(4.85 MB) to fp32 (67.1 MB)"),
}

KERNEL_SOURCES = {
    "iq1_s": ["ggml_iq_codebook_amd/csrc/iq1s_encode.hip",
              "ggml_iq_codebook_amd/csrc/device_common.hpp"],
    "iq1_m": ["ggml_iq_codebook_amd/csrc/iq1s_encode.hip",
              "ggml_iq_codebook_amd/csrc/device_common.hpp"],
    "iq2_xs": ["ggml_iq_codebook_amd/csrc/iq2xs_encode.hip",
               "ggml_iq_codebook_amd/csrc/device_common.hpp"],
}
KERNEL_NAMES = {"iq1_s": "iq1s_payload_wide_kernel<0, 0, 0>", "iq2_xs": "iq2xs_wide_kernel<0, 0>",
                "iq1_m": "iq1s_payload_wide_kernel<2, 0, 0>"}
DEQUANT_KERNELS = {"iq1_s": "dequant_iq1s_kernel", "iq2_xs": "dequant_iq2xs_kernel",
                   "iq1_m": "dequant_iq1m_kernel"}
DEQUANT_SOURCES = ["ggml_iq_codebook_amd/csrc/dequant.hip",
                   "ggml_iq_codebook_amd/csrc/device_common.hpp"]
SEARCH_SOURCES = ["ggml_iq_codebook_amd/csrc/choice_search.hip",
                  "ggml_iq_codebook_amd/csrc/device_common.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(rels):
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_mean(csv_path, kernel_substr, counter):
    """Mean per-dispatch value of a rocprofv3 counter for the matching kernel."""
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit("no %s samples for %s in %s" % (counter, kernel_substr, csv_path))
    return sum(vals) / len(vals), len(vals)


CONFIG_FMT = {"c1": "iq1_s", "c2": "iq1_s", "c3": "iq2_xs", "c4": "iq1_s", "c5": "iq2_xs",
              "c5_iq1s": "iq1_s", "c5_weight": "iq2_xs", "c2_every": "iq1_s", "c2_fake": "iq1_s",
              "c2_pinned": "iq1_s", "c2_iq1m": "iq1_m", "c2_dequant": "iq1_s",
              "c3_dequant": "iq2_xs"}

# The kernel each workload's counters and traffic records belong to (the
# dominant kernel of its step): (record name, kernel name, sources).
_IQ1 = KERNEL_SOURCES["iq1_s"]
_IQ2 = KERNEL_SOURCES["iq2_xs"]
PROFILED = {
    "c1": ("iq1s_encode_c1", KERNEL_NAMES["iq1_s"], _IQ1),
    "c2": ("iq1s_encode_c2", KERNEL_NAMES["iq1_s"], _IQ1),
    "c3": ("iq2xs_encode_c3", KERNEL_NAMES["iq2_xs"], _IQ2),
    "c4": ("iq1s_encode_c4", KERNEL_NAMES["iq1_s"], _IQ1),
    "c2_pinned": ("iq1s_encode_c2_pinned", KERNEL_NAMES["iq1_s"], _IQ1),
    "c2_iq1m": ("iq1m_encode_c2_iq1m", KERNEL_NAMES["iq1_m"], _IQ1),
    "c2_every": ("iq1s_every_c2", "iq1s_payload_wide_kernel<0, 1, 0>", _IQ1),
    "c2_fake": ("iq1s_fake_c2", "iq1s_payload_wide_kernel<0, 2, 0>", _IQ1),
    "c5": ("iq2xs_candidates_c5", "iq2xs_wide_kernel<3, 0>", _IQ2),
    "c5_iq1s": ("iq1s_candidates_c5_iq1s", "iq1s_payload_wide_kernel<0, 3, 0>", _IQ1),
    "c5_weight": ("iq2xs_candidates_c5_weight", "iq2xs_wide_kernel<3, 0>", _IQ2),
    "c2_dequant": ("dequant_iq1s_c2", DEQUANT_KERNELS["iq1_s"], DEQUANT_SOURCES),
    "c3_dequant": ("dequant_iq2xs_c3", DEQUANT_KERNELS["iq2_xs"], DEQUANT_SOURCES),
}


# The choice search of the candidate workloads, recorded beside the candidate
# encode: (record name, kernel name, sources).
PROFILED_SEARCH = {
    "c5": ("choice_search_c5", "choice_search_kernel<16>", SEARCH_SOURCES),
    "c5_iq1s": ("choice_search_c5_iq1s", "choice_search_kernel<32>", SEARCH_SOURCES),
    "c5_weight": ("choice_search_c5_weight", "choice_search_kernel<16>", SEARCH_SOURCES),
}


def profiled_kernel(config):
    """(record name, kernel name, kernel sources) of the kernel a workload's
    counters and traffic belong to."""
    return PROFILED[config]


def _pmc_csv(pmc_dir, config, what):
    # pmc_<config>_<what>/ if present, else pmc_<what>/ (the c2 run)
    for d in ("pmc_%s_%s" % (config, what), "pmc_%s" % what):
        path = os.path.join(pmc_dir, d, "enc_counter_collection.csv")
        if os.path.exists(path):
            return path
    raise SystemExit("no %s counter run under %s" % (what, pmc_dir))


def record_traffic(config, pmc_dir, which=None):
    """Turn the FETCH_SIZE / WRITE_SIZE counter runs of a workload's kernel and
    of a plain 256 MiB copy into HBM bytes per launch, written to
    profiles/traffic_<kernel>_<config>.json.

    pmc_dir holds pmc_<config>_FETCH_SIZE/enc_counter_collection.csv and
    pmc_<config>_WRITE_SIZE/... (or pmc_FETCH_SIZE/... for c2) and the copy runs
    pmc_copy_FETCH_SIZE/copy_counter_collection.csv, pmc_copy_WRITE_SIZE/...
    The copy reads and writes exactly 268435456 bytes; each counter is scaled by
    known bytes / (counted KiB * 1024) of that copy."""
    name, kernel, sources = which or profiled_kernel(config)
    kname = kernel.split("<")[0]
    known = 64 * 1024 * 1024 * 4
    f_enc, nf = _counter_mean(_pmc_csv(pmc_dir, config, "FETCH_SIZE"), kname, "FETCH_SIZE")
    w_enc, nw = _counter_mean(_pmc_csv(pmc_dir, config, "WRITE_SIZE"), kname, "WRITE_SIZE")
    f_cp, _ = _counter_mean(os.path.join(pmc_dir, "pmc_copy_FETCH_SIZE", "copy_counter_collection.csv"),
                            "copyBuffer", "FETCH_SIZE")
    w_cp, _ = _counter_mean(os.path.join(pmc_dir, "pmc_copy_WRITE_SIZE", "copy_counter_collection.csv"),
                            "copyBuffer", "WRITE_SIZE")
    ff, wf = known / (f_cp * 1024), known / (w_cp * 1024)
    rec = {
        "kernel": kernel,
        "kernel_source_sha": source_sha(sources),
        "fetch_kib_per_launch": f_enc, "fetch_dispatches": nf,
        "write_kib_per_launch": w_enc, "write_dispatches": nw,
        "copy_known_bytes": known, "copy_fetch_kib": f_cp, "copy_write_kib": w_cp,
        "fetch_scale": ff, "write_scale": wf,
        "hbm_bytes_per_launch": int(round(f_enc * 1024 * ff + w_enc * 1024 * wf)),
    }
    out = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


# The VALU / matrix-core / LDS counters of one rocprofv3 pass (8 SQ counters
# and 2 GRBM counters at most per pass on this GPU).
VALU_COUNTERS = ["SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU2", "SQ_INSTS_MFMA",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS", "SQ_BUSY_CYCLES",
                 "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"]
N_XCD, N_CU, N_SIMD = 8, 256, 1024


def record_counters(config, pmc_dir, units, which=None):
    """Turn a VALU counter pass (pmc_<config>_valu/enc_counter_collection.csv)
    into profiles/counters_<kernel>_<config>.json: the VALU issue-port busy
    fraction (quad-cycles with at least one VALU issue per SIMD over the
    kernel's quad-cycles; a dual issue puts two instructions in one), the
    dual-issued share, the matrix-core busy fraction, the share of the
    kernel's cycles an LDS (one per CU) is stalled on bank conflicts, and the
    VALU lane-instructions per (group, entry)."""
    name, kernel, sources = which or profiled_kernel(config)
    kname = kernel.split("<")[0]
    path = _pmc_csv(pmc_dir, config, "valu")
    v = {c: _counter_mean(path, kname, c)[0] for c in VALU_COUNTERS}
    cycles = v["GRBM_GUI_ACTIVE"] / N_XCD
    issue_quads = (v["SQ_INSTS_VALU"] - v["SQ_ACTIVE_INST_VALU2"]) / N_SIMD
    rec = {
        "kernel": kernel,
        "kernel_source_sha": source_sha(sources),
        "counters_per_dispatch": v,
        "kernel_cycles_per_xcd": cycles,
        "valu_issue_busy": issue_quads / (cycles / 4.0),
        "dual_issued_share": 2.0 * v["SQ_ACTIVE_INST_VALU2"] / v["SQ_INSTS_VALU"],
        "mfma_busy": v["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * cycles),
        "lds_conflict_share": v["SQ_LDS_BANK_CONFLICT"] / (N_CU * cycles),
        "valu_lane_instr_per_unit": (v["SQ_INSTS_VALU"] * 64 / units) if units else None,
        "units_per_launch": units,
    }
    out = os.path.join(ROOT, "profiles", "counters_%s.json" % name)
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def _profile_record(kind, name, sha):
    """A committed counter record (kind "traffic" or "counters"), if it was
    taken on this kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "%s_%s.json" % (kind, name))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != sha:
        return None
    return t


def traffic_for(name, sha):
    t = _profile_record("traffic", name, sha)
    return None if t is None else t.get("hbm_bytes_per_launch")


def counters_for(name, sha):
    t = _profile_record("counters", name, sha)
    if t is None:
        return None
    return {k: round(t[k], 4) if isinstance(t[k], float) else t[k]
            for k in ("valu_issue_busy", "dual_issued_share", "mfma_busy",
                      "lds_conflict_share", "valu_lane_instr_per_unit") if k in t}


def host_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_usable": affinity}


def cpu_baseline(cfg, fmt, full_budget_s=45.0, sample_s=20.0):
    """The oracle on this host's cores: the whole workload when a short trial
    predicts it finishes within full_budget_s, else its first rows, sized to
    about sample_s."""
    import oracle
    w, grid, imp = cfg["w"], cfg["grid"], cfg["importance"]
    threads = oracle.num_threads()
    B, R, C = w.shape
    trial = min(R, 32)
    t0 = time.perf_counter()
    oracle.encode(fmt, w[:1, :trial], grid, None if imp is None else imp[:1])
    rate = trial * C / max(time.perf_counter() - t0, 1e-6)          # values per second
    if w.size / rate <= full_budget_s:
        sub, ims, what = w, imp, "the whole workload"
    else:
        rows = max(1, min(R, int(sample_s * rate / C)))
        sub, ims = w[:1, :rows], None if imp is None else imp[:1]
        what = "the first %d rows x %d cols of the workload" % (rows, C)
    t0 = time.perf_counter()
    oracle.encode(fmt, sub, grid, ims)
    dt = time.perf_counter() - t0
    rec = {"value": sub.size * 4 / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": "%s (%d blocks), %.1f s" % (what, sub.size // 256, dt)}
    rec.update(host_info())
    return rec


def search_flops_per_row(G, C, sweeps):
    """Algorithmic fp32 flops of the choice search of one row of one 256-column
    block: r = H e, step 2's e^T H_gg e for every candidate, and per sweep and
    group the rest r_g - H_gg e_cur, one dot product per candidate and the
    update r += H[:, g] (e_new - e_cur)."""
    L = 256 // G
    step2 = G * C * (2 * L * L + 2 * L)
    sweep = G * (2 * L * L + C * 2 * L + 2 * 256 * L)
    return 2 * 256 * 256 + step2 + sweeps * sweep


def encode_roofline(fmt, weighted, units, kernel_ms, alg_bytes, config):
    """The roofline record of an encode-type kernel: `units` (group, grid
    entry) pairs per launch, `alg_bytes` algorithmic HBM bytes per launch."""
    name, kernel, sources = profiled_kernel(config)
    sha = source_sha(sources)
    t = kernel_ms * 1e-3
    con = CONTRACTION_FLOPS[(fmt, weighted)] * units
    ele = ELEMENTWISE_FLOPS[(fmt, weighted)] * units
    bound = {"fp32_vector_ms": round(ele / (PEAK_FP32_VECTOR_TFLOPS * 1e12) * 1e3, 5),
             "bf16_mfma_ms": round(con / (PEAK_BF16_MFMA_TFLOPS * 1e12) * 1e3, 5),
             "hbm_ms": round(alg_bytes / (PEAK_HBM_GBPS * 1e9) * 1e3, 5)}
    achieved = ele / t / 1e12
    return {
        "bound": "alu",
        "achieved": round(achieved, 3),
        "peak": PEAK_FP32_VECTOR_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_FP32_VECTOR_TFLOPS, 4),
        "traffic": traffic_for(name, sha),
        "kernel": kernel,
        "kernel_ms": round(kernel_ms, 5),
        "work": ("elementwise fp32 flops of the search (16 choice keys + shift terms): %d per "
                 "(group, grid entry) x %d pairs" % (ELEMENTWISE_FLOPS[(fmt, weighted)], units)),
        "mfma": {"achieved": round(con / t / 1e12, 3), "peak": PEAK_BF16_MFMA_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(con / t / 1e12 / PEAK_BF16_MFMA_TFLOPS, 4),
                 "work": "contraction flops (weighted dot products): %d per pair"
                         % CONTRACTION_FLOPS[(fmt, weighted)]},
        "bound_ms": bound,
        "frac_of_bound": round(max(bound.values()) / kernel_ms, 4),
        "algorithmic_flops_per_launch": con + ele,
        "algorithmic_bytes_per_launch": alg_bytes,
        "counters": counters_for(name, sha),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 200 for the decode workloads, whose "
                         "launches take about 15 us)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 10 and at least 1 s of them, "
                         "so the clocks have settled; the count run is reported)")
    ap.add_argument("--config", default="c2", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 256 MiB device copy (for counter calibration) and exit")
    ap.add_argument("--record-traffic", metavar="PMC_DIR",
                    help="convert the FETCH_SIZE / WRITE_SIZE counter CSVs of --config under "
                         "PMC_DIR into profiles/traffic_<kernel>_<config>.json and exit "
                         "(no GPU needed)")
    ap.add_argument("--record-counters", metavar="PMC_DIR",
                    help="convert the VALU counter CSV of --config under PMC_DIR into "
                         "profiles/counters_<kernel>_<config>.json and exit (no GPU needed)")
    args = ap.parse_args()

    if args.steps is None:
        args.steps = 200 if args.config.endswith("_dequant") else 20
    if args.record_traffic:
        record_traffic(args.config, args.record_traffic)
        if args.config in PROFILED_SEARCH:
            record_traffic(args.config, args.record_traffic, PROFILED_SEARCH[args.config])
        return
    if args.record_counters:
        import workloads
        cfg = getattr(workloads, WORKLOADS[args.config][0])()
        units = None
        if not args.config.endswith("_dequant"):
            units = cfg["w"].size // 8 * cfg["grid"].shape[0]
        record_counters(args.config, args.record_counters, units)
        if args.config in PROFILED_SEARCH:
            record_counters(args.config, args.record_counters, None,
                            PROFILED_SEARCH[args.config])
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the encode shards by rows/experts with no "
              "exchange, and it is measured here on a single MI355X (--gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import ggml_iq_codebook_amd as iq

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        n = 64 * 1024 * 1024
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: %d bytes read, %d bytes written per copy" % (n * 4, n * 4))
        return

    iq.load(build_if_missing=True)
    fn, desc = WORKLOADS[args.config]
    cfg = getattr(workloads, fn)()
    fmt = cfg["fmt"]
    grid = torch.from_numpy(cfg["grid"]).to(dev)
    w_np = cfg["w"]
    w = torch.from_numpy(w_np).to(dev)
    imp = None if cfg["importance"] is None else torch.from_numpy(cfg["importance"]).to(dev)
    stream = torch.cuda.current_stream()
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    dequant = args.config.endswith("_dequant")

    if args.config.startswith("c5"):
        H = torch.from_numpy(cfg["H"]).to(dev)
        w2 = w[0].contiguous()
        imp2 = imp[0].contiguous()
        G = iq.CHOICE_GROUPS[fmt]
        R, C = w2.shape
        shape = (R, G, 8, 256 // G) if H.dim() == 2 else (R, C // 256, G, 8, 256 // G)

        def step():
            err, ch, _ = iq.encode_candidates(w2, grid, imp2, fmt=fmt, top_c=8, status=status,
                                              check=False)
            iq.choice_search(H, err.view(shape), sweeps=2)
    elif dequant:
        B, R, C = w.shape
        # the payload of the workload's encode, decoded once per step
        packed = iq.encode(w, grid, imp, fmt=fmt)
        xhat = torch.empty_like(w)

        def step():
            iq.dequant(packed, grid, fmt=fmt, out=xhat, status=status, check=False)
    elif args.config.endswith("_every"):
        B, R, C = w.shape
        out = torch.empty((16, B, R, C // 256, iq.BLOCK_BYTES[fmt]), dtype=torch.uint8, device=dev)

        def step():
            iq.encode_every_choice(w, grid, imp, fmt=fmt, out=out, status=status, check=False)
    elif args.config.endswith("_fake"):
        xhat = torch.empty_like(w)

        def step():
            iq.fake_quant(w, grid, imp, fmt=fmt, out=xhat, status=status, check=False)
    else:
        B, R, C = w.shape
        out = torch.empty((B, R, C // 256, iq.BLOCK_BYTES[fmt]), dtype=torch.uint8, device=dev)
        scales = None
        if args.config.endswith("_pinned"):
            # the scales a previous encode chose, as a QAD re-encode pins them
            iq.encode(w, grid, imp, fmt=fmt, out=out)
            o = out.view(-1, iq.BLOCK_BYTES[fmt])
            scales = (o[:, 0].to(torch.int32) | (o[:, 1].to(torch.int32) << 8)).to(torch.int16)
            scales = scales.view(B, R, C // 256).contiguous()

        def step():
            iq.encode(w, grid, imp, fmt=fmt, scales=scales, out=out, status=status, check=False)

    if args.warmup is None:
        nwarm, tw = 0, time.perf_counter()
        while nwarm < 10 or time.perf_counter() - tw < 1.0:
            step()
            nwarm += 1
            if nwarm % 10 == 0:
                torch.cuda.synchronize()
        args.warmup = nwarm
    else:
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise SystemExit("the library reported status %d" % int(status.item()))

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Whole-step time from the host clock between the two synchronizations; the
    # kernel's per-launch time from HIP events on its launch stream (one launch
    # per step outside the c5 workloads).
    ms_per_step = 1e3 * wall / args.steps
    kernel_ms = ev0.elapsed_time(ev1) / args.steps

    nweights = w_np.size
    nblk = nweights // 256
    value = nweights * 4 / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": "weights encoded/sec (GB/s fp32 in) + % FP32/MFMA roofline, IQ1_S 4096x4096",
        "value": round(value, 4),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": desc, "config": args.config, "rows": int(w_np.shape[-2]),
                   "cols": int(w_np.shape[-1]), "batch": int(w_np.shape[0]),
                   "weights_per_sec": round(nweights / (ms_per_step * 1e-3), 1)},
    }
    if dequant:
        name, kernel, sources = profiled_kernel(args.config)
        alg = nblk * (iq.BLOCK_BYTES[fmt] + 256 * 4)
        achieved = alg / (kernel_ms * 1e-3) / 1e9
        result["metric"] = "weights decoded/sec (GB/s fp32 out), %s 4096x4096" % fmt.upper()
        result["value"] = round(nweights * 4 / (ms_per_step * 1e-3) / 1e9, 4)
        result["roofline"] = {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic_for(name, source_sha(sources)),
            "kernel": kernel, "kernel_ms": round(kernel_ms, 5),
            "work": "payload read + fp32 values written: %d bytes per 256-value block x %d blocks"
                    % (iq.BLOCK_BYTES[fmt] + 1024, nblk),
            "algorithmic_bytes_per_launch": alg,
        }
    elif args.config.startswith("c5"):
        # Per-kernel times, after the timed region (so that it is not
        # perturbed): HIP events on the launch stream around `steps`
        # back-to-back launches of each kernel alone (an event pair around
        # every launch adds several microseconds to kernels this short).  The
        # candidate encode, the dominant kernel, carries the roofline (the
        # same sweep as the encode, so the same algorithmic flops per group
        # and entry); the choice search is reported beside it against its own
        # bounds.
        err0, _, _ = iq.encode_candidates(w2, grid, imp2, fmt=fmt, top_c=8, status=status,
                                          check=False)
        cand_in = err0.view(shape)

        def per_launch(fn):
            fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps

        cand_ms = per_launch(lambda: iq.encode_candidates(w2, grid, imp2, fmt=fmt, top_c=8,
                                                          status=status, check=False))
        search_ms = per_launch(lambda: iq.choice_search(H, cand_in, sweeps=2))
        units = w2.numel() // 8 * cfg["grid"].shape[0]
        # candidates written: [rows][blocks][G][8][256/G] fp32 + choices int32
        cand_bytes = R * (C // 256) * (G * 8 * (256 // G) * 4 + G * 8 * 4)
        roof = encode_roofline(fmt, True, units, cand_ms, w2.numel() * 4 + cand_bytes,
                               args.config)
        nsearch = R * (C // 256)
        sflops = nsearch * search_flops_per_row(G, 8, 2)
        sbytes = cand_bytes + H.numel() * 4 + nsearch * G * 4
        sb = {"fp32_ms": round(sflops / (PEAK_FP32_VECTOR_TFLOPS * 1e12) * 1e3, 5),
              "hbm_ms": round(sbytes / (PEAK_HBM_GBPS * 1e9) * 1e3, 5)}
        sname, skernel, ssrc = PROFILED_SEARCH[args.config]
        roof["search"] = {"kernel": skernel, "kernel_ms": round(search_ms, 5),
                          "algorithmic_flops": sflops,
                          "algorithmic_bytes": sbytes, "bound_ms": sb,
                          "frac_of_bound": round(max(sb.values()) / search_ms, 4),
                          "traffic": traffic_for(sname, source_sha(ssrc)),
                          "counters": counters_for(sname, source_sha(ssrc))}
        result["roofline"] = roof
    else:
        weighted = imp is not None
        units = nweights // 8 * cfg["grid"].shape[0]
        mult = 16 if args.config.endswith("_every") else 1
        out_bytes = nblk * (256 * 4 if args.config.endswith("_fake")
                            else mult * iq.BLOCK_BYTES[fmt])
        alg_bytes = nweights * 4 + out_bytes + (0 if imp is None else imp.numel() * 4)
        result["roofline"] = encode_roofline(fmt, weighted, units, kernel_ms, alg_bytes,
                                             args.config)
    if not args.no_cpu_baseline and args.config in ("c1", "c2", "c3", "c4"):
        result["cpu_baseline"] = cpu_baseline(cfg, fmt)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
