#!/usr/bin/env python3
"""Benchmark of the importance-weighted IQ1_S encode on one MI355X.

A step is one call of the encode (scale prediction, grid staging, the
exhaustive candidate scoring over the 2048-entry grid, the argmin reductions
and the bit-packing, all in one kernel) over the 4096 x 4096 fp32 weight with
per-column lognormal importance.  Inputs are resident in HBM before the timed
region.  The JSON line carries:

* value: fp32 input bytes encoded per second (GB/s), whole job;
* roofline: the encode kernel's algorithmic FP32 flops per launch divided by
  its average launch time (HIP events on the launch stream), against the
  MI355X FP32 vector peak, plus the HBM traffic of one launch from the
  committed rocprofv3 counter summary when it was taken on the current source;
* cpu_baseline: the CPU oracle timed on a bounded sample of the same workload
  on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2|c1|c3|c4|c5]
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

# Algorithmic FP32 work of the exhaustive search per (8-value group, grid entry),
# counted once (FMA = 2 flops, compares excluded):
#   IQ1_S weighted: 3 weighted dot products of 8 (48) + the delta terms of
#   U(+-1/8), V(+-1/8) (10) + 16 choice keys, one FMA each (32) = 90;
#   IQ1_S unweighted: the entry norms do not depend on the group (16 + 10 + 32) = 58;
#   IQ2_XS weighted: 2 dot products (32) + 1 + 16 keys (32) = 65;
#   IQ1_M: the IQ1_S search (16 (k, shift) keys per group and entry): 90 / 58.
FLOPS_PER_GROUP_ENTRY = {("iq1_s", True): 90, ("iq1_s", False): 58,
                         ("iq2_xs", True): 65, ("iq2_xs", False): 65,
                         ("iq1_m", True): 90, ("iq1_m", False): 58}

PEAK_FP32_VECTOR_TFLOPS = 157.3     # MI355X: 256 CU x 4 SIMD x 16 lanes x 2 (FMA) x 2 (packed) x 2.4 GHz
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
}

KERNEL_SOURCES = {
    "iq1_s": ["ggml_iq_codebook_amd/csrc/iq1s_encode.hip",
              "ggml_iq_codebook_amd/csrc/device_common.hpp"],
    "iq1_m": ["ggml_iq_codebook_amd/csrc/iq1s_encode.hip",
              "ggml_iq_codebook_amd/csrc/device_common.hpp"],
    "iq2_xs": ["ggml_iq_codebook_amd/csrc/iq2xs_encode.hip",
               "ggml_iq_codebook_amd/csrc/device_common.hpp"],
}
KERNEL_NAMES = {"iq1_s": "iq1s_payload_wide_kernel<0, 0, 0>", "iq2_xs": "iq2xs_payload_wide_kernel<0>",
                "iq1_m": "iq1s_payload_wide_kernel<2, 0, 0>"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(rels):
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_kib(csv_path, kernel_substr, counter):
    """Mean per-dispatch value of a rocprofv3 counter for the matching kernel."""
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit("no %s samples for %s in %s" % (counter, kernel_substr, csv_path))
    return sum(vals) / len(vals), len(vals)


def record_traffic(name, fmt, pmc_dir):
    """Turn the FETCH_SIZE / WRITE_SIZE counter runs of the encode and of a plain
    256 MiB copy into HBM bytes per launch, written to profiles/traffic_<name>.json.

    pmc_dir holds pmc_FETCH_SIZE/enc_counter_collection.csv and
    pmc_WRITE_SIZE/enc_counter_collection.csv (or pmc_<config>_FETCH_SIZE/...
    for a workload other than c2) and the copy runs
    pmc_copy_FETCH_SIZE/copy_counter_collection.csv, pmc_copy_WRITE_SIZE/...
    The copy reads and writes exactly 268435456 bytes; each counter is scaled by
    known bytes / (counted KiB * 1024) of that copy."""
    kname = KERNEL_NAMES[fmt].split("<")[0]
    known = 64 * 1024 * 1024 * 4
    cfg = name.rsplit("_", 1)[-1]

    def enc_csv(counter):
        # pmc_<config>_<COUNTER>/ if present, else pmc_<COUNTER>/ (the c2 run)
        for d in ("pmc_%s_%s" % (cfg, counter), "pmc_%s" % counter):
            path = os.path.join(pmc_dir, d, "enc_counter_collection.csv")
            if os.path.exists(path):
                return path
        raise SystemExit("no %s counter run under %s" % (counter, pmc_dir))

    f_enc, nf = _counter_kib(enc_csv("FETCH_SIZE"), kname, "FETCH_SIZE")
    w_enc, nw = _counter_kib(enc_csv("WRITE_SIZE"), kname, "WRITE_SIZE")
    f_cp, _ = _counter_kib(os.path.join(pmc_dir, "pmc_copy_FETCH_SIZE", "copy_counter_collection.csv"),
                           "copyBuffer", "FETCH_SIZE")
    w_cp, _ = _counter_kib(os.path.join(pmc_dir, "pmc_copy_WRITE_SIZE", "copy_counter_collection.csv"),
                           "copyBuffer", "WRITE_SIZE")
    ff, wf = known / (f_cp * 1024), known / (w_cp * 1024)
    rec = {
        "kernel": KERNEL_NAMES[fmt],
        "kernel_source_sha": source_sha(KERNEL_SOURCES[fmt]),
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


def traffic_for(name, sha):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on this kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != sha:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, fmt, budget_s=15.0):
    """The oracle on the first rows of the workload, on this host's cores."""
    import oracle
    w, grid, imp = cfg["w"], cfg["grid"], cfg["importance"]
    threads = oracle.num_threads()
    rows = 2
    while True:
        sub = w[:1, :rows, :]
        t0 = time.perf_counter()
        oracle.encode(fmt, sub, grid, None if imp is None else imp[:1])
        dt = time.perf_counter() - t0
        if dt >= 0.6 * budget_s or rows >= w.shape[1]:
            break
        rows = min(w.shape[1], max(rows * 2, int(rows * budget_s / max(dt, 1e-3))))
    nbytes = sub.size * 4
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "first %d rows x %d cols of the workload (%d blocks), %.1f s"
                      % (rows, w.shape[2], sub.size // 256, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 10 and at least 1 s of them, "
                         "so the clocks have settled; the count run is reported)")
    ap.add_argument("--config", default="c2", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 256 MiB device copy (for counter calibration) and exit")
    ap.add_argument("--record-traffic", metavar="PMC_DIR",
                    help="convert rocprofv3 counter CSVs under PMC_DIR into "
                         "profiles/traffic_<kernel>_<config>.json and exit (no GPU needed)")
    args = ap.parse_args()

    if args.record_traffic:
        fmt = "iq2_xs" if args.config == "c3" else "iq1_s"
        record_traffic("%s_encode_%s" % (fmt.replace("_", ""), args.config), fmt,
                       args.record_traffic)
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

    if args.config.startswith("c5"):
        H = torch.from_numpy(cfg["H"]).to(dev)
        w2 = w[0].contiguous()
        imp2 = imp[0].contiguous()
        G = iq.CHOICE_GROUPS[fmt]
        R, C = w2.shape
        shape = (R, G, 8, 256 // G) if H.dim() == 2 else (R, C // 256, G, 8, 256 // G)

        def step(ev=None):
            if ev:
                ev[0].record(stream)
            err, ch, _ = iq.encode_candidates(w2, grid, imp2, fmt=fmt, top_c=8, status=status,
                                              check=False)
            if ev:
                ev[1].record(stream)
            iq.choice_search(H, err.view(shape), sweeps=2)
            if ev:
                ev[2].record(stream)
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
        raise SystemExit("encode reported status %d" % int(status.item()))

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
    # encode kernel's per-launch time from HIP events on its launch stream (one
    # launch per step).
    ms_per_step = 1e3 * wall / args.steps
    kernel_ms = ev0.elapsed_time(ev1) / args.steps

    nweights = w_np.size
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
    if args.config.startswith("c5"):
        # Per-kernel times from HIP events around each launch of a second run
        # of the same steps (after the timed region, so that it is not
        # perturbed): the candidate encode, the dominant kernel, carries the
        # roofline (the same sweep as the encode, so the same algorithmic
        # flops per group and entry); the choice search is reported beside it.
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for e in evs:
            step(e)
        torch.cuda.synchronize()
        cand_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
        search_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
        groups = w2.numel() // 8
        flops = groups * cfg["grid"].shape[0] * FLOPS_PER_GROUP_ENTRY[(fmt, True)]
        achieved = flops / (cand_ms * 1e-3) / 1e12
        result["roofline"] = {
            "bound": "alu",
            "achieved": round(achieved, 3),
            "peak": PEAK_FP32_VECTOR_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP32_VECTOR_TFLOPS, 4),
            "traffic": None,
            "kernel": "candidate encode",
            "kernel_ms": round(cand_ms, 5),
            "algorithmic_flops_per_launch": flops,
            "search_ms": round(search_ms, 5),
        }
    else:
        groups = nweights // 8
        weighted = imp is not None
        flops = groups * cfg["grid"].shape[0] * FLOPS_PER_GROUP_ENTRY[(fmt, weighted)]
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        name = "%s_encode_%s" % (fmt.replace("_", ""), args.config)
        result["roofline"] = {
            "bound": "alu",
            "achieved": round(achieved, 3),
            "peak": PEAK_FP32_VECTOR_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP32_VECTOR_TFLOPS, 4),
            "traffic": traffic_for(name, source_sha(KERNEL_SOURCES[fmt])),
            "kernel_ms": round(kernel_ms, 5),
            "algorithmic_flops_per_launch": flops,
        }
    if not args.no_cpu_baseline and args.config in ("c1", "c2", "c3", "c4"):
        result["cpu_baseline"] = cpu_baseline(cfg, fmt)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
