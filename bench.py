#!/usr/bin/env python3
"""Benchmark of the multi-LoRA adapter branch on one MI355X.

Default workload: the full decode-step adapter branch of a Llama-2-7B-shaped
stack -- 32 layers x 7 adapted projections (q, k, v, o 4096->4096; gate, up
4096->11008; down 11008->4096), 1024 tokens, 1000 adapters resident in one
paged pool of 16 x 4096 bf16 pages (ranks drawn from {8, 16, 32, 64}, ids
bounded-Zipf s = 1.2), fused into supplied Y_base.  One step = one segment
build for the batch plus the branch of all 224 projections; inside a layer
the projections that share an input are issued together (q/k/v, o,
gate/up, down: four calls per layer, the grouping a real forward pass allows).

Prints ONE JSON line.  ``value`` is whole-step algorithmic HBM GB/s (bytes the
method must move: activations once, each distinct adapter's unpadded A and B
once) with every input already resident in HBM, for the step captured once in
a HIP graph and replayed (its replays are checked bit for bit against the
eager step first); the eager step is reported under ``eager``.  ``roofline`` covers the
dominant kernel: at 1024 tokens lora_apply runs each projection group as one
launch of the apply kernel, timed by HIP events around every call of the
eager step (on the stream the library launches on); ``roofline.rocprof``
gives the same kernel's mean duration from the committed rocprofv3 summary.
After the timed steps the same groups also run through lora_shrink /
lora_expand (the two-launch path, same items, Y checked bit-identical), whose
kernels are reported under ``kernels``.  ``traffic`` is the HBM bytes per
launch from the committed rocprofv3 counter summary, or null when the kernel
sources changed since it was taken.
``cpu_baseline`` is the CPU oracle on a bounded sample of the same step.

``--summarize-profile DIR`` (no GPU) turns rocprofv3 CSV output (kernel
stats, or FETCH_SIZE / WRITE_SIZE counter runs that include
``--calibration-copy``) into the text summaries kept under profiles/.
``prefill`` reports the MBGMM prefill workload (32 sequences of 128..2048
tokens, 16 adapters) in TFLOP/s against the bf16 MFMA peak.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
KERNEL_SOURCES = ("heterogeneous_adapters_amd/csrc/lora_kernels.hip", "heterogeneous_adapters_amd/csrc/lora_kernels.h",
                  "heterogeneous_adapters_amd/csrc/lora_plan.h", "include/lora.h")
TRAFFIC_SUMMARY = "profiles/lora_kernels.llama7b_decode_T1024.hbm_traffic.txt"
STATS_SUMMARY = "profiles/lora_kernels.llama7b_decode_T1024.kernel_stats.txt"
# rocprofv3 summaries of the single-workload runs (bench.py --only configN / prefill)
CONFIG_SUMMARIES = {
    2: ("profiles/lora_kernels.hetero_decode_mlp_T512.kernel_stats.txt",
        "profiles/lora_kernels.hetero_decode_mlp_T512.hbm_traffic.txt"),
    3: ("profiles/mbgmm_prefill_T38781.kernel_stats.txt", "profiles/mbgmm_prefill_T38781.hbm_traffic.txt"),
}
# rocprof kernel names of the decode step's kernels (bf16, wide pages)
APPLY_KERNEL = "apply_kernel<lora::Bf16, true, true>"
SHRINK_KERNEL = "shrink_kernel<lora::Bf16, true>"
EXPAND_KERNEL = "expand_kernel<lora::Bf16, true>"
CALIB_BYTES = 1 << 30          # calibration copy: 1 GiB read + 1 GiB written


def kernel_source_hash(root: str = ROOT) -> str:
    """Hash of the kernel sources with comments and blank space removed, so
    that a documentation edit does not orphan a measurement."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(root, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _read_summary(rel: str, kernel_hash: str):
    """Key/value lines and table rows of a committed profile summary; None
    when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None
    kv, rows = {}, []
    with open(path) as f:
        for line in f:
            if line.startswith("  "):
                rows.append(line.split())
            elif ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_hash:
        return None
    return kv, rows


def load_traffic(kernel_hash: str, path: str = ""):
    """HBM bytes per launch of the kernels (apply, shrink, expand) from a
    committed counter summary (default: the decode step's), or None."""
    got = _read_summary(path or TRAFFIC_SUMMARY, kernel_hash)
    if got is None:
        return None
    out = {}
    for key in ("apply", "shrink", "expand"):
        try:
            out[key] = int(float(got[0][f"{key}_hbm_bytes_per_launch"]))
        except (KeyError, ValueError):
            pass
    return out or None


def load_stats(kernel_hash: str, path: str = ""):
    """Mean duration (us) per launch of each lora kernel from a committed
    rocprofv3 kernel-stats summary (default: the decode step's), or None."""
    got = _read_summary(path or STATS_SUMMARY, kernel_hash)
    if got is None:
        return None
    out = {}
    for r in got[1]:
        if len(r) >= 7 and r[0].isdigit():
            name = " ".join(r[6:])
            for k in (APPLY_KERNEL, SHRINK_KERNEL, EXPAND_KERNEL):
                if k in name:
                    out[k] = float(r[1])
    return out or None


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--grouping", choices=["layer", "all"], default="layer",
                    help="layer: q/k/v | o | gate/up | down per call; all: 16 projections per call")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed prefill + decode batch")
    ap.add_argument("--no-padded", action="store_true", help="skip the padded-to-max-rank baseline")
    ap.add_argument("--no-upload", action="store_true", help="skip the pool upload / overlap leg")
    ap.add_argument("--no-stream-ref", action="store_true",
                    help="skip the streaming reference (a plain device copy and read of 1 GiB)")
    ap.add_argument("--no-configs", action="store_true", help="skip the configs 1-2 leg (config 3 still runs)")
    ap.add_argument("--only", choices=["prefill", "configs", "config1", "config2"],
                    help="run only this leg and print its JSON (for profiling one workload)")
    ap.add_argument("--rotate-bytes", type=float, default=1.0,
                    help="GB of input/pool copies the configs leg rotates over (more than the 256 MB MALL)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (the headline is otherwise the HIP-graph replay of the step)")
    ap.add_argument("--pool-layout", choices=["scattered", "contiguous"], default="scattered",
                    help="physical page placement: seeded random permutation, or consecutive per adapter")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="end with a plain elementwise copy of 1 GiB (counter calibration)")
    ap.add_argument("--summarize-profile", metavar="DIR", nargs="+",
                    help="summarize rocprofv3 CSV output under the DIRs and exit (no GPU)")
    ap.add_argument("--profile-command", default="", help="command line recorded in the summary")
    return ap.parse_args()


def groups_for(n_layers, names, mode):
    if mode == "all":
        idx = list(range(n_layers * len(names)))
        return [idx[i:i + 16] for i in range(0, len(idx), 16)]
    pos = {n: i for i, n in enumerate(names)}
    out = []
    for l in range(n_layers):
        base = l * len(names)
        for grp in (("q_proj", "k_proj", "v_proj"), ("o_proj",), ("gate_proj", "up_proj"), ("down_proj",)):
            out.append([base + pos[n] for n in grp])
    return out


PARITY_TOL = 1e-2  # bf16: row-wise infinity-norm relative error against the oracle


def fail(msg: str) -> None:
    """End the run without a headline (non-zero exit)."""
    print(f"bench.py: FAILED: {msg}", file=sys.stderr, flush=True)
    sys.exit(3)


def log(msg: str) -> None:
    """Progress on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


MI355X_CUS, MI355X_XCDS = 256, 8  # compute units, and the XCDs they sit in


def derived_counter_lines(per):
    """Ratios of counters read in one pass, per kernel (mean over dispatches):
    instructions per wave (SQ_INSTS_* / SQ_WAVES), the L2 read latency seen
    by the vector caches (TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ, in
    cycles), the share of L2 cycles with reads to DRAM stalled for credits,
    reads to DRAM in flight per L2 channel (RDREQ_LEVEL / TCC_CYCLE, both
    summed over the channels), the L2 hit rate, and the share of a CU's busy
    cycles its vector L1 / texture units spent stalled (per CU, over
    GRBM_GUI_ACTIVE per XCD)."""
    import numpy as np
    mean = {}
    for (name, ctr), disp in per.items():
        mean.setdefault(name, {})[ctr] = float(np.mean(list(disp.values())))
    out = []
    for name, m in sorted(mean.items()):
        if "lora::" not in name and "neg_kernel" not in name:
            continue
        short = name[:90]
        ratios = []
        if m.get("SQ_WAVES"):
            for ctr in sorted(c for c in m if c.startswith("SQ_INSTS_")):
                ratios.append((f"per_wave_{ctr[9:].lower()}", m[ctr] / m["SQ_WAVES"]))
        if m.get("TCP_TCC_READ_REQ_sum"):
            if "TCP_TCC_READ_REQ_LATENCY_sum" in m:
                ratios.append(("l2_read_latency_cycles", m["TCP_TCC_READ_REQ_LATENCY_sum"] / m["TCP_TCC_READ_REQ_sum"]))
        if m.get("TCC_CYCLE_sum"):
            if "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum" in m:
                ratios.append(("dram_credit_stall_share", m["TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum"] / m["TCC_CYCLE_sum"]))
            if "TCC_EA0_RDREQ_LEVEL_sum" in m:
                ratios.append(("dram_reads_in_flight_per_channel", m["TCC_EA0_RDREQ_LEVEL_sum"] / m["TCC_CYCLE_sum"]))
        if m.get("TCC_HIT_sum", 0) + m.get("TCC_MISS_sum", 0) > 0 and "TCC_HIT_sum" in m and "TCC_MISS_sum" in m:
            ratios.append(("l2_hit_rate", m["TCC_HIT_sum"] / (m["TCC_HIT_sum"] + m["TCC_MISS_sum"])))
        if m.get("GRBM_GUI_ACTIVE"):
            # per-CU counters (summed over the CUs) over the dispatch's busy
            # cycles (GRBM_GUI_ACTIVE, summed over the XCDs)
            cyc = m["GRBM_GUI_ACTIVE"] / MI355X_XCDS
            for ctr, key in (("TCP_PENDING_STALL_CYCLES", "tcp_pending_stall_share"),
                             ("TCP_TCP_TA_DATA_STALL_CYCLES", "tcp_ta_data_stall_share"),
                             ("TD_TC_STALL", "td_tc_stall_share"), ("TD_TD_BUSY", "td_busy_share"),
                             ("TA_DATA_STALLED_BY_TC_CYCLES", "ta_data_stalled_by_tc_share"),
                             ("TA_ADDR_STALLED_BY_TC_CYCLES", "ta_addr_stalled_by_tc_share")):
                if ctr in m:
                    ratios.append((key, m[ctr] / MI355X_CUS / cyc))
        out.extend(f"{key} {val:.4g}  {short}" for key, val in ratios)
    return out


def summarize_profile(dirs, command):
    """Text summary of rocprofv3 CSV output under the directories in dirs
    (kernel stats, and/or FETCH_SIZE / WRITE_SIZE counter runs that end with
    the calibration copy)."""
    import glob
    import numpy as np
    lines = [f"command: {command}" if command else "command: (not recorded)",
             f"kernel_source_hash: {kernel_source_hash()}"]
    found = lambda pat: sorted(p for d in dirs for p in glob.glob(os.path.join(d, "**", pat), recursive=True))
    for path in found("*kernel_stats.csv"):
        lines.append("kernel stats (rocprofv3 --kernel-trace --stats), lora kernels and their share of all GPU time:")
        rows = _read_csv(path)
        tot = sum(float(r["TotalDurationNs"]) for r in rows)
        lines.append(f"  {'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_ms':>10} {'pct':>6}  name")
        for r in rows:
            if "lora::" not in r["Name"]:
                continue
            lines.append(f"  {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                         f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['TotalDurationNs']) / 1e6:10.3f} "
                         f"{100 * float(r['TotalDurationNs']) / tot:6.2f}  {r['Name']}")
    per = {}
    for path in found("*counter_collection.csv"):
        for r in _read_csv(path):
            # a dispatch is (file, id): ids restart in every profiled run, and
            # a counter read in several runs must not add up across them
            # (within one run, the rows of one dispatch's counter are summed)
            d = per.setdefault((r["Kernel_Name"], r["Counter_Name"]), {})
            key = (path, r["Dispatch_Id"])
            d[key] = d.get(key, 0.0) + float(r["Counter_Value"])
    if per:
        calib = {}
        for (name, ctr), disp in per.items():
            if "neg_kernel" in name and ctr in ("FETCH_SIZE", "WRITE_SIZE"):  # the byte counters (KiB)
                calib[ctr] = (CALIB_BYTES / 1024) / float(np.median(list(disp.values())))
        lines.append("counters (rocprofv3 --pmc), per dispatch as read (FETCH_SIZE and WRITE_SIZE in KiB)"
                     + (f"; calibration: a plain elementwise copy (torch.neg) of {CALIB_BYTES >> 20} MiB fp32 reads "
                        "and writes exactly that many bytes" if calib else ""))
        for (name, ctr), disp in sorted(per.items()):
            if "lora::" in name or "neg_kernel" in name:
                vals = np.array(list(disp.values()))
                lines.append(f"  {ctr:10s} dispatches {len(vals):5d} mean {vals.mean():12.1f} min {vals.min():12.1f} "
                             f"max {vals.max():12.1f}  {name[:90]}")
        for ctr, f in sorted(calib.items()):
            lines.append(f"{ctr.lower()}_scale: {f:.4f}")
        # MFMA activity (derived counters MfmaUtil: % of SIMD cycles with the
        # matrix core busy; MfmaFlopsBF16: 512 x bf16 MFMA ops issued)
        for (name, ctr), disp in sorted(per.items()):
            if "lora::" in name and ctr in ("MfmaUtil", "MfmaFlopsBF16"):
                key = "mfma_util_pct" if ctr == "MfmaUtil" else "mfma_bf16_flops_per_dispatch"
                lines.append(f"{key} {float(np.mean(list(disp.values()))):.4g}  {name[:90]}")
        lines.extend(derived_counter_lines(per))
        for kname, key in ((APPLY_KERNEL, "apply"), (SHRINK_KERNEL, "shrink"), (EXPAND_KERNEL, "expand")):
            tot, have = 0.0, 0
            for (name, ctr), disp in per.items():
                if kname in name and ctr in calib:
                    b = float(np.mean(list(disp.values()))) * 1024 * calib[ctr]
                    lines.append(f"{key}_{ctr.lower()}_bytes_per_launch: {b:.0f}")
                    tot += b
                    have += 1
            if have == 2:
                lines.append(f"{key}_hbm_bytes_per_launch: {tot:.0f}")
    print("\n".join(lines))


CONFIG_NAMES = {1: "uniform-rank-decode-q_proj: T=256, 32 adapters rank 16, Zipf 1.1, 4096->4096",
                2: "hetero-rank-decode-mlp: T=512, 128 adapters ranks {8,16,32,64}, Zipf 1.1, "
                   "up 4096->11008 + down 11008->4096, scattered pages",
                3: "prefill-mbgmm: 32 sequences of 128..2048 tokens, 16 adapters ranks {8,16,32,64}, 4096->4096"}


def configs_leg(which, steps, rotate_gb):
    """Configs 1-3 through lora_apply with the timing protocol of a
    cache-cold run: K device copies of the inputs and the pool (together at
    least rotate_gb GB, more than the 256 MB MALL) are used in turn, so every
    call reads its bytes from HBM.  HIP events around every call; the median
    is reported, and the segment build is timed on its own."""
    import numpy as np
    import torch

    import workloads as W
    from heterogeneous_adapters_amd import batch, lora, traffic

    out = {}
    for k in which:
        w = W.make_workload(k, keep_dense=False)
        b0 = batch.to_device(w)
        per_copy = (b0.pool.base.numel() * b0.pool.base.element_size()
                    + sum(t.numel() * t.element_size() for t in b0.X + b0.Y_base + b0.Y))
        K = max(1, int(np.ceil(rotate_gb * 1e9 / per_copy)))
        copies = [b0]
        for _ in range(K - 1):
            pool = b0.pool.base.clone()
            X = [x.clone() for x in b0.X]
            Yb = [y.clone() for y in b0.Y_base]
            Y = [torch.empty_like(y) for y in Yb]
            copies.append(batch.DeviceBatch(b0.T, b0.dtype, b0.ids, b0.adapters, lora.Pool(pool, w.page_width),
                                            b0.tables, X, Yb, Y))
        projs = [[c.proj(p) for p in range(w.n_projs)] for c in copies]
        segs = lora.Segments(w.T, w.N)
        ws = lora.workspace(w.T, w.N, w.n_projs, max(t.d_in for t in w.tables))
        seg_ms = []
        for i in range(steps + 3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            lora.lora_build_segments(b0.ids, b0.adapters, segs, ws)
            e1.record()
            torch.cuda.synchronize()
            if i >= 3:
                seg_ms.append(e0.elapsed_time(e1))
        n_calls = max(steps, 2 * K)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_calls)]
        for i in range(K):  # one warm-up pass over every copy
            c = copies[i % K]
            lora.lora_apply(None, segs, w.T, projs[i % K], c.adapters, c.pool, ws)
        torch.cuda.synchronize()
        for i in range(n_calls):
            c = copies[i % K]
            ev[i][0].record()
            lora.lora_apply(None, segs, w.T, projs[i % K], c.adapters, c.pool, ws)
            ev[i][1].record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        # the two kernels of the two-launch path on the same rotation, each
        # timed on its own (lora_shrink, then lora_expand of that call's v)
        stride = max(w.T, 1) * lora.LORA_MAX_RANK
        vbuf = [torch.empty(lora.lora_v_slices(t.d_in) * stride, dtype=torch.float32, device=b0.pool.base.device)
                for t in w.tables]
        ks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(n_calls)]
        for i in range(n_calls):
            c = copies[i % K]
            ks[i][0].record()
            lora.lora_shrink(projs[i % K], c.adapters, segs, c.pool, vbuf, stride)
            ks[i][1].record()
            lora.lora_expand(projs[i % K], c.adapters, segs, c.pool, vbuf, 0, stride)
            ks[i][2].record()
        torch.cuda.synchronize()
        shr_us = float(np.median([a.elapsed_time(b) for a, b, _ in ks])) * 1e3
        exp_us = float(np.median([b.elapsed_time(c) for _, b, c in ks])) * 1e3
        split = [traffic.group_split_bytes(w.ids, w.ranks, [(t.d_in, t.d_out, i)], 2) for i, t in enumerate(w.tables)]
        sb, eb = sum(x[0] for x in split), sum(x[1] for x in split)
        del vbuf
        by = sum(traffic.algorithmic_bytes(w.ids, w.ranks, t.d_in, t.d_out, 2) for t in w.tables)
        fl = sum(traffic.algorithmic_flops(w.ids, w.ranks, t.d_in, t.d_out) for t in w.tables)
        tf = fl / (ms * 1e-3) / 1e12
        out[str(k)] = {"workload": CONFIG_NAMES[k] + f" (T={w.T})", "copies_rotated": K,
                       "bytes_rotated_gb": round(K * per_copy / 1e9, 2), "calls": n_calls,
                       "ms_per_call_median": round(ms, 4), "algorithmic_mb": round(by / 1e6, 1),
                       "gbs": round(by / (ms * 1e-3) / 1e9, 1),
                       "frac_hbm_peak": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "tflops": round(tf, 2), "frac_bf16_mfma_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                       "intensity_flop_per_byte": round(fl / by, 2),
                       "segment_build_us_median": round(float(np.median(seg_ms)) * 1e3, 1),
                       "two_launch_kernels": {
                           "shrink_us_median": round(shr_us, 2), "shrink_gbs": round(sb / shr_us / 1e3, 1),
                           "expand_us_median": round(exp_us, 2), "expand_gbs": round(eb / exp_us / 1e3, 1),
                           "timing": "hip events around each lora_shrink and lora_expand call, same rotation"}}
        if k in CONFIG_SUMMARIES:
            out[str(k)]["rocprof"] = config_rocprof(k, {"apply": by, "shrink": sb, "expand": eb})
        del copies, projs, b0, w
        torch.cuda.empty_cache()
    return out


def config_rocprof(k, algorithmic):
    """Per-kernel rocprofv3 figures of config k from its committed summaries
    (mean launch duration, HBM bytes per launch and their ratio to the
    algorithmic bytes), when they were taken on the current kernel sources."""
    hsh = kernel_source_hash()
    stats_path, traffic_path = CONFIG_SUMMARIES[k]
    stats = load_stats(hsh, stats_path) or {}
    hbm = load_traffic(hsh, traffic_path) or {}
    out = {"stats_source": stats_path if stats else None, "traffic_source": traffic_path if hbm else None}
    for kname, key in ((APPLY_KERNEL, "apply"), (SHRINK_KERNEL, "shrink"), (EXPAND_KERNEL, "expand")):
        us, hb = stats.get(kname), hbm.get(key)
        if us is None and hb is None:
            continue
        alg = algorithmic[key]
        out[key] = {"mean_launch_us": us, "gbs": round(alg / us / 1e3, 1) if us else None,
                    "algorithmic_bytes_per_launch": int(alg), "hbm_bytes_per_launch": hb,
                    "hbm_over_algorithmic": round(hb / alg, 3) if hb else None}
    return out


def stream_reference(dev, reps=20):
    """Streaming rates of this GPU measured in the same run, the secondary
    reference for the GB/s figures: a plain device-to-device copy of 1 GiB
    (1 GiB read + 1 GiB written) and a row-wise integer max over the same GiB
    viewed as int32 (read only; a float sum reads at about half that rate),
    HIP events around each call, medians over `reps` calls after warm-up."""
    import numpy as np
    import torch

    n = CALIB_BYTES // 2
    src = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_()
    dst = torch.empty_like(src)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    copy_ms = timed(lambda: dst.copy_(src))
    rows = src.view(torch.int32).view(-1, 4096)
    read_ms = timed(lambda: rows.amax(dim=1))
    del src, dst, rows
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2 * CALIB_BYTES / (copy_ms * 1e-3) / 1e9, 1),
            "read_gbs": round(CALIB_BYTES / (read_ms * 1e-3) / 1e9, 1), "bytes": CALIB_BYTES, "reps": reps}


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.profile_command)
        return
    if args.gpus != 1:
        print(f"bench.py: the adapter branch is measured on one GPU; --gpus {args.gpus} is not supported "
              "(tokens shard across GPUs with no exchange; see the sharding design)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    from workloads.device import host_subset, make_device_workload, tensor_bits
    from heterogeneous_adapters_amd import lora, traffic

    torch.cuda.set_device(0)
    if args.only:
        which = {"prefill": [3], "configs": [1, 2, 3], "config1": [1], "config2": [2]}[args.only]
        print(json.dumps({"configs": configs_leg(which, args.prefill_steps, args.rotate_bytes)}), flush=True)
        if args.calibration_copy:
            calibration_copy()
        return
    dev = "cuda"
    log("generating the decode-step workload on the device")
    t_gen = time.perf_counter()
    dw = make_device_workload(4, dev, overrides=dict(scatter=args.pool_layout == "scattered"))
    T, N = dw.T, dw.N
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    ids = i32(dw.ids)
    adapters = lora.Adapters(i32(dw.ranks), torch.from_numpy(dw.alpha).to(dev))
    pool = lora.Pool(dw.pool, dw.page_width)
    tabs = [(i32(t.a_indptr), i32(t.a_pages), i32(t.b_indptr), i32(t.b_pages)) for t in dw.tables]
    Y = [torch.empty_like(y) for y in dw.Y_base]
    projs = [lora.Proj(dw.X[p], dw.Y_base[p], Y[p], *tabs[p]) for p in range(dw.n_projs)]
    names = [n for (n, _, _) in W.CONFIGS[4]["projs"]]
    groups = groups_for(W.CONFIGS[4]["layers"], names, args.grouping)
    segs = lora.Segments(T, N)
    ws_seg = lora.workspace(T, N, 0, 0)
    ws = lora.workspace(T, N, max(len(g) for g in groups), max(t.d_in for t in dw.tables))
    arrays = [(lora.lora_proj_t * len(g))(*[projs[i].c for i in g]) for g in groups]
    L = lora.lib()
    import ctypes
    seg_c, ad_c, pool_c = ctypes.byref(segs.c), ctypes.byref(adapters.c), ctypes.byref(pool.c)
    ws_ptr, ws_n = ctypes.c_void_p(ws.data_ptr()), ws.numel()
    gen_s = time.perf_counter() - t_gen

    # algorithmic bytes / flops per call and per step; projections of a call
    # that read one activation tensor (q/k/v, gate/up) count it once
    e = 2
    call_split = [traffic.group_split_bytes(dw.ids, dw.ranks, [(dw.tables[i].d_in, dw.tables[i].d_out,
                                                                dw.X[i].data_ptr()) for i in g], e)
                  for g in groups]
    call_bytes = [sum(sp) for sp in call_split]
    call_flops = [sum(traffic.algorithmic_flops(dw.ids, dw.ranks, dw.tables[i].d_in, dw.tables[i].d_out) for i in g)
                  for g in groups]
    step_bytes = sum(call_bytes)
    step_flops = sum(call_flops)

    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def step(evs=None):
        lora.lora_build_segments(ids, adapters, segs, ws_seg, stream)
        for gi, arr in enumerate(arrays):
            if evs is not None:
                evs[gi][0].record(stream)
            st = L.lora_apply(None, seg_c, T, arr, len(groups[gi]), ad_c, pool_c, ws_ptr, ws_n, sptr)
            if st != 0:
                raise lora.LoraError("lora_apply", st)
            if evs is not None:
                evs[gi][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in groups]
           for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for k in range(args.steps):
        step(evs[k])
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    ms_step_ev = e0.elapsed_time(e1) / args.steps
    call_ms = np.array([[a.elapsed_time(b) for a, b in row] for row in evs])  # [steps][calls]
    seg = segs.arrays()
    if seg["flags"] != 0:
        fail(f"device flags {seg['flags']} after the timed steps")

    log("eager steps timed; per-kernel leg")
    # per-kernel leg: the same groups through lora_shrink / lora_expand (the
    # two launches lora_apply makes, same grid), HIP events around each
    # launch on the library's stream; Y must come out bit-identical
    y_apply = [y.clone() for y in Y[:7]]
    v_stride = T * lora.LORA_MAX_RANK
    max_g = max(len(g) for g in groups)
    vbuf = [torch.empty(lora.lora_v_slices(max(t.d_in for t in dw.tables)) * v_stride, dtype=torch.float32,
                        device=dev) for _ in range(max_g)]
    vptrs = [(ctypes.c_void_p * len(g))(*[vbuf[j].data_ptr() for j in range(len(g))]) for g in groups]
    kev = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in groups] for _ in range(args.steps)]
    for k in range(args.steps):
        for gi, arr in enumerate(arrays):
            ev = kev[k][gi]
            ev[0].record(stream)
            st = L.lora_shrink(arr, len(groups[gi]), ad_c, seg_c, pool_c, vptrs[gi], v_stride, sptr)
            ev[1].record(stream)
            st = st or L.lora_expand(arr, len(groups[gi]), ad_c, seg_c, pool_c, vptrs[gi], 0, v_stride, sptr)
            ev[2].record(stream)
            if st != 0:
                raise lora.LoraError("lora_shrink/lora_expand", st)
    torch.cuda.synchronize()
    split_same = all(torch.equal(a, b) for a, b in zip(y_apply, Y[:7]))
    shr_ms = np.array([[ev[0].elapsed_time(ev[1]) for ev in row] for row in kev]).mean(axis=0)  # per group
    exp_ms = np.array([[ev[1].elapsed_time(ev[2]) for ev in row] for row in kev]).mean(axis=0)
    del vbuf

    log("graph capture and replay")
    # The headline step: the same step captured once in a HIP graph and
    # replayed (a decode step is replayed, not re-launched, in serving; the
    # graph holds only kernel nodes).  Every warm-up replay is checked bit for
    # bit against the eager step, with eager work in between.
    graph = None
    if not args.no_graph:
        ref_y = [y.clone() for y in Y]
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            gsptr = ctypes.c_void_p(side.cuda_stream)

            def gstep():
                lora.lora_build_segments(ids, adapters, segs, ws_seg, side)
                for gi, arr in enumerate(arrays):
                    st = L.lora_apply(None, seg_c, T, arr, len(groups[gi]), ad_c, pool_c, ws_ptr, ws_n, gsptr)
                    if st != 0:
                        raise lora.LoraError("lora_apply", st)
            gstep()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg, stream=side):
            gstep()
        torch.cuda.synchronize()
        checked = 0
        for _ in range(max(args.warmup, 2)):
            for y in Y:
                y.zero_()
            torch.cuda.synchronize()
            cg.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(ref_y, Y)):
                raise RuntimeError("graph replay differs from the eager step")
            checked += 1
        del ref_y
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        ge0, ge1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ge0.record(stream)
        for _ in range(args.steps):
            cg.replay()
        ge1.record(stream)
        torch.cuda.synchronize()
        gms = (time.perf_counter() - g0) * 1e3 / args.steps
        graph = {"ms_per_step": round(gms, 4), "ms_per_step_events": round(ge0.elapsed_time(ge1) / args.steps, 4),
                 "replays_checked_bit_exact": checked}
        del cg

    log("sampled parity of every projection")
    # Parity gate, part 1: every one of the 224 projections on sampled tokens
    # (random ones, the hottest adapter's, singletons), each computed by the
    # oracle token by token from the pages those tokens use.  Part 2 is the
    # whole-layer comparison of the CPU-baseline leg.  A failure of either (or
    # a device flag) ends the run without a headline.
    import oracle
    rng = np.random.default_rng(0)
    cnt_ids = np.bincount(dw.ids[dw.ids >= 0], minlength=N)
    hot = np.nonzero(dw.ids == cnt_ids.argmax())[0]
    single = np.nonzero((dw.ids >= 0) & (cnt_ids[np.maximum(dw.ids, 0)] == 1))[0]
    sample = np.unique(np.concatenate([rng.choice(T, 16, replace=False), hot[:8], single[:8]]))
    sub_ids = dw.ids[sample]
    parity_sampled = 0.0
    nl_all = W.CONFIGS[4]["layers"]
    for l in range(nl_all):
        idx = list(range(l * 7, l * 7 + 7))
        hpool, htabs = host_subset(dw.pool, [dw.tables[i] for i in idx], np.unique(sub_ids[sub_ids >= 0]))
        for j, i in enumerate(idx):
            ref = W.as_f64(oracle.apply(tensor_bits(dw.X[i])[sample], tensor_bits(dw.Y_base[i])[sample], sub_ids,
                                        dw.ranks, dw.alpha, htabs[j], hpool, dw.page_width, "bf16"), "bf16")
            got = W.as_f64(tensor_bits(Y[i])[sample], "bf16")
            err = float((np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)).max()) \
                if np.isfinite(got).all() else float("inf")
            parity_sampled = max(parity_sampled, err)
        del hpool, htabs
    parity = {"tolerance": PARITY_TOL, "sampled_tokens": int(len(sample)), "sampled_projections": len(dw.tables),
              "sampled_max_rowwise_rel_err": float(f"{parity_sampled:.3e}")}
    if parity_sampled >= PARITY_TOL:
        fail(f"parity: sampled max row-wise relative error {parity_sampled:.3e} >= {PARITY_TOL}")

    eager_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    head_ms = graph["ms_per_step"] if graph else ms_step
    gbs = step_bytes / (head_ms * 1e-3) / 1e9
    mean_call_ms = call_ms.mean(axis=0)
    hsh = kernel_source_hash()
    stats = load_stats(hsh) or {}
    hbm = load_traffic(hsh) or {}

    def rocprof_part(kname, bytes_per_launch):
        us = stats.get(kname)
        if us is None:
            return None
        gb = bytes_per_launch / (us * 1e-6) / 1e9
        return {"source": STATS_SUMMARY, "mean_launch_us": us, "achieved": round(gb, 1),
                "frac": round(gb / HBM_PEAK_GBS, 4)}

    kernels = {}
    # The step's kernel: at T = 1024 lora_apply runs each group as one launch
    # of the apply kernel (lora_set_launch_mode, automatic choice); HIP events
    # around every call of the eager step time it (they include the gap
    # between launches), the committed rocprofv3 summary gives its duration
    apply_b = float(np.mean(call_bytes))
    gb_apply = float(np.sum(call_bytes) / (mean_call_ms.sum() * 1e-3) / 1e9)
    kernels[APPLY_KERNEL] = {"launches_per_step": len(groups), "mean_launch_us": round(float(mean_call_ms.mean()) * 1e3, 2),
                             "timing": "hip events around each lora_apply call, eager step",
                             "algorithmic_bytes_per_launch": int(apply_b), "gbs": round(gb_apply, 1),
                             "frac_hbm_peak": round(gb_apply / HBM_PEAK_GBS, 4),
                             "rocprof": rocprof_part(APPLY_KERNEL, apply_b), "hbm_bytes_per_launch": hbm.get("apply")}
    # the two-launch path's kernels (lora_shrink / lora_expand on the same
    # groups, the same items; Y checked bit-identical)
    for kname, ms_g, part, tkey in ((SHRINK_KERNEL, shr_ms, 0, "shrink"), (EXPAND_KERNEL, exp_ms, 1, "expand")):
        kb = [sp[part] for sp in call_split]
        gb = float(np.sum(kb) / (ms_g.sum() * 1e-3) / 1e9)
        kernels[kname] = {"launches_per_step": len(groups), "mean_launch_us": round(float(ms_g.mean()) * 1e3, 2),
                          "timing": "hip events around each lora_shrink / lora_expand launch",
                          "algorithmic_bytes_per_launch": int(np.mean(kb)), "gbs": round(gb, 1),
                          "frac_hbm_peak": round(gb / HBM_PEAK_GBS, 4),
                          "rocprof": rocprof_part(kname, float(np.mean(kb))), "hbm_bytes_per_launch": hbm.get(tkey)}
    # the two kernels by projection group (q/k/v, o, gate/up, down), as
    # mean launch time and GB/s over the layers, and the single launch
    by_group = {}
    for gi, g in enumerate(groups):
        key = "+".join(names[i % len(names)].replace("_proj", "") for i in g)
        d = by_group.setdefault(key, {"shrink_us": [], "expand_us": [], "shrink_b": [], "expand_b": [],
                                      "apply_us": [], "apply_b": []})
        d["shrink_us"].append(shr_ms[gi] * 1e3)
        d["expand_us"].append(exp_ms[gi] * 1e3)
        d["apply_us"].append(mean_call_ms[gi] * 1e3)
        d["shrink_b"].append(call_split[gi][0])
        d["expand_b"].append(call_split[gi][1])
        d["apply_b"].append(call_bytes[gi])
    for key, d in by_group.items():
        su, eu, au = (float(np.mean(d[k])) for k in ("shrink_us", "expand_us", "apply_us"))
        by_group[key] = {"apply_us": round(au, 2), "apply_gbs": round(float(np.mean(d["apply_b"])) / au / 1e3, 1),
                         "shrink_us": round(su, 2), "shrink_gbs": round(float(np.mean(d["shrink_b"])) / su / 1e3, 1),
                         "expand_us": round(eu, 2), "expand_gbs": round(float(np.mean(d["expand_b"])) / eu / 1e3, 1)}
    kernels["by_group"] = by_group
    dom = kernels[APPLY_KERNEL]
    roofline = {"bound": "hbm", "achieved": dom["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": dom["frac_hbm_peak"], "traffic": hbm.get("apply"),
                "kernel": APPLY_KERNEL, "timing": dom["timing"], "mean_launch_us": dom["mean_launch_us"],
                "rocprof": dom["rocprof"], "traffic_source": TRAFFIC_SUMMARY if hbm.get("apply") else None,
                "algorithmic_bytes_per_launch": dom["algorithmic_bytes_per_launch"],
                "launches_per_step": len(groups)}

    log("CPU oracle baseline")
    # ---------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        valid = (dw.ids >= 0) & (dw.ids < N)
        distinct = np.unique(dw.ids[valid])
        spent = 0.0
        done_bytes = 0
        layers = 0
        worst = 0.0
        nl = W.CONFIGS[4]["layers"]
        for l in range(nl):
            idx = list(range(l * 7, l * 7 + 7))
            hpool, htabs = host_subset(dw.pool, [dw.tables[i] for i in idx], distinct)
            for j, i in enumerate(idx):
                Xh, Ybh = tensor_bits(dw.X[i]), tensor_bits(dw.Y_base[i])
                c0 = time.perf_counter()
                ref = oracle.apply(Xh, Ybh, dw.ids, dw.ranks, dw.alpha, htabs[j], hpool, dw.page_width, "bf16",
                                   nthreads=threads)
                spent += time.perf_counter() - c0
                got = W.as_f64(tensor_bits(Y[i]), "bf16")
                rf = W.as_f64(ref, "bf16")
                worst = max(worst, float((np.abs(got - rf).max(axis=1) / np.abs(rf).max(axis=1)).max()))
            # the layer's algorithmic bytes, a shared activation counted once (as for the GPU)
            done_bytes += sum(traffic.group_split_bytes(dw.ids, dw.ranks, [(dw.tables[i].d_in, dw.tables[i].d_out,
                                                                           dw.X[i].data_ptr()) for i in idx], e))
            layers += 1
            if spent >= args.cpu_seconds:
                break
        cpu = {"value": round(done_bytes / spent / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{layers} of {nl} layers x 7 projections, all {T} tokens "
                         f"({done_bytes / 1e9:.2f} GB algorithmic, {spent:.1f} s)",
               "parity_max_rowwise_rel_err": float(f"{worst:.3e}")}
        parity["whole_layers"] = layers
        parity["whole_layer_max_rowwise_rel_err"] = float(f"{worst:.3e}")
        if worst >= PARITY_TOL:
            fail(f"parity: whole-layer max row-wise relative error {worst:.3e} >= {PARITY_TOL}")
        # the small workloads on all threads and on one (best of 3; configs 2
        # and 3 on one thread: a single run), over the same algorithmic bytes
        per_cfg = {}
        for k in (0, 1, 2, 3):
            wk = W.make_workload(k, keep_dense=False)
            by = sum(traffic.algorithmic_bytes(wk.ids, wk.ranks, t.d_in, t.d_out, 2 if wk.dtype == "bf16" else 4)
                     for t in wk.tables)
            res = {}
            for nth in (threads, 1):
                best = float("inf")
                for _ in range(1 if (k >= 2 and nth == 1) else 3):
                    c0 = time.perf_counter()
                    for p in range(wk.n_projs):
                        oracle.apply(wk.X[p], wk.Y_base[p], wk.ids, wk.ranks, wk.alpha, wk.tables[p], wk.pool,
                                     wk.page_width, wk.dtype, nthreads=nth)
                    best = min(best, time.perf_counter() - c0)
                res[nth] = best
            per_cfg[str(k)] = {"ms": round(res[threads] * 1e3, 2), "gbs": round(by / res[threads] / 1e9, 3),
                               "ms_1_thread": round(res[1] * 1e3, 2), "gbs_1_thread": round(by / res[1] / 1e9, 3)}
            del wk
        cpu["configs"] = per_cfg

    log("configs leg (configs 1-3, cache-cold rotation)")
    # ---------------------------------------------------------- configs 1-3
    # the small benchmark workloads, each rotated over >= 1 GB of copies so
    # its bytes come from HBM; config 3 is the prefill (MBGMM) line
    prefill, configs = None, None
    del projs, arrays
    which = ([] if args.no_configs else [1, 2]) + ([] if args.no_prefill else [3])
    if which:
        configs = configs_leg(which, args.prefill_steps, args.rotate_bytes)
        prefill = configs.get("3")

    log("shared-activation leg")
    # ---------------------------------------------------------- shared activation
    # q/k/v of a prefill batch (config 3's 32 sequences, 3 x 4096->4096) in one
    # call: one X tensor read by all three (the launch walks their shrink items
    # side by side) against three separate copies of it
    shared = None
    if not args.no_prefill:
        w6 = W.make_workload(3, dict(projs=(("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096))),
                             keep_dense=False)
        from heterogeneous_adapters_amd import batch
        b6 = batch.to_device(w6)
        s6 = lora.Segments(w6.T, w6.N)
        ws6 = lora.workspace(w6.T, w6.N, 3, 4096)
        lora.lora_build_segments(b6.ids, b6.adapters, s6, ws6)
        res = {}
        for mode in ("separate", "shared"):
            for p in (1, 2):
                b6.X[p] = b6.X[0] if mode == "shared" else b6.X[0].clone()
            pj = [b6.proj(p) for p in range(3)]
            for _ in range(2):
                lora.lora_apply(None, s6, w6.T, pj, b6.adapters, b6.pool, ws6)
            torch.cuda.synchronize()
            x0, x1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            x0.record()
            for _ in range(5):
                lora.lora_apply(None, s6, w6.T, pj, b6.adapters, b6.pool, ws6)
            x1.record()
            torch.cuda.synchronize()
            res[mode] = x0.elapsed_time(x1) / 5
        sb = traffic.group_split_bytes(w6.ids, w6.ranks, [(4096, 4096, "x")] * 3, 2)
        shared = {"workload": f"prefill q/k/v: T={w6.T}, 16 adapters, 3 x 4096->4096 in one call",
                  "separate_x_ms_per_call": round(res["separate"], 4), "shared_x_ms_per_call": round(res["shared"], 4),
                  "speedup": round(res["separate"] / res["shared"], 3),
                  "shared_x_gbs": round(sum(sb) / (res["shared"] * 1e-3) / 1e9, 1)}
        del b6, w6

    log("mixed-batch leg")
    # ---------------------------------------------------------- mixed batch
    # continuous batching: prefill chunks (MBGMM segments) and decode tokens
    # (MBGMV segments) of 1000 adapters in one lora_apply
    mixed = None
    if not args.no_mixed:
        w5 = W.make_workload(5, keep_dense=False)
        from heterogeneous_adapters_amd import batch
        b5 = batch.to_device(w5)
        s5 = lora.Segments(w5.T, w5.N)
        ws5 = lora.workspace(w5.T, w5.N, 1, 4096)
        lora.lora_build_segments(b5.ids, b5.adapters, s5, ws5)
        for _ in range(3):
            lora.lora_apply(None, s5, w5.T, b5.projs, b5.adapters, b5.pool, ws5)
        torch.cuda.synchronize()
        m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m0.record()
        for _ in range(args.prefill_steps):
            lora.lora_apply(None, s5, w5.T, b5.projs, b5.adapters, b5.pool, ws5)
        m1.record()
        torch.cuda.synchronize()
        ms = m0.elapsed_time(m1) / args.prefill_steps
        by = traffic.algorithmic_bytes(w5.ids, w5.ranks, 4096, 4096, 2)
        fl = traffic.algorithmic_flops(w5.ids, w5.ranks, 4096, 4096)
        _, cnt = np.unique(w5.ids, return_counts=True)
        mixed = {"workload": f"mixed-prefill-decode: {len(w5.seq_lens)} prefill chunks "
                             f"({int(sum(w5.seq_lens))} tokens) + {W.CONFIGS[5]['ndecode']} decode tokens, "
                             f"1000 adapters, 4096->4096",
                 "T": int(w5.T), "segments": int(len(cnt)), "mbgmm_segments": int((cnt >= 16).sum()),
                 "ms_per_call": round(ms, 4), "gbs": round(by / (ms * 1e-3) / 1e9, 1),
                 "frac_hbm_peak": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "tflops": round(fl / (ms * 1e-3) / 1e12, 2)}
        del b5, w5

    log("padded-baseline leg")
    # ---------------------------------------------------------- padded baseline
    # the cost of padding: the heterogeneous-rank decode batch of 128 adapters
    # (up + down MLP projections) against the same adapters zero-padded to
    # rank 64 (a fixed-rank slot layout), through the same kernels; GB/s is
    # over the unpadded algorithmic bytes for both
    padded = None
    w2 = W.make_workload(2) if not (args.no_padded and args.no_upload) else None
    if not args.no_padded:
        from heterogeneous_adapters_amd import batch

        def time_calls(wk):
            bk = batch.to_device(wk)
            sk = lora.Segments(wk.T, wk.N)
            wsk = lora.workspace(wk.T, wk.N, len(bk.projs), 11008)
            lora.lora_build_segments(bk.ids, bk.adapters, sk, wsk)
            for _ in range(3):
                lora.lora_apply(None, sk, wk.T, bk.projs, bk.adapters, bk.pool, wsk)
            torch.cuda.synchronize()
            q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            q0.record()
            for _ in range(args.prefill_steps):
                lora.lora_apply(None, sk, wk.T, bk.projs, bk.adapters, bk.pool, wsk)
            q1.record()
            torch.cuda.synchronize()
            return q0.elapsed_time(q1) / args.prefill_steps

        w2p = W.pad_to_rank(w2, 64)
        ms_h, ms_p = time_calls(w2), time_calls(w2p)
        by = sum(traffic.algorithmic_bytes(w2.ids, w2.ranks, t.d_in, t.d_out, 2) for t in w2.tables)
        byp = sum(traffic.algorithmic_bytes(w2p.ids, w2p.ranks, t.d_in, t.d_out, 2) for t in w2p.tables)
        padded = {"workload": "hetero-rank-decode-mlp: T=512, 128 adapters ranks {8,16,32,64}, Zipf 1.1, "
                              "up 4096->11008 + down 11008->4096; padded = every adapter zero-padded to rank 64",
                  "heterogeneous_ms_per_call": round(ms_h, 4), "padded_ms_per_call": round(ms_p, 4),
                  "padded_over_heterogeneous_time": round(ms_p / ms_h, 3),
                  "heterogeneous_gbs": round(by / (ms_h * 1e-3) / 1e9, 1),
                  "padded_gbs_of_unpadded_bytes": round(by / (ms_p * 1e-3) / 1e9, 1),
                  "padded_bytes_over_unpadded": round(byp / by, 3)}
        del w2p

    log("pool-upload leg")
    # ------------------------------------------------------------ pool upload
    # the pool manager's miss path on the same 128 adapters: every adapter's
    # pages from pinned host memory into an empty device pool (cache
    # admission, page assignment, one transfer per run of consecutive pages),
    # the same bytes page by page onto scattered page ids, and the upload on
    # its side stream while lora_apply calls run on the compute stream
    upload = None
    if not args.no_upload:
        from heterogeneous_adapters_amd import batch
        from heterogeneous_adapters_amd.pool import ManagedPool, host_tier_from_pool
        hp = torch.from_numpy(np.ascontiguousarray(w2.pool).view(np.int16)).view(torch.bfloat16)
        tier = host_tier_from_pool(hp, w2.tables, w2.N)
        ipt = [(t.a_indptr, t.b_indptr) for t in w2.tables]
        n_pg = int(tier.shape[0])
        up_bytes = tier.numel() * 2
        b2 = batch.to_device(w2)
        s2 = lora.Segments(w2.T, w2.N)
        ws2 = lora.workspace(w2.T, w2.N, len(b2.projs), 11008)
        lora.lora_build_segments(b2.ids, b2.adapters, s2, ws2)
        cur = torch.cuda.current_stream()

        def ev():
            return torch.cuda.Event(enable_timing=True)

        def upload_alone():
            mp = ManagedPool(ipt, tier, w2.page_width, n_pg)
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record(mp.upload_stream)
            mp.ensure(range(w2.N))
            e1.record(mp.upload_stream)
            torch.cuda.synchronize()
            assert mp.misses == w2.N and mp.pages_uploaded == n_pg
            return e0.elapsed_time(e1), mp

        upload_alone()  # warm-up (first transfers, allocator)
        t_up, mp = upload_alone()
        # page by page onto a random permutation of the pool (no runs to merge)
        perm = np.random.default_rng(0).permutation(n_pg).astype(np.int32)
        side = torch.cuda.Stream()
        e0, e1 = ev(), ev()
        e0.record(side)
        lora.lora_upload_pages(mp.pool, tier, perm, stream=side)
        e1.record(side)
        torch.cuda.synchronize()
        t_scatter = e0.elapsed_time(e1)
        assert torch.equal(mp.base[torch.from_numpy(perm[:8].astype(np.int64)).cuda()].cpu().view(torch.int16),
                           tier[:8].view(torch.int16))
        del mp

        def applies(k):
            for _ in range(k):
                lora.lora_apply(None, s2, w2.T, b2.projs, b2.adapters, b2.pool, ws2)

        applies(3)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        applies(20)
        e1.record()
        torch.cuda.synchronize()
        call_ms = e0.elapsed_time(e1) / 20
        K = max(20, int(math.ceil(t_up / call_ms)))
        e0, e1 = ev(), ev()
        e0.record()
        applies(K)
        e1.record()
        torch.cuda.synchronize()
        t_apply = e0.elapsed_time(e1)
        # both: the uploads are enqueued first (on the side stream, after a
        # common start event), then the calls on the compute stream
        mp = ManagedPool(ipt, tier, w2.page_width, n_pg)
        torch.cuda.synchronize()
        t0, ua, a0, a1 = ev(), ev(), ev(), ev()
        t0.record(cur)
        mp.upload_stream.wait_event(t0)
        for a in range(w2.N):
            hit, pages, _ = mp.cache.admit(a, mp.n_pages(a))
            lora.lora_upload_pages(mp.pool, tier[mp.offsets[a]:mp.offsets[a + 1]], pages, stream=mp.upload_stream)
        ua.record(mp.upload_stream)
        a0.record(cur)
        applies(K)
        a1.record(cur)
        torch.cuda.synchronize()
        span = max(t0.elapsed_time(ua), t0.elapsed_time(a1))
        upload = {"workload": f"hetero-rank-decode-mlp adapters: {w2.N} adapters ranks {{8,16,32,64}}, "
                              f"up 4096->11008 + down 11008->4096, {n_pg} pages of 16x4096 bf16 "
                              f"({up_bytes / 2 ** 20:.0f} MiB) from pinned host memory",
                  "upload_ms": round(t_up, 3), "upload_gbs": round(up_bytes / (t_up * 1e-3) / 1e9, 1),
                  "transfers": int(w2.N),
                  "page_by_page_ms": round(t_scatter, 3),
                  "page_by_page_gbs": round(up_bytes / (t_scatter * 1e-3) / 1e9, 1),
                  "apply_calls": K, "apply_ms_alone": round(t_apply, 3),
                  "apply_ms_during_upload": round(a0.elapsed_time(a1), 3),
                  "upload_ms_during_apply": round(t0.elapsed_time(ua), 3),
                  "both_span_ms": round(span, 3),
                  "overlap_frac": round((t_up + t_apply - span) / min(t_up, t_apply), 3)}
        del mp, b2, tier
    w2 = None

    out = {
        "metric": "adapter-branch HBM GB/s (decode MBGMV) + TFLOP/s (prefill MBGMM), % roofline",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama2-7b-decode-step: 32 layers x 7 projections (q,k,v,o 4096->4096; "
                               "gate,up 4096->11008; down 11008->4096), T=1024 tokens, 1000 adapters "
                               "ranks {8,16,32,64}, ids Zipf s=1.2, paged pool 16x4096 bf16 pages",
                   "grouping": args.grouping, "pool_layout": args.pool_layout, "pool_pages": dw.num_pages,
                   "pool_gib": round(dw.num_pages * 16 * 4096 * 2 / 2 ** 30, 1),
                   "distinct_adapters": int(seg["S"]),
                   "step_algorithmic_bytes": int(step_bytes), "step_algorithmic_flops": int(step_flops)},
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "tflops": round(step_flops / (head_ms * 1e-3) / 1e12, 2),
        "timing": ("hip-graph replay of the whole step (segment build + every lora_apply call), captured once; "
                   "eager launches reported under 'eager'") if graph else "eager launches",
        "eager": {"ms_per_step": round(ms_step, 4), "ms_per_step_events": round(ms_step_ev, 4),
                  "gbs": round(eager_gbs, 1)},
        "roofline": roofline,
        "kernels": dict(kernels, **{"lora_apply_call": {
            "mean_call_us": round(float(mean_call_ms.mean()) * 1e3, 2),
            "algorithmic_bytes_per_call": int(np.mean(call_bytes)),
            "gbs": round(float(np.sum(call_bytes) / (mean_call_ms.sum() * 1e-3) / 1e9), 1)},
            "split_matches_apply": bool(split_same)}),
        "cpu_baseline": cpu,
        "parity": parity,
        "prefill": prefill,
        "configs": configs,
        "shared_activation": shared,
        "mixed": mixed,
        "padded_baseline": padded,
        "pool_upload": upload,
        "graph_replay": graph,
        "setup_s": round(gen_s, 1),
    }
    if not args.no_stream_ref:
        log("streaming reference")
        ref = stream_reference(dev)
        ref["value_over_copy"] = round(gbs / ref["copy_gbs"], 4)
        ref["value_over_read"] = round(gbs / ref["read_gbs"], 4)
        out["stream_reference"] = ref
    print(json.dumps(out), flush=True)
    if args.calibration_copy:
        calibration_copy()


def calibration_copy():
    """A plain elementwise copy of CALIB_BYTES (read and written), whose
    FETCH_SIZE / WRITE_SIZE readings calibrate the counters' units."""
    import torch
    a = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()


if __name__ == "__main__":
    main()
