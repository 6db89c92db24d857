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
once) with every input already resident in HBM.  ``roofline`` covers the
dominant launch unit (one call = shrink kernel + expand kernel over a group
of projections), timed with HIP events on the stream the library launches
on.  ``cpu_baseline`` is the CPU oracle on a bounded sample of the same step.
``prefill`` reports the MBGMM prefill workload (32 sequences of 128..2048
tokens, 16 adapters) in TFLOP/s against the bf16 MFMA peak.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


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
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay measurement")
    ap.add_argument("--pool-layout", choices=["scattered", "contiguous"], default="scattered",
                    help="physical page placement: seeded random permutation, or consecutive per adapter")
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(tokens shard across GPUs with no exchange; see the sharding design)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    from workloads.device import host_subset, make_device_workload, tensor_bits
    from heterogeneous_adapters_amd import lora, traffic

    torch.cuda.set_device(0)
    dev = "cuda"
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

    # algorithmic bytes / flops per call and per step
    e = 2
    call_bytes, call_flops = [], []
    for g in groups:
        bsum = fsum = 0
        for i in g:
            t = dw.tables[i]
            bsum += traffic.algorithmic_bytes(dw.ids, dw.ranks, t.d_in, t.d_out, e)
            fsum += traffic.algorithmic_flops(dw.ids, dw.ranks, t.d_in, t.d_out)
        call_bytes.append(bsum)
        call_flops.append(fsum)
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
        raise RuntimeError(f"device flags {seg['flags']}")

    # the same step captured once in a HIP graph and replayed (removes host
    # launch cost; results checked bit for bit against the eager step)
    graph = None
    if not args.no_graph:
        ref_y = [y.clone() for y in Y[:7]]
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
        for y in Y[:7]:
            y.zero_()
        for _ in range(args.warmup):
            cg.replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for _ in range(args.steps):
            cg.replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - g0) * 1e3 / args.steps
        same = all(torch.equal(a, b) for a, b in zip(ref_y, Y[:7]))
        graph = {"ms_per_step": round(gms, 4), "gbs": round(step_bytes / (gms * 1e-3) / 1e9, 1),
                 "matches_eager": bool(same)}
        del cg

    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    mean_call_ms = call_ms.mean(axis=0)
    achieved = float(np.sum(call_bytes) / (mean_call_ms.sum() * 1e-3) / 1e9)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "lora_apply call = shrink_kernel<Bf16> + expand_kernel<Bf16>",
                "launches_per_step": len(groups), "mean_call_us": round(float(mean_call_ms.mean()) * 1e3, 2),
                "algorithmic_bytes_per_call": int(np.mean(call_bytes))}

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
                t = dw.tables[i]
                done_bytes += traffic.algorithmic_bytes(dw.ids, dw.ranks, t.d_in, t.d_out, e)
                got = W.as_f64(tensor_bits(Y[i]), "bf16")
                rf = W.as_f64(ref, "bf16")
                worst = max(worst, float((np.abs(got - rf).max(axis=1) / np.abs(rf).max(axis=1)).max()))
            layers += 1
            if spent >= args.cpu_seconds:
                break
        cpu = {"value": round(done_bytes / spent / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{layers} of {nl} layers x 7 projections, all {T} tokens "
                         f"({done_bytes / 1e9:.2f} GB algorithmic, {spent:.1f} s)",
               "parity_max_rowwise_rel_err": float(f"{worst:.3e}")}

    # ---------------------------------------------------------- prefill
    prefill = None
    if not args.no_prefill:
        del projs, arrays
        w3 = W.make_workload(3, keep_dense=False)
        from heterogeneous_adapters_amd import batch
        b3 = batch.to_device(w3)
        s3 = lora.Segments(w3.T, w3.N)
        ws3 = lora.workspace(w3.T, w3.N, 1, 4096)
        lora.lora_build_segments(b3.ids, b3.adapters, s3, ws3)
        for _ in range(3):
            lora.lora_apply(None, s3, w3.T, b3.projs, b3.adapters, b3.pool, ws3)
        torch.cuda.synchronize()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record()
        for _ in range(args.prefill_steps):
            lora.lora_apply(None, s3, w3.T, b3.projs, b3.adapters, b3.pool, ws3)
        p1.record()
        torch.cuda.synchronize()
        ms = p0.elapsed_time(p1) / args.prefill_steps
        fl = traffic.algorithmic_flops(w3.ids, w3.ranks, 4096, 4096)
        by = traffic.algorithmic_bytes(w3.ids, w3.ranks, 4096, 4096, 2)
        tf = fl / (ms * 1e-3) / 1e12
        prefill = {"workload": f"prefill-mbgmm: 32 sequences, T={w3.T}, 16 adapters, 4096->4096",
                   "ms_per_call": round(ms, 4), "tflops": round(tf, 2),
                   "frac_bf16_mfma_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                   "gbs": round(by / (ms * 1e-3) / 1e9, 1),
                   "frac_hbm_peak": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "intensity_flop_per_byte": round(fl / by, 2)}

    out = {
        "metric": "adapter-branch HBM GB/s (decode MBGMV) + TFLOP/s (prefill MBGMM), % roofline",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama2-7b-decode-step: 32 layers x 7 projections (q,k,v,o 4096->4096; "
                               "gate,up 4096->11008; down 11008->4096), T=1024 tokens, 1000 adapters "
                               "ranks {8,16,32,64}, ids Zipf s=1.2, paged pool 16x4096 bf16 pages",
                   "grouping": args.grouping, "pool_layout": args.pool_layout, "pool_pages": dw.num_pages,
                   "pool_gib": round(dw.num_pages * 16 * 4096 * 2 / 2 ** 30, 1),
                   "distinct_adapters": int(seg["S"]),
                   "step_algorithmic_bytes": int(step_bytes), "step_algorithmic_flops": int(step_flops)},
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "tflops": round(step_flops / (ms_step * 1e-3) / 1e12, 2),
        "ms_per_step_events": round(ms_step_ev, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "prefill": prefill,
        "graph_replay": graph,
        "setup_s": round(gen_s, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
