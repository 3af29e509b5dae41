#!/usr/bin/env python3
"""Throughput of the IndexCache sparse-attention hot path on one MI355X.

A step is one pass of the whole path over one batch: indexer -> top-k ->
sparse MLA with sink, through ic_layer_stack. The default workload is one full
decode layer at batch 1 over a 131,072-token cache (indexer 64x128 fp8, top-2048,
MLA 128 heads over 576-wide bf16 latent rows). Inputs are resident in HBM
before timing starts; R independently seeded input sets are rotated so that
the working set (R x ~168 MB) does not fit in the 256 MB Infinity Cache.

Prints one JSON line (rank 0). Other workloads (--workload) are for reports;
the default line is the headline figure.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA


def algorithmic_bytes(n: int, k: int, H_I: int, D_I: int, H: int, D_qk: int, D_v: int, full: bool):
    """Bytes the method itself must move for one query-layer (score round
    trips are overhead, not work): the shared part reads the selected rows,
    the index and the query and writes the output; a full layer also streams
    every key row, reads the indexer query and weights, and writes the index."""
    kp = min(k, n)
    shared = 4 * kp + 2 * D_qk * kp + H * (2 * D_qk + 2 * D_v + 4)
    if not full:
        return shared
    return shared + D_I * n + H_I * (D_I + 4) + 4 * kp


def indexer_bytes(n: int, H_I: int, D_I: int) -> int:
    """Algorithmic bytes of one query's indexer pass: key rows + q + w."""
    return D_I * n + H_I * (D_I + 4)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="decode_128k")
    ap.add_argument("--sets", type=int, default=8, help="rotating input sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--kernel-steps", type=int, default=400, help="launches timed for the dominant kernel")
    ap.add_argument("--only", choices=["all", "step", "indexer"], default="all",
                    help="profiling aid: run only the stack steps or only the indexer launches")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU runs are not supported "
                                   "(the path shards by sequence, see the design notes)"}))
        sys.exit(2)

    import numpy as np
    import torch

    from cross_layer_index_amd import ic
    from cross_layer_index_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = W.WORKLOADS[args.workload]
    R = max(1, args.sets)
    n = wl.n_valid()
    qs = ic.make_queries(wl.base(), n, wl.rows(), wl.same_seq, device=dev)
    d = ic.dims(wl.H_I, wl.D_I, wl.k, wl.H, wl.D_qk, wl.D_v)
    rmap = ic.reuse_map_last_full(wl.is_full())

    # ---- inputs: set 0 from the CPU generator (what the oracle sees), the
    # rest from the device generator with their own seeds
    host0 = [W.layer_inputs(wl, l) for l in range(wl.n_layers)] if not args.no_cpu_baseline else None
    sets = []
    for i in range(R):
        wli = wl if i == 0 else W.scaled(wl, seed=wl.seed * 1000 + i)
        lays = []
        for l in range(wl.n_layers):
            full = rmap[l] == l
            if i == 0 and host0 is not None:
                x = host0[l]
                li = W.LayerInputs(*[None if t is None else t.to(dev) for t in
                                     (x.q_idx, x.w, x.k_idx, x.q, x.kv, x.sink)])
            else:
                li = W.layer_inputs(wli, l, device=dev, with_indexer=full)
            out = torch.empty((wl.T, wl.H, wl.D_v), dtype=torch.bfloat16, device=dev)
            lays.append(dict(q_idx=li.q_idx, w=li.w, k_idx=li.k_idx, q=li.q, kv=li.kv, sink=li.sink, out=out))
        sets.append(ic.LayerStack(lays, rmap, qs, d, wl.scale, device=dev))
    torch.cuda.synchronize()

    # ---- graphs: one step per set, plus a long chain of R*4 steps
    def capture(fns):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for f in fns:          # warm the capture stream once
                f()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for f in fns:
                f()
        torch.cuda.synchronize()
        return g

    chain = 4 * R
    step_fns = [sets[i % R] for i in range(chain)]
    g_chain = capture(step_fns)
    g_one = [capture([sets[i]]) for i in range(R)]

    def run_steps(K):
        for _ in range(K // chain):
            g_chain.replay()
        for i in range(K % chain):
            g_one[i % R].replay()

    result = {}
    if args.only in ("all", "step"):
        run_steps(args.warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(args.steps)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        ms = el * 1e3 / args.steps
        ql_per_step = wl.T * wl.n_layers
        result.update(value=ql_per_step * args.steps / el, ms_per_step=ms)

    # ---- dominant kernel: the indexer, timed alone with events on its stream
    idx_ms = None
    if args.only in ("all", "indexer"):
        scores = [torch.empty((wl.T, ic.score_ld(qs.max_n)), dtype=torch.float32, device=dev) for _ in range(R)]
        full0 = rmap.index(0)

        def idx_fn(i):
            y = sets[i].layers[full0]
            return lambda: ic.indexer_score(y["q_idx"], y["w"], y["k_idx"], qs, scores[i])

        g_idx = capture([idx_fn(i % R) for i in range(chain)])
        for _ in range(max(1, args.warmup // chain)):
            g_idx.replay()
        reps = max(1, args.kernel_steps // chain)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g_idx.replay()
        e1.record()
        torch.cuda.synchronize()
        idx_ms = e0.elapsed_time(e1) / (reps * chain)

    if args.only != "all":
        print(json.dumps({"only": args.only, **result, "indexer_ms": idx_ms}))
        return

    nn = n.numpy()
    full_layers = sum(1 for l in range(wl.n_layers) if rmap[l] == l)
    idx_bytes = sum(indexer_bytes(int(x), wl.H_I, wl.D_I) for x in nn)
    achieved = idx_bytes / (idx_ms * 1e-3) / 1e9

    # ---- CPU baseline: the oracle on this host, rank 0 only
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        os.environ.setdefault("OMP_NUM_THREADS", str(threads))
        x = host0
        base, nv = wl.base().numpy(), nn
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.layer_stack(x, rmap, base, nv, wl.k, wl.scale, wl.D_v)
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        el = time.perf_counter() - t0
        cpu = {"value": reps * wl.T * wl.n_layers / el, "unit": "query-layers/s",
               "cores": int(os.environ.get("OMP_NUM_THREADS", threads)), "kind": "oracle",
               "sample": f"{reps} full passes of input set 0 ({wl.n_layers} layer(s) x {wl.T} query, "
                         f"L={int(nn.max())}) through the C oracle (fp64, OpenMP)"}

    line = {
        "metric": "decode query-layers/s at L=128K (index+topk+sparse MLA); % of HBM roofline",
        "value": result["value"],
        "unit": "query-layers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": result["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "L": int(nn.max()), "layers": wl.n_layers,
                   "full_layers": full_layers, "k": wl.k, "H_I": wl.H_I, "D_I": wl.D_I, "H": wl.H,
                   "D_qk": wl.D_qk, "D_v": wl.D_v, "rotating_sets": R, "graph": True},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "indexer_decode_kernel", "kernel_ms": idx_ms,
                     "algorithmic_bytes_per_launch": idx_bytes},
        "cpu_baseline": cpu,
    }
    step_bytes = sum(algorithmic_bytes(int(x), wl.k, wl.H_I, wl.D_I, wl.H, wl.D_qk, wl.D_v, rmap[l] == l)
                     for l in range(wl.n_layers) for x in nn)
    line["step_hbm_frac"] = step_bytes / (result["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS
    print(json.dumps(line))


if __name__ == "__main__":
    main()
