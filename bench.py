#!/usr/bin/env python3
"""Throughput of the IndexCache sparse-attention hot path on one MI355X.

A step is one pass of the whole path over one batch, through ic_layer_stack:
for every full layer indexer -> top-k -> stored index, for every layer sparse
MLA with sink over its (own or inherited) index. The default workload is one
full decode layer at batch 1 over a 131,072-token cache (indexer 64x128 fp8,
top-2048, MLA 128 heads over 576-wide bf16 latent rows). Inputs are resident in
HBM before timing starts; for the default workload R independently seeded input
sets are rotated so that the working set (R x ~168 MB) does not fit in the
256 MB Infinity Cache.

Prints one JSON line. The default line is the headline figure; --workload
selects the other synthetic workloads for reports (the 78-layer stack line
also carries the all-full-layers comparison).
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
METRIC = "decode query-layers/s at L=128K (index+topk+sparse MLA); % of HBM roofline"


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


def default_sets(wl, nn) -> int:
    """Input sets the timed steps rotate over: enough that the bytes one step
    touches, summed over the sets, reach 1 GiB -- four times the 256 MB
    last-level cache -- so every step reads its caches from HBM. Prefill
    (one shared sequence, matrix-core bound) uses one set."""
    if wl.same_seq:
        return 1
    per_step = indexer_launch_bytes(wl, nn) * sum(wl.is_full())
    per_step += sum(min(wl.k, x) * wl.D_qk * 2 for x in nn) * wl.n_layers
    return int(min(64, max(1, -(-(1 << 30) // per_step))))


def indexer_launch_bytes(wl, nn) -> int:
    """Algorithmic bytes of one indexer launch: every query's q and w, and the
    key rows of every sequence once (queries of a draft/verify group share
    their sequence's key stream, and causal prefill queries all read one)."""
    if wl.same_seq:
        return max(nn, default=0) * wl.D_I + len(nn) * wl.H_I * (wl.D_I + 4)
    g = max(1, wl.group)
    if g == 1:
        return sum(indexer_bytes(x, wl.H_I, wl.D_I) for x in nn)
    keys = sum(max(nn[i:i + g]) for i in range(0, len(nn), g)) * wl.D_I
    return keys + len(nn) * wl.H_I * (wl.D_I + 4)


def indexer_bytes(n: int, H_I: int, D_I: int) -> int:
    """Algorithmic bytes of one query's indexer pass: key rows + q + w."""
    return D_I * n + H_I * (D_I + 4)


def indexer_flops(n: int, H_I: int, D_I: int) -> int:
    return 2 * H_I * D_I * n


# source files whose text a kernel's counters were taken on
KERNEL_SOURCES = {
    "indexer_decode_kernel": ["indexer.hip", "radix_key.h"],
    "indexer_prefill_kernel": ["indexer.hip", "lds_dma.h"],
    "sparse_mla_kernel": ["sparse_mla.hip", "select.h", "lds_dma.h"],
    "sparse_mla_kernel<selecting>": ["sparse_mla.hip", "select.h", "lds_dma.h"],
    "mla_combine_kernel": ["sparse_mla.hip"],
    "topk_collect_kernel": ["topk.hip", "select.h", "radix_key.h"],
    "topk_finish_kernel": ["topk.hip", "select.h", "radix_key.h"],
    "topk_row_kernel": ["topk.hip", "select.h", "radix_key.h"],
    "indexer_prefill_sample": ["indexer.hip", "lds_dma.h"],
    "indexer_prefill_collect": ["indexer.hip", "radix_key.h", "lds_dma.h"],
    "prefill_bound_kernel": ["topk.hip", "select.h", "radix_key.h"],
    "prefill_select_kernel": ["topk.hip", "select.h", "radix_key.h"],
}


def source_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        h.update(open(os.path.join(ROOT, "cross_layer_index_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summaries (FETCH_SIZE and WRITE_SIZE, calibrated), if they were taken on
    the kernel's current source (else None)."""
    import glob
    import re
    digest = source_digest(kernel)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for m in re.finditer(r"<!-- traffic: (.*?) -->", open(path).read()):
            f = dict(kv.split("=", 1) for kv in m.group(1).split())
            if f.get("kernel") == kernel and f.get("workload") == workload and f.get("source_sha256") == digest:
                return float(f["bytes_per_launch"])
    return None


def kernel_work(name: str, wl, nn, full: bool, splits_combined: bool, collecting: bool = False):
    """Algorithmic bytes and flops of one launch of kernel `name` in one layer
    of the workload (the per-query-layer bytes of the method, split among the
    kernels that move them: score round trips, split partials and survivor
    lists are overhead and count nowhere). Returns (bytes, flops, flops_dtype)."""
    kp = [min(wl.k, x) for x in nn]
    if name in ("indexer_decode_kernel", "indexer_prefill_kernel", "indexer_prefill_collect"):
        if name == "indexer_prefill_kernel" and collecting:
            return 0, 0, None                                    # serves only queries the collection missed
        fl = sum(indexer_flops(x, wl.H_I, wl.D_I) for x in nn)
        return indexer_launch_bytes(wl, nn), fl, "fp8"
    if name == "indexer_prefill_sample":                         # one key in 64
        fl = sum(indexer_flops(-(-x // 64), wl.H_I, wl.D_I) for x in nn)
        return indexer_launch_bytes(wl, [-(-x // 64) for x in nn]), fl, "fp8"
    if name in ("topk_finish_kernel", "topk_row_kernel", "prefill_select_kernel"):
        if name == "topk_row_kernel" and collecting:
            return 0, 0, None
        return 4 * sum(kp), 0, None                              # the index list written
    if name in ("topk_collect_kernel", "clear_hist0_kernel"):
        return 0, 0, None
    if name.startswith("sparse_mla_kernel"):
        by = sum(4 * x + 2 * wl.D_qk * x for x in kp) + wl.T * wl.H * (2 * wl.D_qk + 4)
        if name.endswith("<selecting>"):
            by += 4 * sum(kp)                                    # it writes the layer's index list too
        if not splits_combined:
            by += wl.T * wl.H * 2 * wl.D_v                       # the output, when no combine follows
        fl = sum(wl.H * x * (2 * wl.D_qk + 2 * wl.D_v) for x in kp)
        return by, fl, "bf16"
    if name == "mla_combine_kernel":
        return wl.T * wl.H * 2 * wl.D_v, 0, None
    return 0, 0, None


def gpu_clocks():
    """Current and peak shader/memory clocks as reported by amd-smi (or
    rocm-smi), best effort; None when neither tool answers."""
    import subprocess
    for cmd in (["amd-smi", "metric", "--clock", "--json"], ["rocm-smi", "--showclocks", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
        except Exception:
            continue
        if r.returncode == 0 and r.stdout.strip():
            try:
                return {"tool": cmd[0], "clocks": json.loads(r.stdout)}
            except ValueError:
                return {"tool": cmd[0], "raw": r.stdout.strip()[:2000]}
    return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def reuse_overlap(ic, W, wl, st, rmap, qs, d, dev):
    """Mean fraction of a shared layer's own top-k that its inherited index
    also holds (each shared layer's own indexer run on its own inputs), over
    the shared layers and queries of one input set. On synthetic inputs the
    layers are independent, so the expected value is about k / L; it measures
    the machinery, not the quality of reuse."""
    import torch
    st()                                      # fills the index cache
    slots = {l: i for i, l in enumerate(l for l in range(wl.n_layers) if rmap[l] == l)}
    n = int(qs.max_n)
    fr = []
    for l in range(wl.n_layers):
        if rmap[l] == l:
            continue
        y = st.layers[l]
        own = ic.topk(ic.indexer_score(y["q_idx"], y["w"], y["k_idx"], qs), qs, wl.k)
        inh = st.index_cache[slots[rmap[l]]]
        mask = torch.zeros((wl.T, n + 1), dtype=torch.bool, device=dev)
        mask.scatter_(1, torch.where(inh >= 0, inh, n).long(), True)
        hit = torch.gather(mask, 1, torch.where(own >= 0, own, n).long()) & (own >= 0)
        fr.append((hit.sum(1).float() / (own >= 0).sum(1).clamp(min=1).float()).mean().item())
    return {"mean": sum(fr) / len(fr), "shared_layers": len(fr), "expected_independent": wl.k / n}


def shared_stacks(ic, sets, rmap, qs, d, scale, dev):
    """The sets' layers under another reuse map, sharing one workspace (the
    sets') and one index cache, as the sets themselves do."""
    out = []
    for s in sets:
        out.append(ic.LayerStack(s.layers, rmap, qs, d, scale, device=dev, ws=sets[0].ws,
                                 index_cache=out[0].index_cache if out else None))
    return out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="decode_128k",
                    choices=["decode_128k", "ragged_64", "stack_78", "prefill_1m", "mtp_verify", "tiny_2layer",
                             "decode_128k_recency"])
    ap.add_argument("--sets", type=int, default=None, help="rotating input sets (default: enough for 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--trace-steps", type=int, default=None, help="steps traced per kernel (per-kernel table)")
    ap.add_argument("--no-prefill-indexer", action="store_true",
                    help="leave out the one-launch prefill indexer figure of the default line")
    ap.add_argument("--only", choices=["all", "step", "copy", "floor"], default="all",
                    help="profiling aids: only the timed steps; only a plain 256 MiB device copy (the "
                         "calibration of the HBM traffic counters); only single-launch 16 MiB reads "
                         "(the floor of a launch that streams the indexer's key bytes)")
    return ap.parse_args()


def only_copy(torch, dev, n):
    src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(max(1, n)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"only": "copy", "bytes_read_per_copy": src.numel() * 4, "copies": n}))


def only_floor(torch, dev, steps):
    """Single launches that each read 16 MiB once in plain coalesced loads and
    do nothing else (ic_stream_read), over 64 rotating buffers (1 GiB, four
    times the last-level cache), replayed as one HIP graph: the time per
    launch is the floor of a single launch streaming the decode indexer's
    16 MiB of keys."""
    from cross_layer_index_amd import ic
    bufs = [torch.randint(0, 255, (1 << 24,), dtype=torch.uint8, device=dev) for _ in range(64)]
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    fns = [lambda b=b: ic.stream_read(b, sink) for b in bufs]
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(s_)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    reps = max(1, steps // len(fns))
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * len(fns))
    print(json.dumps({"only": "floor", "kernel": "stream_read_kernel", "bytes_read_per_launch": 1 << 24,
                      "launches": reps * len(fns), "us_per_launch": us, "GB/s": (1 << 24) / us / 1e3,
                      "hbm_frac": (1 << 24) / us / 1e3 / HBM_PEAK_GBS}))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "bench.py measures one GPU only; runs on several GPUs are not supported "
                                   "(decode shards by sequence with no exchange, so one GPU's figure is its share)"}))
        sys.exit(2)

    import torch

    from cross_layer_index_amd import ic
    from cross_layer_index_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only == "copy":
        return only_copy(torch, dev, max(1, args.steps))
    if args.only == "floor":
        return only_floor(torch, dev, args.steps)
    wl = W.WORKLOADS[args.workload]
    n = wl.n_valid()
    nn = [int(x) for x in n.tolist()]
    R = args.sets if args.sets is not None else default_sets(wl, nn)
    qs = ic.make_queries(wl.base(), n, wl.rows(), wl.same_seq, device=dev, group=wl.group)
    d = ic.dims(wl.H_I, wl.D_I, wl.k, wl.H, wl.D_qk, wl.D_v)
    rmap = ic.reuse_map_last_full(wl.is_full())
    small = wl.rows() * wl.D_qk * 2 * wl.n_layers < (1 << 30)
    cpu_wanted = not args.no_cpu_baseline and args.only == "all"

    # ---- inputs: set 0 of the small workloads from the CPU generator (what the
    # oracle sees), everything else from the device generator
    host0 = None
    if cpu_wanted and small:
        host0 = [W.layer_inputs(wl, l, with_indexer=(rmap[l] == l)) for l in range(wl.n_layers)]
    sets = []
    for i in range(R):
        lays = []
        for l in range(wl.n_layers):
            full = rmap[l] == l
            if host0 is not None and i == 0:
                x = host0[l]
                li = W.LayerInputs(*[None if t is None else t.to(dev) for t in
                                     (x.q_idx, x.w, x.k_idx, x.q, x.kv, x.sink)])
            else:
                # set i > 0: new values, the same geometry (qs describes every set)
                li = W.layer_inputs(wl, l, device=dev, with_indexer=full or wl.name == "stack_78", variant=i)
            out = torch.empty((wl.T, wl.H, wl.D_v), dtype=torch.bfloat16, device=dev)
            lays.append(dict(q_idx=li.q_idx, w=li.w, k_idx=li.k_idx, q=li.q, kv=li.kv, sink=li.sink, out=out))
        # one workspace and index cache for every set: steps never overlap,
        # and a decode loop reuses its scratch each step (only inputs rotate)
        sets.append(ic.LayerStack(lays, rmap, qs, d, wl.scale, device=dev,
                                  ws=sets[0].ws if sets else None,
                                  index_cache=sets[0].index_cache if sets else None))
    torch.cuda.synchronize()

    def capture(fns):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for f in fns:          # run once on the capture stream first
                f()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for f in fns:
                f()
        torch.cuda.synchronize()
        return g

    def runner(fns):
        """Callable running K steps (rotating over fns), through HIP graphs
        when a step is short enough for launch overhead to matter."""
        t0 = time.perf_counter()
        fns[0]()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 > 0.05:
            def run(K, prepare=False):
                if prepare:
                    return
                for i in range(K):
                    fns[i % len(fns)]()
            return run
        chain = len(fns) * max(1, -(-64 // len(fns)))      # >= 64 launches per graph
        g_chain = capture([fns[i % len(fns)] for i in range(chain)])
        tails = {}

        def run(K, prepare=False):
            r = K % chain
            if r and r not in tails:
                # one graph for the remainder too, so no launch gap is timed
                tails[r] = capture([fns[i % len(fns)] for i in range(r)])
            if prepare:
                return
            for _ in range(K // chain):
                g_chain.replay()
            if r:
                tails[r].replay()
        return run

    def timed(run, K, W_, blocks=1):
        """Time exactly K steps after W_ warmup steps, as `blocks` runs of
        consecutive steps between events (one bracketed region in all):
        returns the wall time, the event time and the per-step ms of each block."""
        run(W_)
        sizes = [K // blocks + (1 if b < K % blocks else 0) for b in range(blocks)]
        for sz in set(sizes):
            run(sz, prepare=True)          # any graph the timed steps need is built here
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
        t0 = time.perf_counter()
        ev[0].record()
        for b, sz in enumerate(sizes):
            run(sz)
            ev[b + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = [ev[b].elapsed_time(ev[b + 1]) / sizes[b] for b in range(blocks) if sizes[b]]
        return wall, ev[0].elapsed_time(ev[-1]) * 1e-3, per

    def step_launches(f):
        """The kernels one step launches, in order (the library's trace)."""
        tr = ic.Trace(4 * wl.n_layers + 8)
        with tr:
            f()
        torch.cuda.synchronize()
        return [name for name, _ in tr.read()]

    def kernel_costs(fns, names, full_step_s, K, W_):
        """Each kernel's cost in the step, measured as the timed step (HIP
        events around graph replays of the rotating sets) minus the same step
        with that kernel left out (ic_trace_skip), per launch."""
        out = {}
        for name in sorted(set(names)):
            def skipping(f, name=name):
                def g():
                    with ic.SkipKernel(name):
                        f()
                return g
            _, ev, _ = timed(runner([skipping(f) for f in fns]), K, W_)
            out[name] = (full_step_s - ev / K) / names.count(name)
        return out

    big = wl.name in ("stack_78", "prefill_1m")
    steps = min(args.steps, 20) if big else args.steps
    warm = min(args.warmup, 2) if big else args.warmup
    result = {}
    run = runner(sets)
    el, ev_s, per = timed(run, steps, warm, blocks=5 if steps >= 5 else 1)
    result.update(value=wl.T * wl.n_layers * steps / el, ms_per_step=el * 1e3 / steps)
    per_sorted = sorted(per)
    result["repeats"] = {"blocks": len(per), "ms_per_step_mean": sum(per) / len(per),
                         "ms_per_step_median": per_sorted[len(per) // 2], "ms_per_step_min": per_sorted[0],
                         "ms_per_step_max": per_sorted[-1], "event_ms_per_step": ev_s * 1e3 / steps}
    if args.only == "step":
        print(json.dumps({"only": "step", "workload": wl.name, **result}))
        return
    if wl.name == "stack_78":
        ident = list(range(wl.n_layers))
        allfull = shared_stacks(ic, sets, ident, qs, d, wl.scale, dev)
        el2, _, _ = timed(runner(allfull), steps, warm)
        result["all_full"] = {"value": wl.T * wl.n_layers * steps / el2, "ms_per_step": el2 * 1e3 / steps,
                              "indexer_passes": wl.n_layers}
        result["indexcache_speedup"] = el2 / el
        del allfull
        # reuse-pattern variants: the same stack and inputs under other full-layer sets
        pats = {}
        for name, fl in W.REUSE_PATTERNS.items():
            m = ic.reuse_map_last_full([l in set(fl) for l in range(wl.n_layers)])
            st = shared_stacks(ic, sets, m, qs, d, wl.scale, dev)
            elp, _, _ = timed(runner(st), steps, warm)
            pats[name] = {"indexer_passes": len(fl), "ms_per_step": elp * 1e3 / steps,
                          "value": wl.T * wl.n_layers * steps / elp, "speedup_vs_all_full": el2 / elp}
            del st
        result["reuse_patterns"] = pats
        result["reuse_overlap"] = reuse_overlap(ic, W, wl, sets[0], rmap, qs, d, dev)

    # ---- every kernel of the step: its cost in the graph-replayed step, the
    # step's time (HIP events) less the time of the same step without it
    names = step_launches(sets[0])
    full_step_s = ev_s / steps
    costs = kernel_costs(sets, names, full_step_s, steps, warm)
    n_full = sum(1 for l in range(wl.n_layers) if rmap[l] == l)
    combined = "mla_combine_kernel" in costs
    collecting = "indexer_prefill_collect" in costs
    table = []
    for name, sec in costs.items():
        per_step = names.count(name)
        us = sec * 1e6
        by, fl, fdt = kernel_work(name, wl, nn, True, combined, collecting)
        row = {"kernel": name, "launches_per_step": per_step, "us_per_launch": us,
               "us_per_step": us * per_step, "algorithmic_bytes_per_launch": by}
        if by and us > 0:
            row["GB/s"] = by / (us * 1e-6) / 1e9
            row["hbm_frac"] = row["GB/s"] / HBM_PEAK_GBS
        if fl and us > 0:
            peak = FP8_PEAK_TFLOPS if fdt == "fp8" else BF16_PEAK_TFLOPS
            row["algorithmic_flops_per_launch"] = fl
            row["TFLOP/s"] = fl / (us * 1e-6) / 1e12
            row[f"{fdt}_mfma_frac"] = row["TFLOP/s"] / peak
        table.append(row)
    table.sort(key=lambda r: -r["us_per_step"])
    dom = table[0]
    by, fl, fdt = kernel_work(dom["kernel"], wl, nn, True, combined, collecting)
    mfma_bound = fl and (fl / (FP8_PEAK_TFLOPS if fdt == "fp8" else BF16_PEAK_TFLOPS) / 1e12 >
                         by / HBM_PEAK_GBS / 1e9)
    if mfma_bound:
        peak = FP8_PEAK_TFLOPS if fdt == "fp8" else BF16_PEAK_TFLOPS
        achieved = fl / (dom["us_per_launch"] * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                "traffic": measured_traffic(dom["kernel"], wl.name), "kernel": dom["kernel"],
                "kernel_ms": dom["us_per_launch"] * 1e-3, "algorithmic_flops_per_launch": fl,
                "flops_dtype": fdt}
    else:
        achieved = by / (dom["us_per_launch"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(dom["kernel"], wl.name),
                "kernel": dom["kernel"], "kernel_ms": dom["us_per_launch"] * 1e-3,
                "algorithmic_bytes_per_launch": by}
    roof["share_of_step"] = dom["us_per_step"] * 1e-3 / result["ms_per_step"]

    # ---- the chunked-prefill indexer (1M-token cache, 4096 causal queries),
    # one launch as the prefill workload runs it, timed on the default line
    pf = None
    if args.only == "all" and wl.name == "decode_128k" and not args.no_prefill_indexer:
        pw = W.WORKLOADS["prefill_1m"]
        pn = pw.n_valid()
        pqs = ic.make_queries(pw.base(), pn, pw.rows(), True, device=dev)
        pli = W.layer_inputs(W.scaled(pw, D_qk=8, D_v=8, H=1), 0, device=dev)   # indexer tensors only matter
        psc = torch.empty((pw.T, ic.score_ld(pqs.max_n)), dtype=torch.float32, device=dev)
        fn = lambda: ic.indexer_score(pli.q_idx, pli.w, pli.k_idx, pqs, psc)
        fn()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        for i in range(3):
            fn()
            e[i + 1].record()
        torch.cuda.synchronize()
        ms = [e[i].elapsed_time(e[i + 1]) for i in range(3)]
        pfl = sum(indexer_flops(int(x), pw.H_I, pw.D_I) for x in pn.tolist())
        pf = {"workload": "prefill_1m indexer (4096 causal queries over 1,048,576 tokens, 64x128 fp8)",
              "launches": 3, "ms_per_launch": sum(ms) / 3, "ms_min": min(ms),
              "algorithmic_flops_per_launch": pfl, "TFLOP/s": pfl / (sum(ms) / 3 * 1e-3) / 1e12,
              "fp8_mfma_frac": pfl / (sum(ms) / 3 * 1e-3) / 1e12 / FP8_PEAK_TFLOPS}
        del psc, pli

    # ---- the step after the path: gated head output (wv_b, sigmoid gate) for
    # this workload's queries, timed alone over rotating inputs
    gate = None
    if args.only == "all" and wl.D_v == 512 and wl.name in ("decode_128k", "mtp_verify", "prefill_1m"):
        D_o, NG = 128, 8
        gsets = [W.gate_inputs(W.scaled(wl, seed=wl.seed + 100 + i), 0, D_o, device=dev) for i in range(NG)]
        gouts = torch.empty((wl.T, wl.H, D_o), dtype=torch.bfloat16, device=dev)
        gfns = [lambda x=x: ic.gated_output(x.o, x.wv_b, x.gate, out=gouts) for x in gsets]
        grun = runner(gfns)
        gk = 8 * NG
        _, gev, _ = timed(grun, gk, NG)
        g_s = gev / gk
        gbytes = 2 * (wl.H * D_o * wl.D_v + wl.T * wl.H * (wl.D_v + 2 * D_o))
        gflops = 2 * wl.T * wl.H * D_o * wl.D_v
        gate = {"T": wl.T, "H": wl.H, "D_v": wl.D_v, "D_o": D_o, "us": g_s * 1e6,
                "GB/s": gbytes / g_s / 1e9, "hbm_frac": gbytes / g_s / 1e9 / HBM_PEAK_GBS,
                "TFLOP/s": gflops / g_s / 1e12, "bf16_mfma_frac": gflops / g_s / 1e12 / BF16_PEAK_TFLOPS}
        del gsets

    # ---- the step before the path: the cache write of the tokens this
    # workload's queries add (indexer key: LayerNorm, RoPE, fp8 cast; latent
    # row: copy and RoPE), timed alone over rotating inputs at the workload's
    # positions, into caches of T rows
    wpath = None
    if args.only == "all" and wl.D_v == 512 and wl.name in ("decode_128k", "mtp_verify", "ragged_64", "prefill_1m"):
        NW = 8
        D_rope = W.d_rope(wl)
        table_r = W.rope_table(max(1, max(nn)), D_rope).to(dev)
        kc = torch.empty((wl.T, wl.D_I), dtype=torch.uint8, device=dev)
        kvc = torch.empty((wl.T, wl.D_qk), dtype=torch.bfloat16, device=dev)
        dst = torch.arange(wl.T, dtype=torch.int64, device=dev)
        wfns = []
        for i in range(NW):
            x = W.write_inputs(wl, i, device=dev, rope=table_r)
            tk = ic.Tokens(dst, x.pos, wl.T, table_r)
            wfns.append(lambda x=x, tk=tk: ic.write_cache(tk, x.k_pre, x.ln_w, x.ln_b, x.eps, kc, x.kv_pre, kvc))
        wk = 8 * NW
        _, wev, _ = timed(runner(wfns), wk, NW)
        w_s = wev / wk
        per_tok = 3 * wl.D_I + 4 * wl.D_qk + 4 * D_rope + 12
        wbytes = wl.T * per_tok + 8 * wl.D_I
        wpath = {"T": wl.T, "D_I": wl.D_I, "D_qk": wl.D_qk, "D_rope": D_rope, "us": w_s * 1e6,
                 "bytes_per_token": per_tok, "GB/s": wbytes / w_s / 1e9,
                 "hbm_frac": wbytes / w_s / 1e9 / HBM_PEAK_GBS}
        del wfns, table_r

    # ---- CPU baseline: the oracle on this host, on a bounded sample
    cpu = None
    if cpu_wanted:
        import oracle
        threads = len(os.sched_getaffinity(0))
        if host0 is not None:
            x, base, nv, layers_used, qn = host0, wl.base().numpy(), n.numpy(), wl.n_layers, wl.T
            sample = f"full passes of input set 0 ({wl.n_layers} layer(s) x {wl.T} queries)"
            rm = rmap
        else:
            # one query through a full and a shared layer, copied back from the device
            import numpy as np
            t = 0
            rows = slice(int(qs.base[t]), int(qs.base[t]) + nn[t])
            src = sets[0].layers
            l_sh = next((l for l in range(wl.n_layers) if rmap[l] != l), None)
            used = [0] + ([l_sh] if l_sh is not None else [])

            class L:
                pass
            x = []
            for j, l in enumerate(used):
                o = L()
                y = src[l]
                o.q_idx = y["q_idx"][t:t + 1].cpu() if j == 0 else None
                o.w = y["w"][t:t + 1].cpu() if j == 0 else None
                o.k_idx = y["k_idx"][rows].cpu() if j == 0 else None
                o.q, o.kv, o.sink = y["q"][t:t + 1].cpu(), y["kv"][rows].cpu(), y["sink"].cpu()
                x.append(o)
            rm = [0] + ([0] if l_sh is not None else [])
            base, nv, layers_used, qn = np.array([0], np.int64), np.array([nn[t]], np.int32), len(used), 1
            sample = (f"query 0 through a full{' and a shared' if l_sh is not None else ''} layer "
                      f"(L={nn[t]}), repeated")
        reps_c, t0 = 0, time.perf_counter()
        while True:
            oracle.layer_stack(x, rm, base, nv, wl.k, wl.scale, wl.D_v)
            reps_c += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        el_c = time.perf_counter() - t0
        cpu = {"value": reps_c * qn * layers_used / el_c, "unit": "query-layers/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{reps_c} x {sample} through the C oracle (fp64, OpenMP, {threads} threads)"}

    line = {
        "metric": METRIC if wl.name == "decode_128k" else f"{wl.name} query-layers/s (index+topk+sparse MLA)",
        "value": result["value"],
        "unit": "query-layers/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": result["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "L": max(nn) if nn else 0, "layers": wl.n_layers,
                   "full_layers": n_full, "k": wl.k, "H_I": wl.H_I, "D_I": wl.D_I, "H": wl.H,
                   "D_qk": wl.D_qk, "D_v": wl.D_v, "rotating_sets": R},
        "roofline": roof,
        "cpu_baseline": cpu,
        "repeats": result["repeats"],
        "kernels": table,
        "kernel_costs": {"launches_per_step": len(names), "step_us_events": full_step_s * 1e6,
                         "sum_of_kernel_us": sum(r["us_per_step"] for r in table),
                         "method": "per kernel: (timed step - the same step with that kernel left out, "
                                   "ic_trace_skip) / launches, both timed with HIP events around graph "
                                   "replays of the rotating input sets"},
    }
    if not wl.same_seq:
        # per-query byte counts hold only where queries read caches of their own;
        # prefill queries share one key and latent cache, and that path is MFMA-bound
        step_bytes = sum(algorithmic_bytes(x, wl.k, wl.H_I, wl.D_I, wl.H, wl.D_qk, wl.D_v, rmap[l] == l)
                         for l in range(wl.n_layers) for x in nn)
        # a draft/verify group streams its sequence's keys once
        step_bytes -= n_full * (sum(indexer_bytes(x, wl.H_I, wl.D_I) for x in nn) - indexer_launch_bytes(wl, nn))
        line["step_hbm_frac"] = step_bytes / (result["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS
        line["step_algorithmic_bytes"] = step_bytes
    for k2 in ("all_full", "indexcache_speedup", "reuse_patterns", "reuse_overlap"):
        if k2 in result:
            line[k2] = result[k2]
    if pf is not None:
        line["prefill_indexer"] = pf
    if gate is not None:
        line["gated_output"] = gate
    if wpath is not None:
        line["write_path"] = wpath
    line["host"] = {"cpu_model": cpu_model(), "threads": len(os.sched_getaffinity(0))}
    line["gpu"] = {"name": torch.cuda.get_device_name(dev), "clocks": gpu_clocks()}
    print(json.dumps(line))


if __name__ == "__main__":
    main()
