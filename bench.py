"""Benchmark of the routed-MoE layer (Gemma 4 26B-A4B shape, Q4_0 experts) on one MI355X.

One step = one pass of the whole layer (router + top-K, permutation, expert
FFN, combine) over one batch of synthetic tokens.  Default workload: 1-token
decode (H 2816, 128 experts, top-8, I 704, fp32 activations).  Inputs are
resident in HBM before timing.  To keep the 256 MB Infinity Cache from
serving the expert weights, steps rotate over several independently seeded
weight sets (as consecutive layers of a model would).

Prints one JSON line with the metric, the roofline of the dominant kernel
(the expert FFN call) measured with HIP events on the launch stream, and the
single-threaded CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "MoE-layer tokens/sec at 1 MI355X; decode HBM GB/s %peak, prefill MFMA %peak"
Q4_0_EXPERT_BYTES = lambda H, I: 3 * H * I // 32 * 18   # [gate; up] + down
# stored PMC traffic is reported only while the kernel sources are unchanged
KERNEL_SOURCE_DIR = "sparse_moe_amd/csrc"
# kernels of the call the roofline times: the decode layer call, or the expert FFN
DECODE_KERNELS = ("router_logits_gemv", "decode_ffn_one", "decode_gate_up", "decode_down_combine")
FFN_KERNELS = ("ffn_gemv_q4_0", "ffn_mfma")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=1,
                   help="workload: 0 tiny, 1 decode 1 token, 2 decode 8 tokens, 3 prefill 4096, "
                        "4 stack of 30 layers x 512 tokens")
    p.add_argument("--sets", type=int, default=0,
                   help="weight sets in distinct memory (0: 32 for decode, 4 for prefill)")
    p.add_argument("--no-prefill", action="store_true",
                   help="default workload only: leave out the nested 4,096-token prefill leg")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="first copy MIB MiB device to device (a dispatch of known size for "
                        "scaling FETCH_SIZE / WRITE_SIZE counters)")
    # no-GPU helpers that turn rocprofv3 output into the summaries kept in profiles/
    p.add_argument("--summarize-stats", nargs=4, metavar=("CSV_DIR", "OUT_MD", "TITLE", "CMD"),
                   help="write a markdown summary of a --kernel-trace --stats run")
    p.add_argument("--summarize-traffic", nargs=4,
                   metavar=("FETCH_DIR", "WRITE_DIR", "CALIB_MIB", "CMD"),
                   help="store the HBM traffic per roofline call of --config's workload from "
                        "two --pmc runs (FETCH_SIZE, WRITE_SIZE) made with --copy-calibration")
    return p.parse_args()


def ffn_source_digest() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, KERNEL_SOURCE_DIR)
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def stored_traffic(workload: str):
    """HBM bytes per expert-FFN call from the PMC runs kept in profiles/, or None
    when there are none for this workload or the FFN sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            entry = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not entry or entry.get("ffn_source_sha256") != ffn_source_digest():
        return None
    return entry


def _pmc_means(csv_dir: str, counter: str):
    """Per kernel name: mean of `counter` over its dispatches; also the largest
    value among the runtime's copy kernels (the calibration copy)."""
    sums, counts, copy_max = {}, {}, 0.0
    with open(os.path.join(csv_dir, "run_counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            v, name = float(r["Counter_Value"]), r["Kernel_Name"]
            if "rocclr_copyBuffer" in name:
                copy_max = max(copy_max, v)
            sums[name] = sums.get(name, 0.0) + v
            counts[name] = counts.get(name, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}, copy_max


def summarize_traffic(args):
    from sparse_moe_amd import synth
    fetch_dir, write_dir, calib_mib, cmd = args.summarize_traffic
    calib = float(calib_mib) * 1024  # KiB
    spec = synth.SPECS[args.config]
    out = {}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        means, copy_kib = _pmc_means(d, counter)
        if copy_kib <= 0:
            sys.exit("no calibration copy found in %s" % d)
        scale = calib / copy_kib
        names = DECODE_KERNELS if decode_path(spec.T, spec.H, spec.I, spec.K) else FFN_KERNELS
        ffn = {k: v for k, v in means.items() if any(n in k for n in names)}
        out[key + "_bytes"] = sum(ffn.values()) * 1024 * scale
        out[key + "_scale"] = scale
        out[key + "_kib_per_kernel"] = {
            k.replace("(anonymous namespace)::", "").split("(")[0]: v for k, v in ffn.items()}
    out["traffic_bytes"] = out["fetch_bytes"] + out["write_bytes"]
    out["ffn_source_sha256"] = ffn_source_digest()
    out["commands"] = cmd
    try:
        with open(TRAFFIC_FILE) as fh:
            allw = json.load(fh)
    except (OSError, ValueError):
        allw = {}
    allw[spec.name] = out
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(allw, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({spec.name: out}))


def summarize_stats(args):
    csv_dir, out_md, title, cmd = args.summarize_stats
    with open(os.path.join(csv_dir, "run_kernel_stats.csv")) as fh:
        rows = list(csv.DictReader(fh))
    with open(out_md, "w") as f:
        f.write("# %s\n\n" % title)
        f.write("Command (from the repository root on one MI355X, rocprofv3 of ROCm 7.2):\n\n"
                "```\n%s\n```\n\n" % cmd)
        f.write("Calls include the warm-up, the eager passes and the graph replays; the torch "
                "kernels are bench set-up.\n\n")
        f.write("| kernel | calls | avg (us) | min (us) | max (us) | share of GPU time |\n"
                "|---|---|---|---|---|---|\n")
        for r in rows[:14]:
            name = r["Name"].replace("|", "\\|")
            if len(name) > 110:
                name = name[:107] + "..."
            f.write("| `%s` | %s | %.2f | %.2f | %.2f | %.1f%% |\n" % (
                name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    print("wrote", out_md)


def host_info():
    """Cores this process may use, and the host CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_cores": len(os.sched_getaffinity(0)), "host_cores_total": os.cpu_count(),
            "cpu_model": model}


class one_core:
    """Pin this process to one of its cores while the oracle runs."""

    def __enter__(self):
        self.saved = os.sched_getaffinity(0)
        self.core = min(self.saved)
        os.sched_setaffinity(0, {self.core})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.saved)


def cpu_baseline(spec, seconds: float):
    """The oracle as it stands, single-threaded and pinned to one core, on a
    bounded token sample."""
    import oracle
    from sparse_moe_amd import synth
    if spec.layers > 1:
        return cpu_baseline_stack(spec, seconds)
    info = host_info()
    L = synth.make_layer(spec, T=1)
    xs = synth.activations(spec, 64, spec.seed + 77)
    oracle.lib()
    with one_core() as pin:
        n, t0 = 0, time.perf_counter()
        while n < xs.shape[0]:
            oracle.moe_layer(xs[n:n + 1], L.w_router, L.w_gate_up, L.w_down, spec.K,
                             scale=L.expert_scale, bias=L.router_bias)
            n += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "pinned_core": pin.core, **info,
            "sample": "%d tokens of the %s layer, one at a time, full layer per token "
                      "(router over all experts, top-%d, %d expert FFNs, combine), "
                      "single-threaded binary64 C oracle pinned to one core"
                      % (n, spec.name, spec.K, spec.K)}


def bench_stack(args, spec):
    """Stack workload: one step = all layers (RMSNorm -> routing -> expert FFN ->
    combine with residual) over one chunk; every layer has its own weights, all
    resident (no rotation needed: 30 layers of experts far exceed the caches)."""
    import torch
    from sparse_moe_amd import binding, synth
    T, H, E, K, I = spec.T, spec.H, spec.E, spec.K, spec.I
    dev = "cuda"

    def dev_t(a):
        import numpy as np
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    layers = []
    for l in range(spec.layers):
        L = synth.make_layer(spec, seed=synth.stack_layer_seed(l), with_x=False)
        layers.append(dict(wr=dev_t(L.w_router), gu=dev_t(L.w_gate_up), dn=dev_t(L.w_down),
                           sc=dev_t(L.expert_scale), bias=dev_t(L.router_bias),
                           rw=dev_t(L.rms_w)))
        del L
    x0 = dev_t(synth.activations(spec, T, spec.seed))
    xa, xb, xhat = x0.clone(), torch.empty_like(x0), torch.empty_like(x0)
    bufs = [binding.LayerBuffers(T, H, I, E, K, torch.bfloat16) for _ in range(2)]

    def step(evs=None):
        xin, xout = xa, xb
        xin.copy_(x0)
        for l, w in enumerate(layers):
            b = bufs[l & 1]
            binding.moe_rmsnorm(xin, w["rw"], spec.rms_eps, xhat)
            binding.moe_route(xhat, w["wr"], b.logits, b.topk_ids, b.topk_w, b.offsets,
                              b.sorted_slots, b.slot_pos, b.ws_route, logit_bias=w["bias"])
            if evs is not None:
                evs[l][0].record()
            binding.moe_expert_ffn_q4_0(xhat, w["gu"], w["dn"], K, b.offsets, b.sorted_slots,
                                        b.y_sorted, b.ws_ffn)
            if evs is not None:
                evs[l][1].record()
            binding.moe_combine(b.y_sorted, b.slot_pos, b.topk_ids, b.topk_w, w["sc"],
                                residual=xin, out_act=xout, out_f32=b.out)
            xin, xout = xout, xin

    # distinct experts per layer (for the algorithmic bytes)
    distinct = []
    xin, xout = xa, xb
    xin.copy_(x0)
    for l, w in enumerate(layers):
        b = bufs[0]
        binding.moe_rmsnorm(xin, w["rw"], spec.rms_eps, xhat)
        binding.moe_route(xhat, w["wr"], b.logits, b.topk_ids, b.topk_w, b.offsets,
                          b.sorted_slots, b.slot_pos, b.ws_route, logit_bias=w["bias"])
        binding.moe_expert_ffn_q4_0(xhat, w["gu"], w["dn"], K, b.offsets, b.sorted_slots,
                                    b.y_sorted, b.ws_ffn)
        binding.moe_combine(b.y_sorted, b.slot_pos, b.topk_ids, b.topk_w, w["sc"],
                            residual=xin, out_act=xout, out_f32=b.out)
        torch.cuda.synchronize()
        distinct.append(int((b.offsets[1:] - b.offsets[:-1] > 0).sum().item()))
        xin, xout = xout, xin
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    out_graph = (xa if spec.layers % 2 == 0 else xb).clone()
    step()
    torch.cuda.synchronize()
    assert torch.equal(out_graph, xa if spec.layers % 2 == 0 else xb), "graph replay differs"

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in layers]
    reps = max(1, min(args.steps, 5))
    ffn_ms = [0.0] * len(layers)
    for _ in range(reps):
        step(evs)
        torch.cuda.synchronize()
        for l, (a, b) in enumerate(evs):
            ffn_ms[l] += a.elapsed_time(b) / reps
    expert_bytes = Q4_0_EXPERT_BYTES(H, I)
    N = T * K
    ffn_flops = N * 6.0 * H * I
    ffn_total_ms = sum(ffn_ms)
    ffn_bytes = [d * expert_bytes + T * H * 2 + N * I * 2 * 2 + N * H * 4 for d in distinct]
    achieved_gbs = sum(ffn_bytes) / (ffn_total_ms * 1e-3) / 1e9
    achieved_tf = ffn_flops * len(layers) / (ffn_total_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": T * args.steps / (ms_total * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "q4_0 x bf16 (exact bf16 MFMA products, fp32 accumulate)",
        "data": "synthetic (seeded; random-init Q4_0 experts, one weight set per layer)",
        "config": {"workload": "%s: %d Gemma-4-26B-A4B-shaped routed-MoE layers with RMSNorm and "
                               "residual, T=%d, H=%d, E=%d, top-%d, I=%d, Zipf(%.1f) router prior, "
                               "bf16 activations" % (spec.name, spec.layers, T, H, E, K, I,
                                                     spec.zipf_s),
                   "tokens_per_step": T, "layers": spec.layers,
                   "distinct_experts_per_layer_mean": sum(distinct) / len(distinct),
                   "distinct_experts_per_layer_min_max": [min(distinct), max(distinct)],
                   "ffn_mfma_tflops": achieved_tf, "ffn_mfma_frac": achieved_tf / BF16_PEAK_TFLOPS,
                   "wall_s": wall, "timing": "K steps, each a replay of one HIP graph of all layers"},
        "roofline": {"kernel": "moe_expert_ffn_q4_0 over the layers (activation prep, gate/up and "
                               "down bf16 MFMA grouped GEMM launches)",
                     "bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": None,
                     "bytes_per_launch": sum(ffn_bytes) / len(ffn_bytes),
                     "avg_launch_us": ffn_total_ms / len(layers) * 1e3},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def cpu_baseline_stack(spec, seconds: float):
    """Stack workload: tokens one at a time through the first two layers (RMSNorm,
    layer, residual), the rate scaled to all layers."""
    import numpy as np
    import oracle
    from sparse_moe_amd import synth
    Ls = [synth.make_layer(spec, seed=synth.stack_layer_seed(l), T=1, with_x=False) for l in range(2)]
    xs = synth.activations(spec, 64, spec.seed + 77)
    info = host_info()
    oracle.lib()
    with one_core() as pin:
        n, t0 = 0, time.perf_counter()
        while n < xs.shape[0]:
            x = xs[n:n + 1]
            for L in Ls:
                x = oracle.stack_layer(x, L.rms_w, spec.rms_eps, L.w_router, L.w_gate_up,
                                       L.w_down, spec.K, scale=L.expert_scale,
                                       bias=L.router_bias)["x_next"]
            n += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    per_token_layer = dt / (n * len(Ls))
    return {"value": 1.0 / (per_token_layer * spec.layers), "unit": "tokens/s", "cores": 1,
            "kind": "oracle", "pinned_core": pin.core, **info,
            "sample": "%d tokens one at a time through 2 of the %d layers (RMSNorm, router with "
                      "Zipf prior over all experts, top-%d, %d expert FFNs, combine, residual), "
                      "single-threaded binary64 C oracle pinned to one core; rate scaled to %d "
                      "layers" % (n, spec.layers, spec.K, spec.K, spec.layers)}


def mfma_path(act: str, T: int, H: int, I: int) -> bool:
    """Whether moe_expert_ffn_q4_0 takes its bf16 MFMA path (the library's
    dispatch rule, include/sparse_moe.h): bf16 activations, at least 64 tokens,
    H and I multiples of 64."""
    return act == "bf16" and T >= 64 and H % 64 == 0 and I % 64 == 0


def decode_path(T: int, H: int, I: int, K: int) -> bool:
    """Whether the step runs as one moe_layer_decode call: a single token (the
    call serves up to 8 tokens, but from 2 tokens the four calls are faster),
    H and I multiples of 64."""
    return T == 1 and H % 64 == 0 and I % 64 == 0 and K <= 16 and K * (I // 32) * 68 <= 65536


def dev_tensor(a, dev="cuda"):
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def weight_sets(spec, n: int, dev="cuda"):
    """n weight sets of one layer, each in its own device memory: a seeded
    synthetic layer, and n - 1 copies with the experts (and the router rows,
    scales and prior that belong to them) stored in a seeded random order.  A
    token routes to the same expert contents in every set, at different
    addresses, so no set finds another's experts in a cache."""
    import torch
    from sparse_moe_amd import synth
    L = synth.make_layer(spec, seed=spec.seed + 1000, with_x=False)
    base = dict(wr=dev_tensor(L.w_router, dev), gu=dev_tensor(L.w_gate_up, dev),
                dn=dev_tensor(L.w_down, dev), sc=dev_tensor(L.expert_scale, dev),
                bias=None if L.router_bias is None else dev_tensor(L.router_bias, dev))
    del L
    sets = [base]
    gen = torch.Generator().manual_seed(spec.seed + 2000)
    for _ in range(1, n):
        perm = torch.randperm(spec.E, generator=gen).to(dev)
        sets.append({k: None if v is None else v.index_select(0, perm).contiguous()
                     for k, v in base.items()})
    return sets


def bench_layer(spec, steps: int, warmup: int, nsets: int, cpu_seconds: float = 0.0):
    """One routed-MoE layer (routing, expert FFN, combine): K timed steps, each a
    replay of one of G HIP graphs, graph r running weight set r mod nsets on
    token batch r, so consecutive uses of a set are nsets graphs apart and a
    cycle touches G different routings; then the expert-FFN call alone, timed
    over replays of one graph of F calls, call f on set f with the routing of
    batch f."""
    import torch
    from sparse_moe_amd import binding, synth
    T, H, E, K, I = spec.T, spec.H, spec.E, spec.K, spec.I
    act = torch.float32 if spec.act == "f32" else torch.bfloat16
    sets = weight_sets(spec, nsets)
    G = nsets * (2 if T <= 64 else 1)
    F = nsets
    xpool = dev_tensor(synth.activations(spec, T * G, spec.seed + 7)).view(G, T, H)
    bufs = binding.LayerBuffers(T, H, I, E, K, act)

    def route(r, si=None):
        s = sets[r % nsets if si is None else si]
        binding.moe_route(xpool[r], s["wr"], bufs.logits, bufs.topk_ids, bufs.topk_w, bufs.offsets,
                          bufs.sorted_slots, bufs.slot_pos, bufs.ws_route, logit_bias=s["bias"])

    # decode batches run as one moe_layer_decode call (router logits, gate/up with
    # the routing inside, down with the combine inside), others as the four calls
    fused = decode_path(T, H, I, K)

    def step(r, si=None):
        s = sets[r % nsets if si is None else si]
        if fused:
            binding.moe_layer_decode(xpool[r], s["wr"], s["gu"], s["dn"], K, expert_scale=s["sc"],
                                     logit_bias=s["bias"], bufs=bufs)
            return
        route(r, si)
        binding.moe_expert_ffn_q4_0(xpool[r], s["gu"], s["dn"], K, bufs.offsets,
                                    bufs.sorted_slots, bufs.y_sorted, bufs.ws_ffn)
        binding.moe_combine(bufs.y_sorted, bufs.slot_pos, bufs.topk_ids, bufs.topk_w, s["sc"],
                            out_f32=bufs.out)

    # routing of every batch (distinct experts for the algorithmic bytes; the FFN
    # timing graph's per-call routing)
    distinct, routes = [], []
    for r in range(G):
        route(r)
        torch.cuda.synchronize()
        distinct.append(int((bufs.offsets[1:] - bufs.offsets[:-1] > 0).sum().item()))
        if r < F:
            routes.append((bufs.offsets.clone(), bufs.sorted_slots.clone()))
    # every set holds the same experts in another order: one batch's output is the
    # same, bit for bit, whatever the set
    step(0)
    torch.cuda.synchronize()
    out0 = bufs.out.clone()
    if nsets > 1:
        step(0, si=nsets - 1)
        torch.cuda.synchronize()
        assert torch.equal(out0, bufs.out), "weight sets disagree"
    for r in range(warmup):
        step(r % G)
    torch.cuda.synchronize()
    # S consecutive steps per HIP graph (like consecutive layers of a model in
    # one graph), so that the timed loop does not measure the host's per-replay
    # launch cost; graph j holds steps S j .. S j + S - 1
    S = next(s for s in (8, 4, 2, 1) if T <= 64 and steps % s == 0 and G % s == 0 or s == 1)
    NG = G // S
    graphs = []
    for j in range(NG):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(S * j, S * j + S):
                step(r)
        graphs.append(g)
    for i in range(warmup):
        graphs[i % NG].replay()
    torch.cuda.synchronize()
    # a replay reproduces the eager steps bit for bit (the last step's output)
    for j in (0, NG - 1):
        graphs[j].replay()
        torch.cuda.synchronize()
        out_g = bufs.out.clone()
        step(S * j + S - 1)
        torch.cuda.synchronize()
        assert torch.equal(out_g, bufs.out), "graph replay differs from eager execution"

    # timed region: K steps as K / S graph replays
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record()
    for i in range(steps // S):
        graphs[i % NG].replay()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = t_start.elapsed_time(t_end) / steps

    # dominant call, with HIP events on its stream around replays of one graph of
    # F calls (no host launch gap timed): the decode layer call, or else the
    # expert-FFN call
    g_ffn = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_ffn):
        for f in range(F):
            s = sets[f]
            if fused:
                binding.moe_layer_decode(xpool[f], s["wr"], s["gu"], s["dn"], K,
                                         expert_scale=s["sc"], logit_bias=s["bias"], bufs=bufs)
            else:
                binding.moe_expert_ffn_q4_0(xpool[f], s["gu"], s["dn"], K, routes[f][0],
                                            routes[f][1], bufs.y_sorted, bufs.ws_ffn)
    g_ffn.replay()
    torch.cuda.synchronize()
    reps = max(2, steps // F)
    ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev_a.record()
    for _ in range(reps):
        g_ffn.replay()
    ev_b.record()
    torch.cuda.synchronize()
    ffn_ms = ev_a.elapsed_time(ev_b) / (reps * F)

    expert_bytes = Q4_0_EXPERT_BYTES(H, I)
    asz = 4 if act == torch.float32 else 2
    N = T * K
    # algorithmic bytes: the distinct experts' Q4_0 bytes, x, h written and read,
    # y written (FFN call); plus the router, scales and output (layer)
    ffn_bytes = [d * expert_bytes + T * H * asz + N * I * asz * 2 + N * H * 4
                 for d in distinct[:F]]
    ffn_bytes_mean = sum(ffn_bytes) / F
    layer_bytes = sum(d * expert_bytes + E * H * 4 + T * H * asz + E * 4 + T * H * 4
                      for d in distinct) / G
    layer_hbm = layer_bytes / (ms_step * 1e-3) / 1e9
    ffn_flops = N * 6.0 * H * I          # per slot 2 (2I H) + 2 (H I)
    layer_tflops = ffn_flops / (ms_step * 1e-3) / 1e12
    if fused:
        call_bytes = sum(d * expert_bytes + E * H * 4 + T * H * asz + E * 4 + T * H * 4
                         for d in distinct[:F]) / F
        achieved = call_bytes / (ffn_ms * 1e-3) / 1e9
        launches = ("router logits, then gate/up and down in one launch (top-K inside every "
                    "workgroup, h handed over through completion counters): 2 launches"
                    if T == 1 else
                    "router logits, gate/up GEMV with top-K and permutation inside, down GEMV "
                    "with the combine inside: 3 launches")
        roofline = {"kernel": "moe_layer_decode (%s)" % launches,
                    "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                    "bytes_per_launch": call_bytes, "avg_launch_us": ffn_ms * 1e3}
        dtype = ("q4_0 x %s (activation blocks rounded to 15-bit fixed point, exact int4 digit "
                 "products, fp32 accumulate)" % spec.act)
    elif mfma_path(spec.act, T, H, I):
        achieved = ffn_flops / (ffn_ms * 1e-3) / 1e12
        roofline = {"kernel": "moe_expert_ffn_q4_0 (activation prep, gate/up and down bf16 MFMA "
                              "grouped GEMM launches)",
                    "bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None,
                    "flops_per_launch": ffn_flops, "avg_launch_us": ffn_ms * 1e3}
        dtype = "q4_0 x bf16 (exact bf16 MFMA products, fp32 accumulate)"
    else:
        achieved = ffn_bytes_mean / (ffn_ms * 1e-3) / 1e9
        roofline = {"kernel": "moe_expert_ffn_q4_0 (gate/up then down Q4_0 GEMV launches)",
                    "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                    "bytes_per_launch": ffn_bytes_mean, "avg_launch_us": ffn_ms * 1e3}
        dtype = ("q4_0 x %s (activation blocks rounded to 15-bit fixed point, exact int4 digit "
                 "products, fp32 accumulate)" % spec.act)
    tr = stored_traffic(spec.name)
    if tr is not None:
        roofline["traffic"] = tr["traffic_bytes"]
        roofline["traffic_fetch"] = tr["fetch_bytes"]
        roofline["traffic_write"] = tr["write_bytes"]
    res = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; random-init Q4_0 experts; %d weight sets in distinct memory, "
                "%d token batches)" % (nsets, G),
        "config": {"workload": "%s: Gemma-4-26B-A4B-shaped routed-MoE layer, T=%d, H=%d, E=%d, "
                               "top-%d, I=%d, Q4_0 experts, %s activations"
                               % (spec.name, T, H, E, K, I, spec.act),
                   "tokens_per_step": T, "weight_sets": nsets, "graphs": G,
                   "distinct_experts_per_step_mean": sum(distinct) / G,
                   "distinct_experts_per_step_min_max": [min(distinct), max(distinct)],
                   "layer_hbm_gbs": layer_hbm, "layer_hbm_frac": layer_hbm / HBM_PEAK_GBS,
                   "layer_expert_tflops": layer_tflops,
                   "layer_mfma_frac": layer_tflops / BF16_PEAK_TFLOPS,
                   "wall_s": wall,
                   "path": "moe_layer_decode" if fused else "moe_route + moe_expert_ffn_q4_0 + "
                                                            "moe_combine",
                   "steps_per_graph": S,
                   "timing": "K steps as K/%d replays of %d HIP graphs of %d consecutive steps "
                             "(step i on set i mod %d and batch i mod %d); the roofline call over "
                             "replays of one graph of %d calls on %d sets and routings"
                             % (S, NG, S, nsets, G, F, F)},
        "roofline": roofline,
    }
    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(spec, cpu_seconds)
    del graphs, g_ffn, sets, xpool, bufs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.summarize_stats:
        return summarize_stats(args)
    if args.summarize_traffic:
        return summarize_traffic(args)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the layer would shard over experts, one process per GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_moe_amd import synth
    torch.cuda.set_device(0)
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    spec = synth.SPECS[args.config]
    if spec.layers > 1:
        return bench_stack(args, spec)
    nsets = args.sets or (32 if spec.T <= 64 else 4)
    cpu_s = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    res = bench_layer(spec, args.steps, args.warmup, nsets, cpu_s)
    if args.config == 1 and not args.no_prefill:
        # the other half of the metric: the 4,096-token prefill, MFMA-bound
        p = bench_layer(synth.SPECS[3], max(5, args.steps // 10), max(2, args.warmup // 4), 4)
        res["prefill"] = {k: p[k] for k in ("value", "unit", "ms_per_step", "steps", "warmup",
                                            "dtype", "data", "config", "roofline")}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
