"""Benchmark of the grouped NF4 expert GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload olmoe]
                    [--cells cells.jsonl] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch: for each of L MoE
layers (distinct weights and router logits, all resident in HBM),
route/sort -> gate_up grouped GEMM (reading token rows through the sort:
the row gather is fused) -> down grouped GEMM,
every step in libgnf4's kernels.  Weights are packed once beforehand (the
pages quantise at bake time).  L is chosen so the step's expert bytes
exceed the 256 MB Infinity Cache, so each layer's weights stream from HBM.

Printed: ONE JSON line with the effective HBM throughput of the step
(algorithmic bytes / step time), the roofline of the dominant kernel
(average launch duration from HIP events recorded around each of its
launches inside the timed region), and the CPU oracle's throughput on a
bounded sample of the same workload.  --cells additionally measures every
workload's GEMMs alone (decode GB/s, prefill TFLOP/s) into a JSONL file.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak
METRIC = "grouped NF4 GEMM effective HBM GB/s (decode) & TFLOP/s (prefill), % roofline"


ABS_BYTES = 4  # bytes per block absmax: 4 (fp32) or 2 (bf16, --absmax-dtype bf16)
UNFUSED_ROUTE = False  # --unfused-route


def gemm_bytes(n_touched, M, N, K):
    """Algorithmic bytes of one grouped GEMM: each touched expert's codes and
    absmax once, the activations read once, the output written once."""
    return n_touched * (N * K // 2 + ABS_BYTES * N * K // 64) + 2 * M * K + 2 * M * N


def swiglu_bytes(M, I):
    """gate_up [M, 2I] read once, h [M, I] written once (bf16)."""
    return 2 * M * 2 * I + 2 * M * I


def combine_bytes(T, k, M, H):
    """Expert rows [M, H] read once, slot rows and weights read, out [T, H]
    written once."""
    return 2 * M * H + 8 * T * k + 2 * T * H


def route_bytes(T, E, k):
    M = T * k
    return 4 * T * E + 8 * T * k + 4 * (E + 1) + 4 * M + 8 * E + 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="olmoe")
    ap.add_argument("--layers", type=int, default=0, help="0 = the workload's default")
    ap.add_argument("--cells", default="", help="also time every workload's GEMMs into this JSONL")
    ap.add_argument("--mxfp4", default="",
                    help="time the MXFP4 grouped GEMM alone at the decode shapes into this JSONL")
    ap.add_argument("--dgrad", default="",
                    help="time the grouped dgrad alone at each workload's shapes into this JSONL")
    ap.add_argument("--glue", default="",
                    help="time the SwiGLU and top-k combine kernels alone into this JSONL")
    ap.add_argument("--absmax-dtype", choices=("f32", "bf16"), default="f32",
                    help="block absmax of the packed stacks (bf16: 4.25 bits per weight)")
    ap.add_argument("--only", default="",
                    help="comma-separated workload names: restrict --cells / --mxfp4 / --dgrad to them")
    ap.add_argument("--unfused-route", action="store_true",
                    help="run the route/sort as its own launch even where it folds into gate_up")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="launch every kernel from the host instead of replaying a HIP graph")
    ap.add_argument("--sets", type=int, default=0,
                    help="distinct weight sets cycled by the steps (0 = enough for >= 1 GiB)")
    ap.add_argument("--dominant-only", action="store_true",
                    help="only launch the dominant kernel (for counter collection), print its timing")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB --steps times "
                         "(calibrates the HBM byte counters)")
    ap.add_argument("--summarize", default="",
                    help="print a summary of the rocprofv3 CSV output in this directory and exit")
    return ap.parse_args()


class Layer:
    pass


def capture(fn):
    """Record fn's launches (all on the current stream) into a HIP graph."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def build_layers(wl, L, dev, first_layer=0):
    import torch
    from grouped_nf4_expert_amd import gnf4
    from grouped_nf4_expert_amd import workloads as wls

    Kg, Ng = wl.gemm("gate_up")
    Kd, Nd = wl.gemm("down")
    layers = []
    for li in range(first_layer, first_layer + L):
        ly = Layer()
        ly.pg = torch.empty((wl.E, Ng, Kg // 2), dtype=torch.uint8, device=dev)
        adt = torch.bfloat16 if ABS_BYTES == 2 else torch.float32
        ly.ag = torch.empty((wl.E, Ng, Kg // 64), dtype=adt, device=dev)
        ly.pd = torch.empty((wl.E, Nd, Kd // 2), dtype=torch.uint8, device=dev)
        ly.ad = torch.empty((wl.E, Nd, Kd // 64), dtype=adt, device=dev)
        for e in range(wl.E):
            gnf4.pack(wls.expert_weights_device(wl, "gate_up", e, dev, li), out=(ly.pg[e], ly.ag[e]))
            gnf4.pack(wls.expert_weights_device(wl, "down", e, dev, li), out=(ly.pd[e], ly.ad[e]))
        ly.logits = torch.from_numpy(wls.router_logits(wl, li)).to(dev)
        ly.x = wls.activations_device(wl.T, Kg, dev, wl.seed, 21, li)
        ly.xd = wls.activations_device(wl.M, Kd, dev, wl.seed, 22, li)
        ly.route = gnf4.RouteBuffers(wl.T, wl.E, wl.top_k, dev)
        ly.xs = torch.empty((wl.M, Kg), dtype=torch.bfloat16, device=dev)
        ly.yg = torch.empty((wl.M, Ng), dtype=torch.bfloat16, device=dev)
        ly.yd = torch.empty((wl.M, Nd), dtype=torch.bfloat16, device=dev)
        G = min(wl.E, wl.M)
        ly.G = G
        wsg = gnf4.gemm_workspace_size(wl.M, Ng, Kg, G, wl.E)
        wsd = gnf4.gemm_workspace_size(wl.M, Nd, Kd, G, wl.E)
        ly.wsg = torch.empty(max(wsg, 16), dtype=torch.uint8, device=dev)
        wsr = gnf4.library().gnf4_route_gemm_one_token_workspace_size(wl.E, wl.top_k, Ng, Kg)
        ly.wsr = torch.empty(max(wsr, 16), dtype=torch.uint8, device=dev)
        ly.wsd = torch.empty(max(wsd, 16), dtype=torch.uint8, device=dev)
        layers.append(ly)
    torch.cuda.synchronize()
    return layers


def fused_route(wl):
    """A single token with at most 128 experts: the route/sort is folded into
    the gate_up launch (gnf4_route_gemm_one_token), unless --unfused-route."""
    return wl.T == 1 and wl.E <= 128 and not UNFUSED_ROUTE


def gate_up(wl, ly):
    """gate_up GEMM reading the token rows through the sort (fused gather);
    with the route folded in, the same launch also routes the token."""
    from grouped_nf4_expert_amd import gnf4
    if fused_route(wl):
        gnf4.route_gemm_one_token(ly.logits, ly.x, ly.pg, ly.ag, wl.top_k, buffers=ly.route,
                                  y=ly.yg, workspace=ly.wsr)
        return
    r = ly.route.result
    gnf4.grouped_gemm(ly.x, ly.pg, ly.ag, r.group_sizes, r.group_expert_ids, G=ly.G, y=ly.yg,
                      workspace=ly.wsg, sorted_slots=r.sorted_slots, top_k=wl.top_k)


def run_layer(wl, ly):
    from grouped_nf4_expert_amd import gnf4
    if not fused_route(wl):
        gnf4.route_sort(ly.logits, wl.top_k, ly.route)
    gate_up(wl, ly)
    r = ly.route.result
    gnf4.grouped_gemm(ly.xd, ly.pd, ly.ad, r.group_sizes, r.group_expert_ids, G=ly.G, y=ly.yd,
                      workspace=ly.wsd)


def cpu_baseline(wl, seconds):
    """The oracle as it stands, on one layer of the same workload, repeated
    until about `seconds` of CPU time have passed."""
    import oracle
    from grouped_nf4_expert_amd import workloads as wls
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    Kg, Ng = wl.gemm("gate_up")
    Kd, Nd = wl.gemm("down")
    logits = wls.router_logits(wl, 0)
    rr = oracle.ref_route_sort(logits, wl.top_k)
    used = rr["group_expert_ids"][: rr["num_groups"]]
    pg = np.zeros((wl.E, Ng, Kg // 2), np.uint8)
    ag = np.zeros((wl.E, Ng, Kg // 64), np.float32)
    pd = np.zeros((wl.E, Nd, Kd // 2), np.uint8)
    ad = np.zeros((wl.E, Nd, Kd // 64), np.float32)
    for e in used:
        pg[e], ag[e] = oracle.ref_pack(wls.expert_weights(wl, "gate_up", int(e)))
        pd[e], ad[e] = oracle.ref_pack(wls.expert_weights(wl, "down", int(e)))
    x_tok = wls.token_activations(wl, Kg)
    xd = wls.down_input(wl, wl.M, Kd)
    n = len(used)
    layer_bytes = (route_bytes(wl.T, wl.E, wl.top_k) +
                   gemm_bytes(n, wl.M, Ng, Kg) + gemm_bytes(n, wl.M, Nd, Kd))
    reps = 0
    t0 = time.perf_counter()
    while True:
        r = oracle.ref_route_sort(logits, wl.top_k)
        xs = x_tok[r["sorted_slots"] // wl.top_k]
        oracle.ref_grouped_gemm(xs, pg, ag, r["group_sizes"], r["group_expert_ids"])
        oracle.ref_grouped_gemm(xd, pd, ad, r["group_sizes"], r["group_expert_ids"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(layer_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{reps} x one {wl.name} layer (route+sort, gather, gate_up + down GEMM over "
                      f"{n} touched experts) in {el:.1f} s; fp64 numpy, BLAS threads={threads}"}


def time_cells(path, dev, only=()):
    """Each workload's GEMMs alone, cycling over enough weight copies to
    defeat the Infinity Cache; per-launch HIP events."""
    import torch
    from grouped_nf4_expert_amd import gnf4
    from grouped_nf4_expert_amd import workloads as wls
    out = open(path, "w")
    for name in ("olmoe", "qwen3_t1", "qwen3_t8", "gptoss", "dsv3"):
        if only and name not in only:
            continue
        wl = wls.WORKLOADS[name]
        lg = torch.from_numpy(wls.router_logits(wl)).to(dev)
        r = gnf4.route_sort(lg, wl.top_k)
        G = min(wl.E, wl.M)
        ng = int(r.num_groups.cpu()[0])
        for gemm in ("gate_up", "down"):
            K, N = wl.gemm(gemm)
            stack_bytes = wl.E * (N * K // 2 + N * K // 16)
            copies = max(1, min(8, int(np.ceil(600e6 / stack_bytes))))
            stacks = []
            for ci in range(copies):
                p = torch.empty((wl.E, N, K // 2), dtype=torch.uint8, device=dev)
                a = torch.empty((wl.E, N, K // 64), dtype=torch.float32, device=dev)
                for e in range(wl.E):
                    gnf4.pack(wls.expert_weights_device(wl, gemm, e, dev, 100 + ci), out=(p[e], a[e]))
                stacks.append((p, a))
            x = wls.activations_device(wl.M, K, dev, wl.seed, 50, K)
            y = torch.empty((wl.M, N), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(max(gnf4.gemm_workspace_size(wl.M, N, K, G, wl.E), 16),
                             dtype=torch.uint8, device=dev)
            per = 4 * copies if name != "dsv3" else copies

            def launches():
                for i in range(per):
                    p, a = stacks[i % copies]
                    gnf4.grouped_gemm(x, p, a, r.group_sizes, r.group_expert_ids, G=G, y=y,
                                      workspace=ws)
            graph = capture(launches)
            reps = 10 if name != "dsv3" else 3
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(reps)]
            graph.replay()
            torch.cuda.synchronize()
            for i in range(reps):
                evs[i][0].record()
                graph.replay()
                evs[i][1].record()
            torch.cuda.synchronize()
            us = sorted(s.elapsed_time(e) * 1e3 / per for s, e in evs)
            med = us[len(us) // 2]
            byt = gemm_bytes(ng, wl.M, N, K)
            flops = 2.0 * wl.M * N * K
            rec = {"workload": name, "gemm": gemm, "E": wl.E, "top_k": wl.top_k, "T": wl.T,
                   "M": wl.M, "K": K, "N": N, "touched_experts": ng, "median_us": round(med, 2),
                   "min_us": round(us[0], 2), "GBps": round(byt / med / 1e3, 1),
                   "TFLOPs": round(flops / med / 1e6, 2),
                   "hbm_frac": round(byt / med / 1e3 / HBM_PEAK_GBS, 4),
                   "mfma_frac": round(flops / med / 1e6 / MFMA_FP16_PEAK_TFLOPS, 4),
                   "weight_copies": copies}
            out.write(json.dumps(rec) + "\n")
            out.flush()
            print(f"[cell] {json.dumps(rec)}", file=sys.stderr, flush=True)
            del stacks
            torch.cuda.empty_cache()
    out.close()


def time_dgrad(path, dev, only=()):
    """gnf4_grouped_dgrad alone, cycling over enough weight copies to defeat
    the Infinity Cache (as the forward cells); per-launch HIP events over a
    graph of back-to-back launches.  Algorithmic bytes as the forward GEMM
    (each touched expert's codes and absmax once, dy read, dx written)."""
    import torch
    from grouped_nf4_expert_amd import gnf4
    from grouped_nf4_expert_amd import workloads as wls
    out = open(path, "w")
    cells = (("olmoe", "gate_up"), ("olmoe", "down"), ("qwen3_t8", "gate_up"),
             ("gptoss", "gate_up"), ("gptoss", "down"), ("dsv3", "down"), ("dsv3", "gate_up"))
    for name, gemm in cells:
        if only and name not in only:
            continue
        wl = wls.WORKLOADS[name]
        lg = torch.from_numpy(wls.router_logits(wl)).to(dev)
        r = gnf4.route_sort(lg, wl.top_k)
        G = min(wl.E, wl.M)
        ng = int(r.num_groups.cpu()[0])
        K, N = wl.gemm(gemm)
        stack_bytes = wl.E * (N * K // 2 + N * K // 16)
        copies = max(1, min(8, int(np.ceil(600e6 / stack_bytes))))
        stacks = []
        for ci in range(copies):
            p = torch.empty((wl.E, N, K // 2), dtype=torch.uint8, device=dev)
            a = torch.empty((wl.E, N, K // 64), dtype=torch.float32, device=dev)
            for e in range(wl.E):
                gnf4.pack(wls.expert_weights_device(wl, gemm, e, dev, 200 + ci), out=(p[e], a[e]))
            stacks.append((p, a))
        dy = wls.activations_device(wl.M, N, dev, wl.seed, 60, N)
        dx = torch.empty((wl.M, K), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(gnf4.library().gnf4_grouped_dgrad_workspace_size(wl.M, N, K, G, wl.E),
                             16), dtype=torch.uint8, device=dev)
        per = 4 * copies if name != "dsv3" else 1

        def launches():
            for i in range(per):
                p, a = stacks[i % copies]
                gnf4.grouped_dgrad(dy, p, a, r.group_sizes, r.group_expert_ids, G=G, dx=dx,
                                   workspace=ws)
        graph = capture(launches)
        reps = 10 if name != "dsv3" else 2
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        graph.replay()
        torch.cuda.synchronize()
        for i in range(reps):
            evs[i][0].record()
            graph.replay()
            evs[i][1].record()
        torch.cuda.synchronize()
        us = sorted(s_.elapsed_time(e_) * 1e3 / per for s_, e_ in evs)
        med = us[len(us) // 2]
        byt = gemm_bytes(ng, wl.M, N, K)
        flops = 2.0 * wl.M * N * K
        kind = "tile path" if wl.M >= 32 * G else "GEMV path"  # the automatic choice
        rec = {"kernel": f"dgrad ({kind})", "workload": name, "gemm": gemm, "M": wl.M, "N": N, "K": K,
               "touched_experts": ng, "median_us": round(med, 2), "GBps": round(byt / med / 1e3, 1),
               "hbm_frac": round(byt / med / 1e3 / HBM_PEAK_GBS, 4),
               "TFLOPs": round(flops / med / 1e6, 2),
               "mfma_frac": round(flops / med / 1e6 / MFMA_FP16_PEAK_TFLOPS, 4),
               "weight_copies": copies}
        out.write(json.dumps(rec) + "\n")
        out.flush()
        print(f"[dgrad] {json.dumps(rec)}", file=sys.stderr, flush=True)
        del stacks
        torch.cuda.empty_cache()
    out.close()


def time_mxfp4(path, dev, only=()):
    """gnf4_grouped_gemm_mxfp4 alone at the decode shapes (GPT-OSS first: the
    family released in MXFP4) on the decode path, and at DeepSeek-V3's
    prefill shapes on the automatic (tile) path, cycling over enough random
    E2M1/E8M0 stack copies to defeat the Infinity Cache; per-launch HIP
    events over a graph of back-to-back launches with the fused gather.
    Algorithmic bytes: each touched expert's codes (N*K/2) and scales
    (N*K/32) once, the activation rows read once, the output written once;
    flops 2*M*N*K."""
    import torch
    from grouped_nf4_expert_amd import gnf4
    from grouped_nf4_expert_amd import workloads as wls
    out = open(path, "w")
    cells = (("gptoss", "gate_up"), ("gptoss", "down"), ("olmoe", "gate_up"), ("olmoe", "down"),
             ("qwen3_t8", "gate_up"), ("dsv3", "gate_up"), ("dsv3", "down"))
    for name, gemm in cells:
        if only and name not in only:
            continue
        prefill = name == "dsv3"
        path_sel = gnf4.PATH_AUTO if prefill else gnf4.PATH_DECODE
        wl = wls.WORKLOADS[name]
        r = gnf4.route_sort(torch.from_numpy(wls.router_logits(wl)).to(dev), wl.top_k)
        G = min(wl.E, wl.M)
        ng = int(r.num_groups.cpu()[0])
        K, N = wl.gemm(gemm)
        stack_bytes = wl.E * (N * K // 2 + N * K // 32)
        copies = max(1, min(8, int(np.ceil(600e6 / stack_bytes))))
        gen = torch.Generator(device=dev).manual_seed(17)
        stacks = [(torch.randint(0, 256, (wl.E, N, K // 2), dtype=torch.uint8, device=dev,
                                 generator=gen),
                   torch.randint(118, 131, (wl.E, N, K // 32), dtype=torch.uint8, device=dev,
                                 generator=gen)) for _ in range(copies)]
        x = wls.activations_device(wl.T, K, dev, wl.seed, 70, K)
        y = torch.empty((wl.M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(gnf4.gemm_workspace_size(wl.M, N, K, G, wl.E, path_sel), 16),
                         dtype=torch.uint8, device=dev)
        per = copies if prefill else 4 * copies

        def launches():
            for i in range(per):
                p, sc = stacks[i % copies]
                gnf4.grouped_gemm_mxfp4(x, p, sc, r.group_sizes, r.group_expert_ids, G=G, y=y,
                                        workspace=ws, path=path_sel, sorted_slots=r.sorted_slots,
                                        top_k=wl.top_k)
        graph = capture(launches)
        reps = 3 if prefill else 10
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        graph.replay()
        torch.cuda.synchronize()
        for i in range(reps):
            evs[i][0].record()
            graph.replay()
            evs[i][1].record()
        torch.cuda.synchronize()
        us = sorted(s_.elapsed_time(e_) * 1e3 / per for s_, e_ in evs)
        med = us[len(us) // 2]
        byt = ng * (N * K // 2 + N * K // 32) + 2 * wl.M * K + 2 * wl.M * N
        flops = 2.0 * wl.M * N * K
        kind = "tile path" if prefill else "decode path"
        rec = {"kernel": f"mxfp4 grouped GEMM ({kind}, fused gather)", "workload": name,
               "gemm": gemm, "M": wl.M, "N": N, "K": K, "touched_experts": ng,
               "median_us": round(med, 2), "GBps": round(byt / med / 1e3, 1),
               "hbm_frac": round(byt / med / 1e3 / HBM_PEAK_GBS, 4),
               "TFLOPs": round(flops / med / 1e6, 2),
               "mfma_frac": round(flops / med / 1e6 / MFMA_FP16_PEAK_TFLOPS, 4),
               "weight_copies": copies}
        out.write(json.dumps(rec) + "\n")
        out.flush()
        print(f"[mxfp4] {json.dumps(rec)}", file=sys.stderr, flush=True)
        del stacks
        torch.cuda.empty_cache()
    out.close()


def time_glue(path, dev, reps=10):
    """gnf4_swiglu and gnf4_combine alone at the decode (OLMoE, T=1) and
    prefill (DSV3, T=4096) shapes of the MoE layer: back-to-back launches
    from one HIP graph over enough buffer copies that the prefill buffers
    stream from HBM (the decode buffers are a few tens of KB: those launches
    are latency, not bandwidth)."""
    import torch
    from grouped_nf4_expert_amd import gnf4
    from grouped_nf4_expert_amd import workloads as wls
    out = open(path, "w")
    for name in ("olmoe", "dsv3"):
        wl = wls.WORKLOADS[name]
        D, N1 = wl.gemm("gate_up")
        I = N1 // 2
        r = gnf4.route_sort(torch.from_numpy(wls.router_logits(wl)).to(dev), wl.top_k)
        M, T, k = wl.M, wl.T, wl.top_k
        cases = (("swiglu", swiglu_bytes(M, I), (M, 2 * I), (M, I)),
                 ("combine", combine_bytes(T, k, M, D), (M, D), (T, D)))
        for kern, byt, in_shape, out_shape in cases:
            copies = max(2, min(16, -(-(1 << 30) // byt)))
            gen = torch.Generator(device=dev).manual_seed(5)
            ins = [torch.randn(in_shape, device=dev, generator=gen).to(torch.bfloat16)
                   for _ in range(copies)]
            outs = [torch.empty(out_shape, dtype=torch.bfloat16, device=dev)
                    for _ in range(copies)]
            per = 4 * copies

            def launches():
                for i in range(per):
                    c = i % copies
                    if kern == "swiglu":
                        gnf4.swiglu(ins[c], out=outs[c])
                    else:
                        gnf4.combine(ins[c], r.slot_rows, r.topk_w, out=outs[c])
            graph = capture(launches)
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(reps)]
            graph.replay()
            torch.cuda.synchronize()
            for i in range(reps):
                evs[i][0].record()
                graph.replay()
                evs[i][1].record()
            torch.cuda.synchronize()
            us = sorted(s_.elapsed_time(e_) * 1e3 / per for s_, e_ in evs)
            med = us[len(us) // 2]
            rec = {"kernel": kern, "workload": name, "M": M, "T": T, "top_k": k,
                   "width": I if kern == "swiglu" else D, "bytes": byt,
                   "median_us": round(med, 3), "GBps": round(byt / med / 1e3, 1),
                   "hbm_frac": round(byt / med / 1e3 / HBM_PEAK_GBS, 4), "copies": copies}
            out.write(json.dumps(rec) + "\n")
            out.flush()
            print(f"[glue] {json.dumps(rec)}", file=sys.stderr, flush=True)
            del ins, outs
            torch.cuda.empty_cache()
    out.close()


KERNEL_SOURCES = ("grouped_nf4_expert_amd/csrc/decode.hip",
                  "grouped_nf4_expert_amd/csrc/gnf4_internal.h",
                  "grouped_nf4_expert_amd/csrc/route_core.h")


def kernel_digest():
    """Short sha256 over the sources of the decode kernel and its launch rule:
    a stored counter reading is only valid for the code it was taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(wl_name):
    return os.path.join(ROOT, "profiles", f"decode_gate_up_{wl_name}_counters.txt")


def read_traffic(wl_name):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when there is none or the kernel changed since."""
    path = traffic_file(wl_name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_digest") != kernel_digest():
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def summarize(d):
    """Text summary of rocprofv3 CSV output (kernel stats and/or counters)."""
    import csv
    import glob
    import re

    def short(name):
        m = re.search(r"gnf4::\(anonymous namespace\)::(\w+)(<[^>]*>)?", name)
        return (m.group(1) + (m.group(2) or "")) if m else name[:60]

    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        print(f"# kernel statistics ({os.path.relpath(f, d)})")
        print(f"{'kernel':<48} {'calls':>7} {'avg us':>9} {'min us':>9} {'max us':>9} {'total %':>8}")
        for r in csv.DictReader(open(f)):
            print(f"{short(r['Name']):<48} {int(r['Calls']):>7} {float(r['AverageNs'])/1e3:>9.3f} "
                  f"{float(r['MinNs'])/1e3:>9.3f} {float(r['MaxNs'])/1e3:>9.3f} "
                  f"{float(r['Percentage']):>8.2f}")
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        print(f"# counters per dispatch, averaged per kernel ({os.path.relpath(f, d)})")
        agg = {}
        for r in csv.DictReader(open(f)):
            k = (short(r["Kernel_Name"]), r["Counter_Name"])
            agg.setdefault(k, []).append(float(r["Counter_Value"]))
        for (kn, cn), v in sorted(agg.items()):
            print(f"{kn:<48} {cn:<22} dispatches={len(v):>5} mean={sum(v)/len(v):.1f}")


def main():
    global ABS_BYTES, UNFUSED_ROUTE
    args = parse()
    ABS_BYTES = 2 if args.absmax_dtype == "bf16" else 4
    UNFUSED_ROUTE = args.unfused_route
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; it has no multi-GPU path",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from grouped_nf4_expert_amd import gnf4
    from grouped_nf4_expert_amd import workloads as wls

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    gnf4.library()
    dev = torch.device("cuda:0")

    only = tuple(w for w in args.only.split(",") if w)
    if args.glue:
        time_glue(args.glue, dev)
        return
    if args.cells and only:  # the named workloads' GEMM cells alone, no step
        time_cells(args.cells, dev, only)
        return
    if args.dgrad:
        time_dgrad(args.dgrad, dev, only)
        return
    if args.mxfp4:
        time_mxfp4(args.mxfp4, dev, only)
        return

    if args.copy_mb:
        # calibration for the HBM byte counters: a plain copy of known size
        n = args.copy_mb << 20
        src = torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_mib": args.copy_mb, "reps": args.steps}))
        return

    wl = wls.WORKLOADS[args.workload]
    L = args.layers or wl.layers
    Kg, Ng = wl.gemm("gate_up")
    Kd, Nd = wl.gemm("down")
    g_est = min(wl.E, wl.M)
    step_est = L * (gemm_bytes(g_est, wl.M, Ng, Kg) + gemm_bytes(g_est, wl.M, Nd, Kd))
    # enough distinct weight sets that the steps cycle through >= 1 GiB of
    # expert bytes, four times the 256 MB Infinity Cache: every step streams
    # its weights from HBM
    n_sets = args.sets or max(1, min(8, -(-(1 << 30) // step_est)))
    print(f"[bench] building {n_sets} x {L} layers of {wl.name}", file=sys.stderr, flush=True)
    sets = [build_layers(wl, L, dev, first_layer=k * L) for k in range(n_sets)]

    for layers in sets:
        for ly in layers:
            run_layer(wl, ly)
    torch.cuda.synchronize()
    touched = [[int(ly.route.result.num_groups.cpu()[0]) for ly in layers] for layers in sets]
    set_bytes = [sum(route_bytes(wl.T, wl.E, wl.top_k) + gemm_bytes(n, wl.M, Ng, Kg) +
                     gemm_bytes(n, wl.M, Nd, Kd) for n in t) for t in touched]
    # the dominant launch: gate_up, plus the route/sort's bytes when it is folded in
    dom_route = route_bytes(wl.T, wl.E, wl.top_k) if fused_route(wl) else 0
    dom_bytes = [gemm_bytes(n, wl.M, Ng, Kg) + dom_route for t in touched for n in t]

    flat = [ly for layers in sets for ly in layers]

    def dominant_host(reps):
        """The gate_up GEMM launched on its own from the host, cycling every
        layer of every set (for counter collection)."""
        for i in range(reps):
            gate_up(wl, flat[i % len(flat)])
        torch.cuda.synchronize()

    def dominant_timed(replays):
        """The gate_up GEMM of every layer of every set, twice, launched back
        to back from one HIP graph; HIP events on the launch stream bracket
        each replay.  Per-launch duration = replay time / launches."""
        n = 2 * len(flat)
        g = capture(lambda: [gate_up(wl, flat[i % len(flat)]) for i in range(n)])
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(replays)]
        g.replay()
        torch.cuda.synchronize()
        for i in range(replays):
            evs[i][0].record()
            g.replay()
            evs[i][1].record()
        torch.cuda.synchronize()
        return [s.elapsed_time(e) * 1e3 / n for s, e in evs]

    if args.dominant_only:
        dominant_host(max(args.steps, 1))
        print(json.dumps({"kernel": "gate_up decode GEMM", "launches": max(args.steps, 1)}))
        return

    # one step = every layer's launches, captured once per weight set as a
    # HIP graph and replayed (the decode kernels take microseconds: host
    # launch overhead would otherwise dominate)
    graphs = [capture(lambda layers=layers: [run_layer(wl, ly) for ly in layers])
              if args.graph else None for layers in sets]

    def run_step(i):
        k = i % n_sets
        if graphs[k] is not None:
            graphs[k].replay()
        else:
            for ly in sets[k]:
                run_layer(wl, ly)

    for i in range(args.warmup):
        run_step(i)
    # timed region: exactly `steps` steps, synchronised on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    timed_bytes = sum(set_bytes[i % n_sets] for i in range(args.steps))
    value = timed_bytes / ((t1 - t0)) / 1e9

    dur_us = dominant_timed(10)
    avg_us = float(np.mean(dur_us))
    achieved = float(np.mean(dom_bytes)) / (avg_us * 1e-6) / 1e9
    traffic = read_traffic(wl.name) if ABS_BYTES == 4 else None  # counters: fp32 stacks

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: E={wl.E} top_k={wl.top_k} T={wl.T} M={wl.M}, gate_up "
                        f"K={Kg} N={Ng} + down K={Kd} N={Nd}, {L} layers of distinct weights "
                        + ("per step (route/sort folded into gate_up with fused gather + down)"
                           if fused_route(wl) else
                           "per step (route/sort + gate_up with fused gather + down)"),
            "weights": f"NF4 (block 64, {'bf16' if ABS_BYTES == 2 else 'fp32'} absmax)",
            "activations": "bf16",
            "global_batch": wl.T, "layers": L, "parallelism": "none (1 GPU)",
            "launch": "HIP graph per step" if args.graph else "host launches",
            "weight_sets": n_sets, "bytes_per_step": [int(b) for b in set_bytes],
            "touched_experts_per_layer": touched[0],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode-path grouped GEMM (gate_up, fused row gather"
                      + (", route/sort folded in" if fused_route(wl) else "") + "), "
                      f"{2 * len(flat)} launches back to back per HIP graph replay",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_us, 3),
            "median_launch_us": round(float(np.median(dur_us)), 3),
            "launches_timed": 20 * len(flat),
            "algorithmic_bytes_per_launch": int(np.mean(dom_bytes)),
            "kernel_source_digest": kernel_digest(),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)

    if args.cells:
        time_cells(args.cells, dev, only)


if __name__ == "__main__":
    main()
