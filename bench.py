"""Benchmark of the AWQ W4A16 hot path on one MI355X.

One step = one pass of the whole hot path over every single-GPU workload:
  c2  Llama-7B MLP up-projection (K=4096 -> N=11008, fp16, 65536 calibration
      tokens = 128 sequences x 512): mean|x| statistics -> 20-candidate scale
      search -> quantize + pack -> 128 batch-1 decode GEMVs -> 128 batch-8
      products (over 32 resident copies of the packed weights, 755 MB, so that
      every launch streams its weights from HBM, not from the 256 MB last-level
      cache);
  c4  Llama-70B MLP prefill, M=2048 bf16 tokens: the matrix-core W4A16 GEMM
      of the up-projection (8192 -> 28672) and the down-projection
      (28672 -> 8192), weights quantized by the same path during setup; each
      timed as 4 products (pre-pass + GEMM) back to back in one graph, as
      the decode lines are (sustained: the power-limited clock settles lower
      than in a single product, which the graph's own start offsets);
  c1  a single 512 x 512 fp16 linear: statistics, search, quantize + pack and
      one batch-1 product (latency; the layer sits in cache);
  c3  a Llama-7B decoder layer (q/k/v/o 4096^2, gate/up 4096->11008, down
      11008->4096, fp16), quantized by the path during setup: the decode
      products at M = 1, 8 and 32 of each linear over 8 resident copies;
  c5  the 80-layer Llama-70B-shaped stack (hidden 8192, MLP 28672, k/v
      8192->1024): one batch-1 decode pass over its 35.83 GB of packed weights
      (q|k|v and gate|up, which read one input each, as one product each: 320
      launches), with 1/s folded into the producers of x (the deployed form)
      and, separately, applied inside the products; beside it, the same 320
      launches as plain streaming reads of the packed codes (the pass's
      read ceiling on this chip).
The products run from captured HIP graphs.  The c5 stack's layer 0 is
quantized by the full path (statistics, shared-input searches over 131072
calibration tokens, quantize + pack) once, timed apart from the steps; layers
1..79 carry seeded random codes, steps and zero points of the same layout
(--c5-quantize-all quantizes every layer by the path instead, in minutes).

value = effective HBM GB/s of the c2 batch-1 GEMV: packed bytes (codes + fp16
        steps + uint8 zero points, 0.5234 B per weight) per launch / average
        launch time, measured with HIP events on the launch stream.  Beside it,
        roofline.read_ceiling: a plain streaming read of the same bytes per
        launch (awq_read_stream), 128 launches over 32 resident buffers in one
        graph, timed in the same steps: the rate a launch of that size reaches
        on this chip.
All inputs are seeded synthetic tensors (workloads module) resident in HBM.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0
N_ROT = 32          # distinct resident weight copies of the c2 layer (755 MB)
N_PASS = 4          # passes over the copies per decode graph (128 products per replay)
C3_COPIES = 8       # resident copies of the c3 layer (847 MB)
C3_PASS = 4
C4_REPS = 4         # prefill products per graph replay
C3_MS = (1, 8, 32)
C5_LAYERS = 80
# quantizer variants reported beside the timed path: (group, bits, symmetric)
VARIANTS = ((64, 4, False), (128, 4, False), (256, 4, False), (128, 3, False), (128, 8, False),
            (128, 4, True), (128, 3, True))
METRIC = "W4A16 GEMV effective HBM GB/s (M=1) + prefill GEMM TFLOP/s; % of roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle (used under a profiler)")
    ap.add_argument("--sections", default="c1,c3,c4,c5",
                    help="workloads besides the 7B up-projection (always run): any of c1,c3,c4,c5")
    ap.add_argument("--no-c5", action="store_true", help="leave out the 80-layer stack")
    ap.add_argument("--c5-quantize-all", action="store_true",
                    help="quantize every layer of the 80-layer stack by the full path (minutes)")
    return ap.parse_args()


def packed_bytes(N: int, K: int, group: int = 128) -> int:
    return N * K // 2 + N * (K // group) * 3


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary,
    or None when the kernel's source changed after the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemv_traffic.json")
    try:
        rec = json.load(open(path))[kernel]
        h = hashlib.sha256()
        for f in rec["kernel_sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except (OSError, KeyError, ValueError):
        return None
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return rec["bytes_per_launch"]


# ----------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on the host, on samples of the same
# bytes the GPU path processes (a reported baseline, not the target)
# ----------------------------------------------------------------------------
def cpu_baseline(c2, c4, budget_gemv_s: float = 8.0) -> dict:
    import numpy as np

    import oracle as O
    cores = len(os.sched_getaffinity(0))
    W = c2["W"].float().cpu().numpy()
    X = c2["X"]
    N, K, T = c2["N"], c2["K"], c2["T"]
    st = {}
    # O1: statistic over 8192 of the 65536 calibration tokens
    Xs = X[:8192].float().cpu().numpy()
    t0 = time.perf_counter()
    m = O.act_mean_abs(Xs)
    el = time.perf_counter() - t0
    st["act_stats"] = {"GB/s": Xs.size * 2 / el / 1e9, "s": el,
                       "sample": "8192 of the 65536 calibration tokens x 4096 channels"}
    # O2-O5: search over 20 candidates on 64 rows x 8192 tokens; the full
    # layer's time extrapolated linearly in rows x tokens
    al = np.arange(20, dtype=np.float64) / 19.0
    t0 = time.perf_counter()
    O.search_scales(W[:64], Xs, m, al)
    el = time.perf_counter() - t0
    st["search"] = {"s": el, "full_layer_s_extrapolated": el * (N / 64) * (T / 8192),
                    "sample": "64 of 11008 rows x 8192 of 65536 tokens, 20 candidates; the full "
                              "layer's time extrapolated linearly in rows x tokens"}
    # O6: quantize + pack of 1024 rows with the GPU's chosen s
    s = c2["s"].cpu().numpy()
    t0 = time.perf_counter()
    r = O.quantize_layer(W[:1024], s)
    O.pack_codes(r["q"])
    el = time.perf_counter() - t0
    st["quantize"] = {"GB/s": 1024 * K * (2 + 0.5234) / el / 1e9, "s": el,
                      "sample": "1024 of 11008 rows"}
    # O7: batch-1 products of the full layer (the line's value)
    words, step, zeros = c2["q"].cpu().numpy(), c2["sc"].cpu().numpy(), c2["z"].cpu().numpy()
    xs = c2["x1"].float().cpu().numpy()
    inv = c2["inv"].cpu().numpy()
    reps, t0 = 0, time.perf_counter()
    while True:
        O.w4a16_matmul(xs, words, step, zeros, inv)
        reps += 1
        el = time.perf_counter() - t0
        if el > budget_gemv_s or reps >= 1000:
            break
    gemv_gbs = packed_bytes(N, K) * reps / el / 1e9
    st["gemv_m1"] = {"GB/s": gemv_gbs, "s": el,
                     "sample": f"{reps} batch-1 products of the full {N}x{K} layer"}
    # O7: the prefill GEMM on 64 output channels of the 70B up-projection
    up = c4["up"]
    xp = up["x"].float().cpu().numpy()
    words, step, zeros = up["q"][:64].cpu().numpy(), up["sc"][:64].cpu().numpy(), up["z"][:64].cpu().numpy()
    inv_up = up["inv"].cpu().numpy()
    t0 = time.perf_counter()
    O.w4a16_matmul(xp, words, step, zeros, inv_up)
    el = time.perf_counter() - t0
    st["gemm_prefill"] = {"TFLOP/s": 2.0 * xp.shape[0] * 64 * xp.shape[1] / el / 1e12, "s": el,
                          "sample": "64 of 28672 output channels x 2048 tokens x 8192"}
    total = sum(v["s"] for v in st.values())
    return {"value": gemv_gbs, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"NumPy oracle (float64; BLAS threads up to {cores}) on samples of the "
                      f"benchmark's own inputs, {total:.1f} s in all; value = batch-1 W4A16 "
                      f"products of the full {N}x{K} layer ({reps} in {st['gemv_m1']['s']:.1f} s); "
                      "per-stage rates under 'stages'",
            "stages": st}


# ----------------------------------------------------------------------------
def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "layout is described, not built", file=sys.stderr)
        return 2
    import torch

    import workloads as WL
    import weight_only_int4_stats_amd as awq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    awq.lib()
    sections = {x.strip() for x in args.sections.split(",") if x.strip()}
    if args.no_c5:
        sections.discard("c5")
    alphas = torch.from_numpy(WL.alpha_grid(20)).to(dev)

    def ws_for(op, M=0, N=0, K=0, T=0, na=0):
        n = awq.awq_workspace_bytes(op, M, N, K, T, na)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=dev)

    def quantize(W, X, group=128):
        """The path on one linear: statistics, search, quantize + pack."""
        m = awq.awq_act_stats(X)
        s, inv, L, b = awq.awq_search_scales(W, X, m, alphas, group)
        q, sc, z = awq.awq_quantize_pack(W, s, group)
        return {"m": m, "s": s, "inv": inv, "L": L, "best": b, "q": q, "sc": sc, "z": z}

    # ---------------- c2: Llama-7B MLP up (fp16)
    wa = WL.workload(2)
    NA, KA = wa.N, wa.K
    print(f"setup: {wa.name}, T={wa.T}", file=sys.stderr, flush=True)
    WA = WL.weight(wa).to(dev)
    XA = WL.calibration(wa).to(dev)
    xa1 = WL.decode_input(wa, 1).to(dev)
    xa8 = WL.decode_input(wa, 8).to(dev)
    GA = KA // 128
    ws_stats = ws_for(awq.AWQ_OP_ACT_STATS, 0, NA, KA, wa.T)
    ws_search = ws_for(awq.AWQ_OP_SEARCH, 0, NA, KA, wa.T, 20)
    m = torch.empty(KA, dtype=torch.float32, device=dev)
    s = torch.empty(KA, dtype=torch.float32, device=dev)
    inv = torch.empty(KA, dtype=torch.float32, device=dev)
    loss = torch.empty(20, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    qs = [torch.empty((NA, KA // 8), dtype=torch.int32, device=dev) for _ in range(N_ROT)]
    scs = [torch.empty((NA, GA), dtype=torch.float16, device=dev) for _ in range(N_ROT)]
    zs = [torch.empty((NA, GA), dtype=torch.uint8, device=dev) for _ in range(N_ROT)]
    y1 = torch.empty((N_ROT, NA), dtype=torch.float16, device=dev)
    y8 = torch.empty((N_ROT, 8, NA), dtype=torch.float16, device=dev)
    awq.awq_act_stats(XA, m, ws=ws_stats)
    awq.awq_search_scales(WA, XA, m, alphas, s_out=s, inv_s_out=inv, loss_out=loss,
                          best_idx_out=best, ws=ws_search)
    awq.awq_quantize_pack(WA, s, qweight=qs[0], scales=scs[0], zeros=zs[0])
    for i in range(1, N_ROT):
        qs[i].copy_(qs[0])
        scs[i].copy_(scs[0])
        zs[i].copy_(zs[0])
    torch.cuda.synchronize()

    # ---------------- c4: Llama-70B MLP prefill (bf16), up and down
    c4 = {}
    for lin in (("up", "down") if "c4" in sections else ()):
        wb = WL.workload(4, lin)
        print(f"setup: {wb.name}, M={wb.Ms[0]}", file=sys.stderr, flush=True)
        WB = WL.weight(wb).to(dev)
        XB = WL.calibration(wb).to(dev)
        qb = quantize(WB, XB)
        del WB
        MB = wb.Ms[0]
        c4[lin] = {"N": wb.N, "K": wb.K, "M": MB, "x": WL.prefill_input(wb, MB).to(dev),
                   "q": qb["q"], "sc": qb["sc"], "z": qb["z"], "inv": qb["inv"],
                   "y": torch.empty((MB, wb.N), dtype=torch.bfloat16, device=dev),
                   "ws": ws_for(awq.AWQ_OP_GEMM, MB, wb.N, wb.K)}
        del XB
        torch.cuda.synchronize()

    # ---------------- c1: single 512 x 512 linear
    w1 = WL.workload(1)
    c1 = {"W": WL.weight(w1).to(dev), "X": WL.calibration(w1).to(dev),
          "x": WL.decode_input(w1, 1).to(dev),
          "ws_st": ws_for(awq.AWQ_OP_ACT_STATS, 0, w1.N, w1.K, w1.T),
          "ws_se": ws_for(awq.AWQ_OP_SEARCH, 0, w1.N, w1.K, w1.T, 20),
          "m": torch.empty(w1.K, dtype=torch.float32, device=dev),
          "s": torch.empty(w1.K, dtype=torch.float32, device=dev),
          "inv": torch.empty(w1.K, dtype=torch.float32, device=dev),
          "q": torch.empty((w1.N, w1.K // 8), dtype=torch.int32, device=dev),
          "sc": torch.empty((w1.N, w1.K // 128), dtype=torch.float16, device=dev),
          "z": torch.empty((w1.N, w1.K // 128), dtype=torch.uint8, device=dev),
          "y": torch.empty((1, w1.N), dtype=torch.float16, device=dev)}

    def c1_pass():
        awq.awq_act_stats(c1["X"], c1["m"], ws=c1["ws_st"])
        awq.awq_search_scales(c1["W"], c1["X"], c1["m"], alphas, s_out=c1["s"], inv_s_out=c1["inv"],
                              ws=c1["ws_se"])
        awq.awq_quantize_pack(c1["W"], c1["s"], qweight=c1["q"], scales=c1["sc"], zeros=c1["z"])
        awq.awq_w4a16_gemm(c1["x"], c1["q"], c1["sc"], c1["z"], c1["inv"], y=c1["y"])

    # ---------------- c3: Llama-7B decoder layer, 8 resident copies
    print("setup: llama7b decoder layer (7 linears)", file=sys.stderr, flush=True)
    c3 = {}
    for lin in (("q", "k", "v", "o", "gate", "up", "down") if "c3" in sections else ()):
        w3 = WL.workload(3, lin)
        qd = quantize(WL.weight(w3).to(dev), WL.calibration(w3).to(dev))
        copies = [(qd["q"], qd["sc"], qd["z"])]
        for _ in range(C3_COPIES - 1):
            copies.append((qd["q"].clone(), qd["sc"].clone(), qd["z"].clone()))
        c3[lin] = {"N": w3.N, "K": w3.K, "inv": qd["inv"], "copies": copies,
                   "x": {M: WL.decode_input(w3, M).to(dev) for M in C3_MS},
                   "y": {M: torch.empty((C3_COPIES, M, w3.N), dtype=torch.float16, device=dev)
                         for M in C3_MS},
                   "ws": {M: ws_for(awq.AWQ_OP_GEMM, M, w3.N, w3.K) for M in C3_MS}}
    torch.cuda.synchronize()

    # ---------------- c5: 80-layer Llama-70B-shaped stack
    c5 = None
    if "c5" in sections:
        c5 = setup_c5(torch, WL, awq, dev, alphas, ws_for, args.c5_quantize_all)

    # ---------------- decode graphs
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.set_stream(stream)

    def decode_c2(x, y):
        for _ in range(N_PASS):
            for i in range(N_ROT):
                awq.awq_w4a16_gemm(x, qs[i], scs[i], zs[i], inv, y=y[i])

    def decode_c3(lin, M):
        d = c3[lin]
        for _ in range(C3_PASS):
            for i, (q, sc, z) in enumerate(d["copies"]):
                awq.awq_w4a16_gemm(d["x"][M], q, sc, z, d["inv"], y=d["y"][M][i], ws=d["ws"][M])

    def decode_c5(folded):
        for L in c5["layers"]:
            for part in L:
                awq.awq_w4a16_gemm(c5["x"][part["K"]], part["q"], part["sc"], part["z"],
                                   None if folded else part["inv"], y=part["y"])

    graphs = {}

    def capture(name, fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        graphs[name] = g

    # The ceiling the batch-1 line is compared with: a plain streaming read of
    # the same bytes per launch (awq_read_stream), over as many resident
    # buffers and launches per graph; the launch shape is the best of a short
    # untimed sweep.
    rd_bytes = packed_bytes(NA, KA)
    rd_bufs = [torch.empty(rd_bytes // 4, dtype=torch.int32, device=dev) for _ in range(N_ROT)]
    rd_xor = torch.empty(4096, dtype=torch.int32, device=dev)

    def read_pass(blocks, unroll):
        for _ in range(N_PASS):
            for b in rd_bufs:
                awq.awq_read_stream(b, blocks, unroll, block_xor=rd_xor)

    rd_best = None
    for blocks in (256, 512, 1024, 2048):
        for unroll in (2, 4, 8):
            read_pass(blocks, unroll)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                read_pass(blocks, unroll)
            ts = []
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            if rd_best is None or min(ts) < rd_best[0]:
                rd_best = (min(ts), blocks, unroll)
            del g
    capture("read_ceiling", lambda: read_pass(rd_best[1], rd_best[2]))
    # the prefill products (pre-pass and GEMM) run from graphs too: the phase
    # then times the GPU work, not the launch of two kernels from Python
    def prefill(d):
        for _ in range(C4_REPS):
            awq.awq_w4a16_gemm(d["x"], d["q"], d["sc"], d["z"], d["inv"], y=d["y"], ws=d["ws"])

    for lin in c4:
        capture(f"gemm_prefill_{lin}", lambda d=c4[lin]: prefill(d))
    if "c1" in sections:
        capture("c1_pipeline", c1_pass)
    capture("gemv_m1", lambda: decode_c2(xa1, y1))
    capture("gemv_m8", lambda: decode_c2(xa8, y8))
    for lin in c3:
        for M in C3_MS:
            capture(f"c3_{lin}_m{M}", lambda lin=lin, M=M: decode_c3(lin, M))
    # The decode pass's ceiling: the same 320 launches as plain streaming reads
    # of each product's packed codes, with each product kind's launch shape the
    # best of a short untimed sweep over all 80 layers.
    c5_rd = {}
    if c5 is not None:
        c5_xor = torch.empty(4096, dtype=torch.int32, device=dev)
        for i in range(len(c5["layers"][0])):
            pick = None
            for blocks in (256, 512, 1024, 2048):
                for unroll in (2, 4, 8):
                    def kind_pass(i=i, blocks=blocks, unroll=unroll):
                        for L in c5["layers"]:
                            awq.awq_read_stream(L[i]["q"], blocks, unroll, block_xor=c5_xor)
                    kind_pass()
                    torch.cuda.synchronize()
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=stream):
                        kind_pass()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    g.replay()
                    e1.record(stream)
                    torch.cuda.synchronize()
                    t = e0.elapsed_time(e1)
                    if pick is None or t < pick[0]:
                        pick = (t, blocks, unroll)
                    del g
            c5_rd[i] = pick[1:]

        def read_c5():
            for L in c5["layers"]:
                for i, part in enumerate(L):
                    awq.awq_read_stream(part["q"], *c5_rd[i], block_xor=c5_xor)
        capture("c5_read_ceiling", read_c5)
    if c5 is not None:
        capture("c5_decode_folded", lambda: decode_c5(True))
        capture("c5_decode_inv_s", lambda: decode_c5(False))
    torch.cuda.synchronize()

    phases = ["act_stats", "search", "quantize", "gemv_m1", "gemv_m8", "read_ceiling"]
    phases += [f"gemm_prefill_{lin}" for lin in c4]
    if "c1" in sections:
        phases.append("c1_pipeline")
    phases += [f"c3_{lin}_m{M}" for lin in c3 for M in C3_MS]
    if c5 is not None:
        phases += ["c5_decode_folded", "c5_decode_inv_s", "c5_read_ceiling"]

    def step(ev):
        k = 0

        def mark():
            nonlocal k
            ev[k].record(stream)
            k += 1
        mark()
        awq.awq_act_stats(XA, m, ws=ws_stats)
        mark()
        awq.awq_search_scales(WA, XA, m, alphas, s_out=s, inv_s_out=inv, loss_out=loss,
                              best_idx_out=best, ws=ws_search)
        mark()
        awq.awq_quantize_pack(WA, s, qweight=qs[0], scales=scs[0], zeros=zs[0])
        mark()
        graphs["gemv_m1"].replay()
        mark()
        graphs["gemv_m8"].replay()
        mark()
        graphs["read_ceiling"].replay()
        mark()
        for lin in c4:
            graphs[f"gemm_prefill_{lin}"].replay()
            mark()
        if "c1" in sections:
            graphs["c1_pipeline"].replay()
            mark()
        for lin in c3:
            for M in C3_MS:
                graphs[f"c3_{lin}_m{M}"].replay()
                mark()
        if c5 is not None:
            graphs["c5_decode_folded"].replay()
            mark()
            graphs["c5_decode_inv_s"].replay()
            mark()
            graphs["c5_read_ceiling"].replay()
            mark()

    def new_events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]

    for _ in range(args.warmup):
        step(new_events())
    torch.cuda.synchronize()
    # the K steps are enqueued back to back (the host runs ahead of the GPU, so
    # the events time GPU work, not the host's enqueue latency) and bracketed
    # by one synchronization on each side
    evs = [new_events() for _ in range(args.steps)]
    per = {n: 0.0 for n in phases}
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for e in evs:
        for i, n in enumerate(phases):
            per[n] += e[i].elapsed_time(e[i + 1])
    K_ = args.steps
    avg = {n: per[n] / K_ for n in phases}            # ms per step per phase
    ms_step = wall * 1000.0 / K_

    # ---------------- c2 figures
    bytes_a = packed_bytes(NA, KA)
    gemv1_us = avg["gemv_m1"] * 1000.0 / (N_ROT * N_PASS)
    gemv8_us = avg["gemv_m8"] * 1000.0 / (N_ROT * N_PASS)
    gemv_gbs = bytes_a / (gemv1_us * 1e-6) / 1e9
    gemv8_gbs = bytes_a / (gemv8_us * 1e-6) / 1e9
    read_us = avg["read_ceiling"] * 1000.0 / (N_ROT * N_PASS)
    read_gbs = rd_bytes / (read_us * 1e-6) / 1e9
    # matrix-core operations the search executes: the direct form contracts
    # over the tokens per candidate; the Gram form (taken by the library when
    # it needs under half of those, see awq_search_scales in include/awq.h)
    # forms X^T X once and per candidate contracts with the 256 x 256 blocks
    # of it on and below the diagonal, each as two fp16 parts
    Tp = (wa.T + 255) // 256 * 256
    gblk = (KA + 255) // 256
    direct_flop = 2.0 * wa.T * NA * KA * 20
    gram_flop = 2.0 * Tp * KA * KA + 20 * 2.0 * NA * 256 * 256 * gblk * (gblk + 1)
    search_gram = KA <= 32768 and gram_flop < 0.5 * direct_flop
    search_flop = gram_flop if search_gram else direct_flop
    loss_h = [float(v) for v in loss.cpu()]
    best_h = int(best.cpu()[0])
    alphas_h = alphas.cpu().numpy()
    stats_bytes = wa.T * KA * 2
    quant_bytes = NA * KA * 2 + bytes_a
    gemm = {}
    for lin in c4:
        d = c4[lin]
        flop = 2.0 * d["M"] * d["N"] * d["K"]
        ms = avg[f"gemm_prefill_{lin}"] / C4_REPS
        gemm[lin] = {"ms": ms, "TFLOP/s": flop / (ms * 1e-3) / 1e12,
                     "frac_fp16_mfma": flop / (ms * 1e-3) / 1e12 / FP16_MFMA_PEAK_TFLOPS,
                     "shape": f"M={d['M']} K={d['K']} N={d['N']} bf16"}
    stages = {
        "act_stats": {"ms": avg["act_stats"], "GB/s": stats_bytes / (avg["act_stats"] * 1e-3) / 1e9},
        "search": {"ms": avg["search"], "form": "gram" if search_gram else "direct",
                   "TFLOP/s": search_flop / (avg["search"] * 1e-3) / 1e12,
                   "frac_fp16_mfma": search_flop / (avg["search"] * 1e-3) / 1e12 / FP16_MFMA_PEAK_TFLOPS,
                   "direct_form_equivalent_TFLOP/s": direct_flop / (avg["search"] * 1e-3) / 1e12,
                   # output MSE over the calibration tokens: alpha = 0 is s = 1, plain
                   # round-to-nearest; the chosen alpha is the searched scale
                   "loss_rtn": loss_h[0], "loss_awq": loss_h[best_h], "alpha": float(alphas_h[best_h]),
                   "rtn_over_awq": loss_h[0] / loss_h[best_h]},
        "quantize": {"ms": avg["quantize"], "GB/s": quant_bytes / (avg["quantize"] * 1e-3) / 1e9},
        "gemv_m1": {"us_per_launch": gemv1_us, "GB/s": gemv_gbs, "frac_hbm": gemv_gbs / HBM_PEAK_GBS,
                    "frac_read_ceiling": gemv_gbs / read_gbs},
        "gemv_m8": {"us_per_launch": gemv8_us, "GB/s": gemv8_gbs, "frac_hbm": gemv8_gbs / HBM_PEAK_GBS,
                    "frac_read_ceiling": gemv8_gbs / read_gbs},
        "read_ceiling": {"us_per_launch": read_us, "GB/s": read_gbs, "frac_hbm": read_gbs / HBM_PEAK_GBS,
                         "bytes_per_launch": rd_bytes, "blocks": rd_best[1], "unroll": rd_best[2],
                         "what": "plain streaming read (awq_read_stream) of the batch-1 line's bytes per "
                                 f"launch, {N_ROT * N_PASS} launches over {N_ROT} resident buffers in one "
                                 "graph, the best of 12 launch shapes: the rate a launch of this size "
                                 "reaches on this chip"},
    }
    if c4:
        stages["gemm_prefill"] = gemm["up"]
        stages["gemm_prefill_down"] = gemm["down"]
    if "c1" in sections:
        stages["c1_single_linear"] = {"us_pipeline": avg["c1_pipeline"] * 1000.0,
                                      "what": "statistics + 20-candidate search + quantize + pack + "
                                              "batch-1 product of the 512 x 512 linear, replayed "
                                              "from one captured graph (cache-resident: a latency)"}
    # ---------------- c3 figures
    c3_out = {"per_linear": {}, "per_layer": {}}
    layer_bytes = sum(packed_bytes(c3[lin]["N"], c3[lin]["K"]) for lin in c3)
    for M in (C3_MS if c3 else ()):
        tot_us = 0.0
        for lin in c3:
            us = avg[f"c3_{lin}_m{M}"] * 1000.0 / (C3_COPIES * C3_PASS)
            tot_us += us
            b = packed_bytes(c3[lin]["N"], c3[lin]["K"])
            c3_out["per_linear"].setdefault(lin, {})[f"M={M}"] = {
                "us": us, "GB/s": b / (us * 1e-6) / 1e9, "frac_hbm": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
        c3_out["per_layer"][f"M={M}"] = {"us": tot_us, "GB/s": layer_bytes / (tot_us * 1e-6) / 1e9,
                                         "frac_hbm": layer_bytes / (tot_us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    c3_out["bytes_per_layer"] = layer_bytes
    if c3:
        stages["c3_decoder_layer"] = c3_out
    # ---------------- c5 figures
    if c5 is not None:
        out5 = {"bytes": c5["bytes"], "launches": c5["launches"], "quantize": c5["quantize"]}
        for form in ("folded", "inv_s"):
            ms = avg[f"c5_decode_{form}"]
            out5[f"decode_{form}"] = {"ms": ms, "GB/s": c5["bytes"] / (ms * 1e-3) / 1e9,
                                      "frac_hbm": c5["bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        codes = sum(part["q"].numel() * 4 for L in c5["layers"] for part in L)
        ms = avg["c5_read_ceiling"]
        rd_gbs = codes / (ms * 1e-3) / 1e9
        out5["read_ceiling"] = {
            "ms": ms, "GB/s": rd_gbs, "frac_hbm": rd_gbs / HBM_PEAK_GBS, "bytes": codes,
            "launch_shapes": {k: list(v) for k, v in zip(("qkv", "o", "gateup", "down"), c5_rd.values())},
            "what": "the same 320 launches as plain streaming reads (awq_read_stream) of each product's "
                    "packed codes, each product kind's launch shape (blocks, unroll) the best of a short "
                    "sweep: the rate one launch per product reaches on this chip"}
        for form in ("folded", "inv_s"):
            out5[f"decode_{form}"]["frac_read_ceiling"] = out5[f"decode_{form}"]["GB/s"] / rd_gbs
        out5["what"] = ("batch-1 decode pass of the 80-layer stack: per layer q|k|v (10240 x 8192), "
                        "o (8192 x 8192), gate|up (57344 x 8192), down (8192 x 28672); folded = 1/s "
                        "folded into the producers of x, inv_s = applied inside the products")
        stages["c5_stack_70b"] = out5

    # Output MSE of plain round-to-nearest (alpha = 0, s = 1) and of the
    # searched scale for the quantizer variants, on the same layer and
    # calibration tokens: one untimed search each, after the timed steps.
    variants = []
    for g, bits, sym in VARIANTS:
        _, _, Lv, bv = awq.awq_search_scales(WA, XA, m, alphas, g, ws=ws_search, bits=bits, symmetric=sym)
        Lv, iv = [float(v) for v in Lv.cpu()], int(bv.cpu()[0])
        variants.append({"group": g, "bits": bits, "grid": "symmetric" if sym else "asymmetric",
                         "loss_rtn": Lv[0], "loss_awq": Lv[iv], "alpha": float(alphas_h[iv]),
                         "rtn_over_awq": Lv[0] / Lv[iv]})
    # the mixed-precision baseline AWQ replaces: the 1 % most salient channels
    # (largest mean |x|) kept in 16-bit, the rest round-to-nearest
    n_keep = KA // 100
    kept = awq.awq_salient_channels(m, n_keep)
    _, _, Lm, _ = awq.awq_search_scales(WA, XA, m, alphas[:1], ws=ws_search, kept=kept)
    mixed = {"kept_channels": n_keep, "group": 128, "bits": 4, "loss": float(Lm.cpu()[0]),
             "loss_rtn": loss_h[0], "loss_awq": loss_h[best_h],
             "loss_over_awq": float(Lm.cpu()[0]) / loss_h[best_h]}
    up = gemm.get("up")
    out = {
        "metric": METRIC,
        "value": gemv_gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "AWQ quantize + W4A16 decode of a Llama-7B MLP up-projection "
                        "(K=4096, N=11008, fp16, 65536 calibration tokens, 20 candidates, "
                        f"{N_ROT * N_PASS} batch-1 and {N_ROT * N_PASS} batch-8 GEMVs over {N_ROT} "
                        "resident weight copies) + W4A16 prefill GEMMs of the Llama-70B MLP "
                        "up- and down-projections (8192->28672, 28672->8192, bf16, M=2048) + "
                        "the 512x512 single linear + Llama-7B decoder-layer decode at M=1,8,32"
                        + ("" if c5 is None else
                           " + batch-1 decode pass of the 80-layer Llama-70B-shaped stack (35.83 GB)"),
            "group_size": 128, "bits": 4,
        },
        "roofline": {"bound": "hbm", "achieved": gemv_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gemv_gbs / HBM_PEAK_GBS, "traffic": measured_traffic("k_gemv1_cu"),
                     "kernel": "k_gemv1_cu (batch 1, one block per compute unit)",
                     "bytes_per_launch": bytes_a,
                     "read_ceiling": read_gbs, "frac_read_ceiling": gemv_gbs / read_gbs},
        "prefill_gemm": None if up is None else {
            "bound": "mfma", "achieved": up["TFLOP/s"], "peak": FP16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": up["frac_fp16_mfma"],
            "flop_per_launch": 2.0 * 2048 * 28672 * 8192, "kernel": "k_gemm"},
        "stages": stages,
        "quantizer_variants": variants,
        "mixed_precision_baseline": mixed,
    }
    if not args.no_cpu_baseline and c4:
        c2 = {"W": WA, "X": XA, "N": NA, "K": KA, "T": wa.T, "s": s, "inv": inv, "q": qs[0],
              "sc": scs[0], "z": zs[0], "x1": xa1}
        out["cpu_baseline"] = cpu_baseline(c2, c4)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def setup_c5(torch, WL, awq, dev, alphas, ws_for, quantize_all: bool):
    """The 80-layer 70B-shaped stack: packed weights of every layer resident
    (35.83 GB), decode inputs and outputs; layer 0 (or every layer) quantized
    by the full path with its timing."""
    print("setup: 80-layer llama70b-shaped stack", file=sys.stderr, flush=True)
    parts_spec = (("qkv", ("q", "k", "v"), 8192), ("o", ("o",), 8192), ("gateup", ("gate", "up"), 8192),
                  ("down", ("down",), 28672))
    layers, nbytes, launches = [], 0, 0
    quant = {"layers_quantized": 0, "ms_per_layer": [], "stage_ms": None}
    sync = torch.cuda.synchronize
    for layer in range(C5_LAYERS):
        L = []
        full = layer == 0 or quantize_all
        if full:
            stage_ms = {}
        for name, lins, K in parts_spec:
            ws = [WL.workload(5, lin, layer) for lin in lins]
            N = sum(w.N for w in ws)
            if full:
                W = torch.empty((N, K), dtype=torch.float16, device=dev)
                r0 = 0
                for w in ws:
                    WL.device_weight(w, dev, out=W[r0:r0 + w.N])
                    r0 += w.N
                X = WL.device_activations(ws[0], ws[0].T, dev)
                sync()
                t0 = torch.cuda.Event(enable_timing=True)
                t1 = torch.cuda.Event(enable_timing=True)
                t0.record()
                m = awq.awq_act_stats(X)
                s, inv, _, _ = awq.awq_search_scales(W, X, m, alphas)
                q, sc, z = awq.awq_quantize_pack(W, s)
                t1.record()
                sync()
                stage_ms[name] = t0.elapsed_time(t1)
                del W, X, m, s
            else:
                q, sc, z = WL.device_packed(N, K, dev, 1000 * layer + len(L))
                inv = torch.ones(K, dtype=torch.float32, device=dev)
            L.append({"K": K, "N": N, "q": q, "sc": sc, "z": z, "inv": inv,
                      "y": torch.empty((1, N), dtype=torch.float16, device=dev)})
            nbytes += packed_bytes(N, K)
            launches += 1
        if full:
            quant["layers_quantized"] += 1
            quant["ms_per_layer"].append(sum(stage_ms.values()))
            if layer == 0:
                quant["stage_ms"] = stage_ms
        layers.append(L)
        if layer % 20 == 19:
            print(f"setup: c5 layers 0..{layer} resident", file=sys.stderr, flush=True)
    sync()
    per = quant["ms_per_layer"]
    quant["layer0_ms"] = per[0]
    if len(per) == C5_LAYERS:
        quant["all_layers_s_measured"] = sum(per) / 1000.0
    else:
        quant["all_layers_s_extrapolated"] = per[0] * C5_LAYERS / 1000.0
    quant["what"] = ("statistics over 131072 calibration tokens per input, 20-candidate searches "
                     "(q|k|v and gate|up each searched on their concatenated rows), quantize + pack; "
                     "measured on the GPU with events, once, outside the timed steps"
                     + ("" if quantize_all else "; layers 1..79 carry seeded random codes, steps "
                        "and zero points, and the 80-layer time is layer 0's x 80 (extrapolated)"))
    quant.pop("ms_per_layer")
    x = {8192: WL.device_activations(WL.workload(5, "q", 0), 1, dev, WL.ROLE_XDEC),
         28672: WL.device_activations(WL.workload(5, "down", 0), 1, dev, WL.ROLE_XDEC)}
    return {"layers": layers, "bytes": nbytes, "launches": launches, "quantize": quant, "x": x}


if __name__ == "__main__":
    sys.exit(main())
