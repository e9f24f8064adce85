"""Benchmark of the AWQ W4A16 hot path on one MI355X.

One step = one pass of the whole path:
  part A, Llama-7B MLP up-projection (K=4096 -> N=11008, fp16, 65536
          calibration tokens = 128 sequences x 512):
          mean|x| statistics -> 20-candidate scale search -> quantize + pack
          -> 32 batch-1 decode GEMVs (one on the freshly packed weights, 31 on
          resident copies of the same size, so every launch streams its
          weights from HBM rather than from the 256 MB last-level cache)
          -> 32 batch-8 GEMVs over the same copies
  part B, Llama-70B MLP up-projection prefill (K=8192 -> N=28672, bf16, 2048
          tokens): the matrix-core W4A16 GEMM on weights quantized (with the
          same AWQ path) during setup.
The decode GEMVs run from a captured HIP graph (back-to-back launches).

value = effective HBM GB/s of the batch-1 GEMV: packed bytes (codes + fp16
        steps + uint8 zero points, 0.5234 B per weight) per launch / average
        launch time, measured with HIP events on the launch stream.
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
N_ROT = 32          # distinct resident weight copies (755 MB: beyond the last-level cache)
N_PASS = 4          # passes over the copies per decode graph: 128 products per replay, so that
                    # the graph's own launch cost (~15 us) is spread as in a whole decode step
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
    return ap.parse_args()


def packed_bytes(N: int, K: int) -> int:
    return N * K // 2 + N * (K // 128) * 3


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


def cpu_baseline(W, q, sc, z, x, budget_s: float = 12.0) -> dict:
    """The CPU oracle's batch-1 product on the same layer, timed on the host."""
    import numpy as np

    import oracle as O
    words = q.cpu().numpy()
    step = sc.cpu().numpy()
    zeros = z.cpu().numpy()
    xs = x.float().cpu().numpy()
    N, K = W.shape
    reps, t0 = 0, time.perf_counter()
    while True:
        O.w4a16_matmul(xs, words, step, zeros)
        reps += 1
        el = time.perf_counter() - t0
        if el > budget_s or reps >= 1000:
            break
    gbs = packed_bytes(N, K) * reps / el / 1e9
    cores = len(os.sched_getaffinity(0))
    return {"value": gbs, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} batch-1 W4A16 products of the full {N}x{K} layer by the NumPy "
                      f"oracle (unpack, fp64 dequantize, fp64 matvec; BLAS threads up to {cores}), "
                      f"{el:.1f} s"}


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

    # ---------------- part A inputs (Llama-7B MLP up, fp16)
    wa = WL.workload(2)
    NA, KA = wa.N, wa.K
    print(f"setup: {wa.name}, T={wa.T}", file=sys.stderr, flush=True)
    WA = WL.weight(wa).to(dev)
    XA = WL.calibration(wa).to(dev)
    xa1 = WL.decode_input(wa, 1).to(dev)
    xa8 = WL.decode_input(wa, 8).to(dev)
    alphas = torch.from_numpy(WL.alpha_grid(20)).to(dev)
    GA = KA // 128
    ws_stats = torch.empty(awq.awq_workspace_bytes(awq.AWQ_OP_ACT_STATS, 0, NA, KA, wa.T, 0),
                           dtype=torch.uint8, device=dev)
    ws_search = torch.empty(awq.awq_workspace_bytes(awq.AWQ_OP_SEARCH, 0, NA, KA, wa.T, 20),
                            dtype=torch.uint8, device=dev)
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

    # resident copies: quantize once so that every copy holds real packed weights
    awq.awq_act_stats(XA, m, ws=ws_stats)
    awq.awq_search_scales(WA, XA, m, alphas, s_out=s, inv_s_out=inv, loss_out=loss,
                          best_idx_out=best, ws=ws_search)
    awq.awq_quantize_pack(WA, s, qweight=qs[0], scales=scs[0], zeros=zs[0])
    for i in range(1, N_ROT):
        qs[i].copy_(qs[0])
        scs[i].copy_(scs[0])
        zs[i].copy_(zs[0])
    torch.cuda.synchronize()

    # ---------------- part B inputs (Llama-70B MLP up prefill, bf16)
    wb = WL.workload(4, "up")
    NB, KB, MB = wb.N, wb.K, wb.Ms[0]
    print(f"setup: {wb.name}, M={MB}", file=sys.stderr, flush=True)
    WB = WL.weight(wb).to(dev)
    XB = WL.calibration(wb).to(dev)
    xpre = WL.prefill_input(wb, MB).to(dev)
    mB = awq.awq_act_stats(XB)
    sB, invB, _, _ = awq.awq_search_scales(WB, XB, mB, alphas)
    qB, scB, zB = awq.awq_quantize_pack(WB, sB)
    del WB
    yB = torch.empty((MB, NB), dtype=torch.bfloat16, device=dev)
    ws_gemm = torch.empty(awq.awq_workspace_bytes(awq.AWQ_OP_GEMM, MB, NB, KB, 0, 0),
                          dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # ---------------- decode graphs
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.set_stream(stream)

    def decode1():
        for _ in range(N_PASS):
            for i in range(N_ROT):
                awq.awq_w4a16_gemm(xa1, qs[i], scs[i], zs[i], inv, y=y1[i])

    def decode8():
        for _ in range(N_PASS):
            for i in range(N_ROT):
                awq.awq_w4a16_gemm(xa8, qs[i], scs[i], zs[i], inv, y=y8[i])

    decode1()
    decode8()
    torch.cuda.synchronize()
    g1, g8 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1, stream=stream):
        decode1()
    with torch.cuda.graph(g8, stream=stream):
        decode8()
    torch.cuda.synchronize()

    names = ["act_stats", "search", "quantize", "gemv_m1", "gemv_m8", "gemm_prefill"]

    def new_events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]

    ev = new_events()

    def step(ev):
        ev[0].record(stream)
        awq.awq_act_stats(XA, m, ws=ws_stats)
        ev[1].record(stream)
        awq.awq_search_scales(WA, XA, m, alphas, s_out=s, inv_s_out=inv, loss_out=loss,
                              best_idx_out=best, ws=ws_search)
        ev[2].record(stream)
        awq.awq_quantize_pack(WA, s, qweight=qs[0], scales=scs[0], zeros=zs[0])
        ev[3].record(stream)
        g1.replay()
        ev[4].record(stream)
        g8.replay()
        ev[5].record(stream)
        awq.awq_w4a16_gemm(xpre, qB, scB, zB, invB, y=yB, ws=ws_gemm)
        ev[6].record(stream)

    for _ in range(args.warmup):
        step(ev)
    torch.cuda.synchronize()
    # the K steps are enqueued back to back (the host runs ahead of the GPU, so
    # the events time GPU work, not the host's enqueue latency) and bracketed
    # by one synchronization on each side
    evs = [new_events() for _ in range(args.steps)]
    per = {n: 0.0 for n in names}
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for e in evs:
        for i, n in enumerate(names):
            per[n] += e[i].elapsed_time(e[i + 1])
    K_ = args.steps
    avg = {n: per[n] / K_ for n in names}            # ms per step per phase
    ms_step = wall * 1000.0 / K_

    bytes_a = packed_bytes(NA, KA)
    gemv1_us = avg["gemv_m1"] * 1000.0 / (N_ROT * N_PASS)
    gemv8_us = avg["gemv_m8"] * 1000.0 / (N_ROT * N_PASS)
    gemv_gbs = bytes_a / (gemv1_us * 1e-6) / 1e9
    gemv8_gbs = bytes_a / (gemv8_us * 1e-6) / 1e9
    gemm_flop = 2.0 * MB * NB * KB
    gemm_tflops = gemm_flop / (avg["gemm_prefill"] * 1e-3) / 1e12
    # matrix-core operations the search executes: the direct form contracts
    # over the tokens per candidate; the Gram form (taken by the library when
    # it needs under half of those, see awq_search_scales in include/awq.h)
    # forms X^T X once and per candidate contracts with the 256 x 256 blocks
    # of it on and below the diagonal, each as two fp16 parts
    Tp = (wa.T + 255) // 256 * 256
    gblk = (KA + 255) // 256
    direct_flop = 2.0 * wa.T * NA * KA * 20
    gram_flop = 2.0 * Tp * KA * KA + 20 * 2.0 * NA * 256 * 256 * gblk * (gblk + 1)
    search_gram = KA <= 16384 and gram_flop < 0.5 * direct_flop
    search_flop = gram_flop if search_gram else direct_flop
    loss_h = [float(v) for v in loss.cpu()]
    best_h = int(best.cpu()[0])
    alphas_h = alphas.cpu().numpy()
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
    stats_bytes = wa.T * KA * 2
    quant_bytes = NA * KA * 2 + bytes_a
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
        "gemv_m1": {"us_per_launch": gemv1_us, "GB/s": gemv_gbs, "frac_hbm": gemv_gbs / HBM_PEAK_GBS},
        "gemv_m8": {"us_per_launch": gemv8_us, "GB/s": gemv8_gbs, "frac_hbm": gemv8_gbs / HBM_PEAK_GBS},
        "gemm_prefill": {"ms": avg["gemm_prefill"], "TFLOP/s": gemm_tflops,
                         "frac_fp16_mfma": gemm_tflops / FP16_MFMA_PEAK_TFLOPS},
    }
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
                        "resident weight copies) + W4A16 prefill GEMM of a "
                        "Llama-70B MLP up-projection (K=8192, N=28672, bf16 input, M=2048)",
            "group_size": 128, "bits": 4,
        },
        "roofline": {"bound": "hbm", "achieved": gemv_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gemv_gbs / HBM_PEAK_GBS, "traffic": measured_traffic("k_gemv1_cu"),
                     "kernel": "k_gemv1_cu (batch 1, one block per compute unit)",
                     "bytes_per_launch": bytes_a},
        "prefill_gemm": {"bound": "mfma", "achieved": gemm_tflops, "peak": FP16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": gemm_tflops / FP16_MFMA_PEAK_TFLOPS,
                         "flop_per_launch": gemm_flop, "kernel": "k_gemm"},
        "stages": stages,
        "quantizer_variants": variants,
        "mixed_precision_baseline": mixed,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(WA, qs[0], scs[0], zs[0], xa1)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
