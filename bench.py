#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 linear-layer hot path on one MI355X.

Workload: the Wan-14B-shaped FFN on one GPU, M = 32760 tokens, hidden 5120, FFN 13824:
    quantize X[32760,5120] -> mm_fp4 fc_in (W1 13824x5120) -> GELU -> quantize H[32760,13824]
    -> mm_fp4 fc_out (W2 5120x13824) -> bf16 out[32760,5120]
The headline step keeps the packed NVFP4 values in the MFMA fragment layout (scales in 128x4); the
same step on row-major packed values is timed beside it ("ffn_step_row_major").
Weights are prequantized once at load (timed separately). Inputs are seeded synthetic bf16
tensors (workloads/, config 4: X ~ N(0,1) with 1% outlier channels x20, W ~ N(0, 0.01^2)),
resident in HBM before timing. One step = one pass of that FFN. The MXFP8 W8A8 path at the same
fc_in shape (config 5: online weight conversion, activation quantize, mm_mxfp8) is timed in a
second loop and reported under "mxfp8".

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP4_TFLOPS = 10100.0   # MI355X dense FP4/FP6 MFMA (published)
PEAK_FP8_TFLOPS = 5000.0    # dense FP8
PEAK_F16_TFLOPS = 2500.0    # dense FP16/BF16
PEAK_HBM_GBS = 8000.0       # HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="tokens of the FFN the CPU oracle runs for cpu_baseline")
    ap.add_argument("--no-mxfp8", action="store_true")
    ap.add_argument("--no-shapes", action="store_true", help="skip the other configurations' shapes")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured-ceiling probes")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device-to-device copy (reference for HBM byte counters)")
    return ap.parse_args()


CSRC = os.path.join(ROOT, "block_scaled_precision_nvfp4_amd", "csrc")
GEMM_SOURCES = ("gemm_fp4.hip", "gemm_common.hpp", "common.hpp")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "mm_fp4_wan14b_ffn_pmc.txt")


def gemm_sources_sha256() -> str:
    """Digest of the sources the NVFP4 GEMM kernel is compiled from (identifies the kernel version)."""
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when the summary
    is missing or was taken on a different version of the GEMM source."""
    try:
        kv = {}
        with open(PMC_SUMMARY) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel sources sha256") != gemm_sources_sha256():
            return None
        return float(kv[f"{kernel} hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def nvfp4_sf_shape(rows, k):
    return (-(-rows // 128) * 128, -(-(k // 16) // 4) * 4)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the FFN would shard "
              "by tokens or by output features with no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_scaled_precision_nvfp4_amd as bsp
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 2}), flush=True)
        return
    cfg = W.config(4)
    tx, tw1, tw2 = cfg.tensor("X"), cfg.tensor("W"), cfg.tensor("W2")
    M, K1, N1 = tx.rows, tx.cols, tw1.rows          # 32760, 5120, 13824
    N2 = tw2.rows                                   # 5120

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    t0 = time.perf_counter()
    x = up(W.generate(tx))
    w1 = up(W.generate(tw1))
    w2 = up(W.generate(tw2))
    log(f"inputs generated and uploaded in {time.perf_counter() - t0:.1f}s")

    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # ---- load time: weight global scale + prequantization, in the pages' row-major layout and with
    # the packed values in the fragment layout (the same codes and 128x4 scales)
    l0, l1, l2 = ev(), ev(), ev()
    # untimed first calls (module and kernel loading), then the timed load of both weights
    _wq = bsp.bsp_nvfp4_prequantize_weight(w1)
    _wq = bsp.bsp_nvfp4_prequantize_weight_frag(w1)
    torch.cuda.synchronize()
    del _wq
    l0.record(stream)
    pw1, sw1, g1, _, _ = bsp.bsp_nvfp4_prequantize_weight(w1)
    pw2, sw2, g2, _, _ = bsp.bsp_nvfp4_prequantize_weight(w2)
    l1.record(stream)
    pw1f, sw1f, g1f, _, _ = bsp.bsp_nvfp4_prequantize_weight_frag(w1)
    pw2f, sw2f, g2f, _, _ = bsp.bsp_nvfp4_prequantize_weight_frag(w2)
    l2.record(stream)
    one = torch.ones(1, dtype=torch.float32, device=dev)
    a1 = bsp.bsp_nvfp4_alpha(one, g1)
    a2 = bsp.bsp_nvfp4_alpha(one, g2)
    torch.cuda.synchronize()
    load_ms, load_frag_ms = l0.elapsed_time(l1), l1.elapsed_time(l2)
    assert g1f.item() == g1.item() and g2f.item() == g2.item()
    del w1, w2

    # ---- step buffers (row-major packed values, and the fragment layout [ceil(rows/32), K/64, 1 KB])
    px = torch.empty((M, K1 // 2), dtype=torch.uint8, device=dev)
    sx = torch.empty(nvfp4_sf_shape(M, K1), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N1), dtype=torch.bfloat16, device=dev)
    ph = torch.empty((M, N1 // 2), dtype=torch.uint8, device=dev)
    sh = torch.empty(nvfp4_sf_shape(M, N1), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N2), dtype=torch.bfloat16, device=dev)
    pxf = torch.empty((-(-M // 32), K1 // 64, 1024), dtype=torch.uint8, device=dev)
    phf = torch.empty((-(-M // 32), N1 // 64, 1024), dtype=torch.uint8, device=dev)

    # one step: quantize X -> fc_in -> GELU fused into the NVFP4 quantize of H -> fc_out. The
    # headline step keeps the packed values in the fragment layout (each wave loads a 1 KB operand
    # fragment with one coalesced read); the same step on row-major packed values is timed beside it.
    names = ["quantize_x", "mm_fp4_fc_in", "gelu_quantize_h", "mm_fp4_fc_out"]
    frag_calls = [lambda: bsp.bsp_nvfp4_quantize_frag(x, one, pxf, sx),
                  lambda: bsp.bsp_mm_fp4_frag(pxf, sx, pw1f, sw1f, M, N1, a1, out=y),
                  lambda: bsp.bsp_nvfp4_quantize_gelu_frag(y, one, phf, sh),
                  lambda: bsp.bsp_mm_fp4_frag(phf, sh, pw2f, sw2f, M, N2, a2, out=out)]
    linear_calls = [lambda: bsp.bsp_nvfp4_quantize(x, one, px, sx),
                    lambda: bsp.bsp_mm_fp4(px, sx, pw1, sw1, a1, out=y),
                    lambda: bsp.bsp_nvfp4_quantize_gelu(y, one, ph, sh),
                    lambda: bsp.bsp_mm_fp4(ph, sh, pw2, sw2, a2, out=out)]

    def timed_steps(calls):
        """W untimed steps, then K timed ones bracketed by synchronizations; HIP events on the
        kernels' stream around every launch. Returns (wall ms per step, mean ms per kernel, spread)."""
        def step(events=None):
            for j, c in enumerate(calls):
                if events:
                    events[j].record(stream)
                c()
            if events:
                events[-1].record(stream)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        evs = [[ev() for _ in range(len(calls) + 1)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = {n: [e[j].elapsed_time(e[j + 1]) for e in evs] for j, n in enumerate(names)}
        per["step"] = [e[0].elapsed_time(e[-1]) for e in evs]
        mean = {n: sum(per[n]) / args.steps for n in names}
        spread = {n: {"median": round(float(np.median(v)), 4), "p10": round(float(np.percentile(v, 10)), 4),
                      "p90": round(float(np.percentile(v, 90)), 4)} for n, v in per.items()}
        return wall * 1e3 / args.steps, mean, spread

    ms_per_step, kms, spread = timed_steps(frag_calls)
    ms_lin, kms_lin, spread_lin = timed_steps(linear_calls)

    # Kernel durations without the event records between a step's launches: the quantize of X (both
    # layouts) and the RMSNorm + quantize prologue back to back over two copies of X and of the
    # outputs in turn (1.1 GB between reuses of a buffer, so no pass is served from the 256 MB
    # Infinity Cache), the GELU-fused quantize of H the same way, and the unfused GELU and plain
    # quantize of H (0.9 GB inputs) on their own. The step's own quantize times stay as *_in_step.
    h = bsp.bsp_gelu_tanh_bf16(y)
    x2 = x.clone()
    px2, sx2, pxf2 = torch.empty_like(px), torch.empty_like(sx), torch.empty_like(pxf)
    reps = max(4, 2 * (args.steps // 4))
    kms["quantize_x_in_step"] = kms["quantize_x"]
    kms["gelu_quantize_h_in_step"] = kms["gelu_quantize_h"]
    xs, pxs, sxs, pxfs = (x, x2), (px, px2), (sx, sx2), (pxf, pxf2)
    qx_calls = [lambda i=i: bsp.bsp_nvfp4_quantize_frag(xs[i], one, pxfs[i], sxs[i]) for i in range(2)]
    ql_calls = [lambda i=i: bsp.bsp_nvfp4_quantize(xs[i], one, pxs[i], sxs[i]) for i in range(2)]
    nq_calls = [lambda i=i: bsp.bsp_nvfp4_quantize_rmsnorm(xs[i], one, None, 1e-6, pxs[i], sxs[i])
                for i in range(2)]
    # the GELU-fused quantize of H back to back over two copies of the fc_in output (in the step it
    # follows fc_in, whose 0.9 GB output is still being written back)
    y2 = y.clone()
    ys, phfs, shs = (y, y2), (phf, torch.empty_like(phf)), (sh, torch.empty_like(sh))
    phs = (ph, torch.empty_like(ph))
    gq_calls = [lambda i=i: bsp.bsp_nvfp4_quantize_gelu_frag(ys[i], one, phfs[i], shs[i]) for i in range(2)]
    gl_calls = [lambda i=i: bsp.bsp_nvfp4_quantize_gelu(ys[i], one, phs[i], shs[i]) for i in range(2)]
    for name, fns in (("quantize_x", qx_calls),
                      ("quantize_x_row_major", ql_calls),
                      ("rmsnorm_quantize_x", nq_calls),
                      ("gelu_quantize_h", gq_calls),
                      ("gelu_quantize_h_row_major", gl_calls),
                      ("gelu", [lambda: bsp.bsp_gelu_tanh_bf16(y, out=h)]),
                      ("quantize_h", [lambda: bsp.bsp_nvfp4_quantize_frag(h, one, phf, sh)])):
        for f in fns:
            f()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for i in range(reps):
            fns[i % len(fns)]()
        e1.record(stream)
        torch.cuda.synchronize()
        kms[name] = e0.elapsed_time(e1) / reps
    del h, x2, px2, sx2, pxf2, y2, ys, phs, phfs, shs

    gemm_flops = 2.0 * M * N1 * K1 + 2.0 * M * N2 * N1
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12

    def qbytes(m, k):
        return 2 * m * k + m * k // 2 + nvfp4_sf_shape(m, k)[0] * k // 16

    def qrate(ms, m, k):
        return {"ms": ms, "GB/s": qbytes(m, k) / ms / 1e6}

    def grate(ms, m, n, k):
        return {"ms": ms, "TFLOPS": 2.0 * m * n * k / ms / 1e9}

    kernels = {
        "quantize_x": qrate(kms["quantize_x"], M, K1),
        "quantize_x_in_step": qrate(kms["quantize_x_in_step"], M, K1),
        "quantize_x_row_major": qrate(kms["quantize_x_row_major"], M, K1),
        "rmsnorm_quantize_x": qrate(kms["rmsnorm_quantize_x"], M, K1),
        "gelu_quantize_h": qrate(kms["gelu_quantize_h"], M, N1),
        "gelu_quantize_h_in_step": qrate(kms["gelu_quantize_h_in_step"], M, N1),
        "gelu_quantize_h_row_major": qrate(kms["gelu_quantize_h_row_major"], M, N1),
        "quantize_h": qrate(kms["quantize_h"], M, N1),
        "gelu": {"ms": kms["gelu"], "GB/s": 4.0 * M * N1 / kms["gelu"] / 1e6},
        "mm_fp4_fc_in": grate(kms["mm_fp4_fc_in"], M, N1, K1),
        "mm_fp4_fc_out": grate(kms["mm_fp4_fc_out"], M, N2, N1),
        "mm_fp4_fc_in_row_major": grate(kms_lin["mm_fp4_fc_in"], M, N1, K1),
        "mm_fp4_fc_out_row_major": grate(kms_lin["mm_fp4_fc_out"], M, N2, N1),
    }
    for k_, v in kernels.items():
        if "GB/s" in v:
            v["frac_hbm"] = v["GB/s"] / PEAK_HBM_GBS
        else:
            v["frac_fp4_peak"] = v["TFLOPS"] / PEAK_FP4_TFLOPS
            v["frac_f16_mfma_peak"] = v["TFLOPS"] / PEAK_F16_TFLOPS
    log(json.dumps(kernels))

    dom = "mm_fp4_fc_in" if kms["mm_fp4_fc_in"] >= kms["mm_fp4_fc_out"] else "mm_fp4_fc_out"
    dom_tf = kernels[dom]["TFLOPS"]
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(dom_tf, 2),
                "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s", "frac": round(dom_tf / PEAK_FP4_TFLOPS, 4),
                "traffic": measured_traffic(dom),
                "mfma_used": "v_mfma_f32_32x32x16_f16 (exact fp16 dequant of e2m1 x e4m3)",
                "frac_of_f16_mfma_peak": round(dom_tf / PEAK_F16_TFLOPS, 4)}

    result = {
        "metric": "mm_fp4 TFLOPS (% FP4 MFMA peak) + quantize GB/s (% HBM) at Wan-14B FFN shape",
        "value": round(value, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "Wan-14B FFN on one GPU: X[32760,5120] -> fc_in 13824x5120 -> GELU "
                               "(fused into the NVFP4 quantize of H) -> fc_out 5120x13824, NVFP4 W4A4, "
                               "bf16 out",
                   "layout": "packed values in the MFMA fragment layout (1 KB per 32-row tile and "
                             "64-K step), scales in 128x4; the row-major step is ffn_step_row_major",
                   "format": "nvfp4 (e2m1 + e4m3 per 16, fp32 global scale); the GEMMs multiply "
                             "exact fp16 dequantized operands with fp32 accumulation, the quantizers "
                             "compute in fp32",
                   "tokens": M, "hidden": K1, "ffn": N1, "value_is": "GEMM FLOPs of both "
                   "projections / whole-step time (quantizes and GELU included)"},
        "roofline": roofline,
        "kernels": {k_: {kk: round(vv, 4) for kk, vv in v.items()} for k_, v in kernels.items()},
        "quantize_GBs": round(min(kernels["quantize_x"]["GB/s"], kernels["quantize_h"]["GB/s"]), 1),
        "quantize_frac_hbm": round(min(kernels["quantize_x"]["frac_hbm"],
                                       kernels["quantize_h"]["frac_hbm"]), 4),
        "load_time_ms": {"prequantize_w1_w2": round(load_ms, 3),
                         "prequantize_w1_w2_fragment_layout": round(load_frag_ms, 3)},
        "event_ms_spread": spread,
        "ffn_step_row_major": {
            "ms_per_step": round(ms_lin, 4), "TFLOPS": round(gemm_flops / (ms_lin * 1e-3) / 1e12, 2),
            "kernel_ms": {n: round(v, 4) for n, v in kms_lin.items()},
            "event_ms_spread": spread_lin},
    }
    log(json.dumps(result["ffn_step_row_major"]))

    # ---- the same FFN step with fc_in's epilogue emitting the NVFP4 of gelu(C) directly
    # (bsp_mm_fp4_gelu_nvfp4: no bf16 H in memory, no separate GELU + quantize launch)
    def step_epi(events=None):
        if events:
            events[0].record(stream)
        bsp.bsp_nvfp4_quantize(x, one, px, sx)
        if events:
            events[1].record(stream)
        bsp.bsp_mm_fp4_gelu_nvfp4(px, sx, pw1, sw1, a1, one, ph, sh)
        if events:
            events[2].record(stream)
        bsp.bsp_mm_fp4(ph, sh, pw2, sw2, a2, out=out)
        if events:
            events[3].record(stream)

    for _ in range(args.warmup):
        step_epi()
    torch.cuda.synchronize()
    eve = [[ev() for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_epi(eve[i])
    torch.cuda.synchronize()
    wall_e = time.perf_counter() - t0
    fcin_epi = sum(e[1].elapsed_time(e[2]) for e in eve) / args.steps
    result["ffn_step_gelu_nvfp4_epilogue"] = {
        "ms_per_step": round(wall_e * 1e3 / args.steps, 4),
        "TFLOPS": round(gemm_flops / (wall_e / args.steps) / 1e12, 2),
        "mm_fp4_gelu_nvfp4_fc_in_ms": round(fcin_epi, 4),
        "row_major_fc_in_plus_gelu_quantize_ms": round(kms_lin["mm_fp4_fc_in"] + kms_lin["gelu_quantize_h"], 4),
        "row_major_two_kernel_ms_per_step": round(ms_lin, 4)}
    log(json.dumps(result["ffn_step_gelu_nvfp4_epilogue"]))

    # ---- per-token activation scales at the fc_in shape: quantize X per row + mm_fp4 with row alphas
    gx = torch.empty((M,), dtype=torch.float32, device=dev)
    for _ in range(max(1, args.warmup)):
        bsp.bsp_nvfp4_quantize_per_token(x, px, sx, gx)
        bsp.bsp_mm_fp4_per_token(px, sx, pw1, sw1, gx, g1, out=y)
    torch.cuda.synchronize()
    ept = [[ev() for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        ept[i][0].record(stream)
        bsp.bsp_nvfp4_quantize_per_token(x, px, sx, gx)
        ept[i][1].record(stream)
        bsp.bsp_mm_fp4_per_token(px, sx, pw1, sw1, gx, g1, out=y)
        ept[i][2].record(stream)
    torch.cuda.synchronize()
    qpt = sum(e[0].elapsed_time(e[1]) for e in ept) / args.steps
    gpt = sum(e[1].elapsed_time(e[2]) for e in ept) / args.steps
    # the per-token quantize back to back over two copies of X and of its outputs (in the loop above
    # each call follows a GEMM whose 0.9 GB output is still being written back)
    x2 = x.clone()
    outs2 = [(px, sx, gx), (torch.empty_like(px), torch.empty_like(sx), torch.empty_like(gx))]
    qpt_b2b = _event_ms([lambda i=i: bsp.bsp_nvfp4_quantize_per_token((x, x2)[i], *outs2[i])
                         for i in range(2)], max(4, 2 * (args.steps // 4)))
    del x2, outs2
    result["per_token"] = {
        "quantize_per_token_x_ms": round(qpt, 4),
        "quantize_per_token_GBs": round(qbytes(M, K1) / qpt / 1e6, 1),
        "quantize_per_token_frac_hbm": round(qbytes(M, K1) / qpt / 1e6 / PEAK_HBM_GBS, 4),
        "quantize_per_token_x_back_to_back_ms": round(qpt_b2b, 4),
        "quantize_per_token_back_to_back_frac_hbm": round(qbytes(M, K1) / qpt_b2b / 1e6 / PEAK_HBM_GBS, 4),
        "mm_fp4_per_token_fc_in_ms": round(gpt, 4),
        "mm_fp4_per_token_TFLOPS": round(2.0 * M * N1 * K1 / gpt / 1e9, 2)}
    log(json.dumps(result["per_token"]))

    # ---- MXFP8 W8A8 at the fc_in shape (config 5)
    if not args.no_mxfp8:
        del y, ph, sh
        c5 = W.config(5)
        x5 = up(W.generate(c5.tensor("X")))
        w5 = up(W.generate(c5.tensor("W")))
        m0, m1 = ev(), ev()
        m0.record(stream)
        qw, sw = bsp.bsp_mxfp8_quantize(w5)       # online BF16 -> MXFP8 weight conversion
        m1.record(stream)
        pw4, sw4 = bsp.bsp_mxfp4_quantize(w5)     # and to MXFP4 for the mm_fp4 MX variant
        pw4f, sw4f = bsp.bsp_mxfp4_quantize_frag(w5)   # (MFMA fragment layout)
        qwf, swf = bsp.bsp_mxfp8_quantize_frag(w5)
        qx = torch.empty((M, K1), dtype=torch.uint8, device=dev)
        sxm = torch.empty((M, K1 // 32), dtype=torch.uint8, device=dev)
        out5 = torch.empty((M, N1), dtype=torch.bfloat16, device=dev)
        del w5

        def step8(e=None):
            if e:
                e[0].record(stream)
            bsp.bsp_mxfp8_quantize(x5, qx, sxm)
            if e:
                e[1].record(stream)
            bsp.bsp_mm_mxfp8(qx, sxm, qw, sw, out=out5)
            if e:
                e[2].record(stream)

        for _ in range(args.warmup):
            step8()
        torch.cuda.synchronize()
        e8 = [[ev() for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            step8(e8[i])
        torch.cuda.synchronize()
        q8 = sum(e[0].elapsed_time(e[1]) for e in e8) / args.steps
        g8 = sum(e[1].elapsed_time(e[2]) for e in e8) / args.steps
        tf8 = 2.0 * M * N1 * K1 / g8 / 1e9
        qb8 = 2 * M * K1 + M * K1 + M * K1 // 32
        # the quantize back to back over two copies of X and of its outputs (as for the NVFP4 one)
        x52 = x5.clone()
        o52 = [(qx, sxm), (torch.empty_like(qx), torch.empty_like(sxm))]
        q8_b2b = _event_ms([lambda i=i: bsp.bsp_mxfp8_quantize((x5, x52)[i], *o52[i]) for i in range(2)],
                           max(4, 2 * (args.steps // 4)))
        del o52
        result["mxfp8"] = {
            "mm_mxfp8_ms": round(g8, 4), "TFLOPS": round(tf8, 2),
            "frac_fp8_peak": round(tf8 / PEAK_FP8_TFLOPS, 4),
            "quantize_ms": round(q8, 4), "quantize_GBs": round(qb8 / q8 / 1e6, 1),
            "quantize_frac_hbm": round(qb8 / q8 / 1e6 / PEAK_HBM_GBS, 4),
            "quantize_back_to_back_ms": round(q8_b2b, 4),
            "quantize_back_to_back_frac_hbm": round(qb8 / q8_b2b / 1e6 / PEAK_HBM_GBS, 4),
            "weight_conversion_ms": round(m0.elapsed_time(m1), 4)}
        log(json.dumps(result["mxfp8"]))
        del qx, sxm

        # ---- the same MXFP8 layer with both operands in the MFMA fragment layout
        qxf, sxf = bsp.bsp_mxfp8_quantize_frag(x5)

        def step8f(e=None):
            if e:
                e[0].record(stream)
            bsp.bsp_mxfp8_quantize_frag(x5, qxf, sxf)
            if e:
                e[1].record(stream)
            bsp.bsp_mm_mxfp8_frag(qxf, sxf, qwf, swf, M, N1, out=out5)
            if e:
                e[2].record(stream)

        for _ in range(args.warmup):
            step8f()
        torch.cuda.synchronize()
        e8f = [[ev() for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            step8f(e8f[i])
        torch.cuda.synchronize()
        q8f = sum(e[0].elapsed_time(e[1]) for e in e8f) / args.steps
        g8f = sum(e[1].elapsed_time(e[2]) for e in e8f) / args.steps
        tf8f = 2.0 * M * N1 * K1 / g8f / 1e9
        qb8f = 2 * M * K1 + (-(-M // 32) * 32) * (K1 + K1 // 32)
        result["mxfp8_frag"] = {
            "mm_mxfp8_frag_ms": round(g8f, 4), "TFLOPS": round(tf8f, 2),
            "frac_fp8_peak": round(tf8f / PEAK_FP8_TFLOPS, 4),
            "quantize_frag_ms": round(q8f, 4), "quantize_GBs": round(qb8f / q8f / 1e6, 1),
            "quantize_frac_hbm": round(qb8f / q8f / 1e6 / PEAK_HBM_GBS, 4),
            "step_ms": round(q8f + g8f, 4), "step_ms_row_major_layout": round(q8 + g8, 4)}
        log(json.dumps(result["mxfp8_frag"]))
        del qxf, sxf, qwf, swf

        # ---- MXFP4 (mm_fp4 with MX scales, the format gfx950's FP4 MFMA takes natively)
        px4 = torch.empty((M, K1 // 2), dtype=torch.uint8, device=dev)
        sx4 = torch.empty((-(-M // 128) * 128, K1 // 128 * 4), dtype=torch.uint8, device=dev)

        def step4(e=None):
            if e:
                e[0].record(stream)
            bsp.bsp_mxfp4_quantize(x5, px4, sx4)
            if e:
                e[1].record(stream)
            bsp.bsp_mm_mxfp4(px4, sx4, pw4, sw4, out=out5)
            if e:
                e[2].record(stream)

        for _ in range(args.warmup):
            step4()
        torch.cuda.synchronize()
        e4 = [[ev() for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            step4(e4[i])
        torch.cuda.synchronize()
        q4 = sum(e[0].elapsed_time(e[1]) for e in e4) / args.steps
        g4 = sum(e[1].elapsed_time(e[2]) for e in e4) / args.steps
        tf4 = 2.0 * M * N1 * K1 / g4 / 1e9
        qb4 = 2 * M * K1 + M * K1 // 2 + (-(-M // 128) * 128) * K1 // 32
        o42 = [(px4, sx4), (torch.empty_like(px4), torch.empty_like(sx4))]
        q4_b2b = _event_ms([lambda i=i: bsp.bsp_mxfp4_quantize((x5, x52)[i], *o42[i]) for i in range(2)],
                           max(4, 2 * (args.steps // 4)))
        del o42
        result["mxfp4"] = {
            "mm_mxfp4_ms": round(g4, 4), "TFLOPS": round(tf4, 2),
            "frac_fp4_peak": round(tf4 / PEAK_FP4_TFLOPS, 4),
            "quantize_ms": round(q4, 4), "quantize_GBs": round(qb4 / q4 / 1e6, 1),
            "quantize_frac_hbm": round(qb4 / q4 / 1e6 / PEAK_HBM_GBS, 4),
            "quantize_back_to_back_ms": round(q4_b2b, 4),
            "quantize_back_to_back_frac_hbm": round(qb4 / q4_b2b / 1e6 / PEAK_HBM_GBS, 4)}
        log(json.dumps(result["mxfp4"]))
        del px4, sx4

        # ---- the same MXFP4 layer with both operands in the MFMA fragment layout
        px4f, sx4f = bsp.bsp_mxfp4_quantize_frag(x5)

        def step4f(e=None):
            if e:
                e[0].record(stream)
            bsp.bsp_mxfp4_quantize_frag(x5, px4f, sx4f)
            if e:
                e[1].record(stream)
            bsp.bsp_mm_mxfp4_frag(px4f, sx4f, pw4f, sw4f, M, N1, out=out5)
            if e:
                e[2].record(stream)

        for _ in range(args.warmup):
            step4f()
        torch.cuda.synchronize()
        e4f = [[ev() for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            step4f(e4f[i])
        torch.cuda.synchronize()
        q4f = sum(e[0].elapsed_time(e[1]) for e in e4f) / args.steps
        g4f = sum(e[1].elapsed_time(e[2]) for e in e4f) / args.steps
        tf4f = 2.0 * M * N1 * K1 / g4f / 1e9
        qb4f = 2 * M * K1 + (-(-M // 32) * 32) * (K1 // 2 + K1 // 32)
        result["mxfp4_frag"] = {
            "mm_mxfp4_frag_ms": round(g4f, 4), "TFLOPS": round(tf4f, 2),
            "frac_fp4_peak": round(tf4f / PEAK_FP4_TFLOPS, 4),
            "quantize_frag_ms": round(q4f, 4), "quantize_GBs": round(qb4f / q4f / 1e6, 1),
            "quantize_frac_hbm": round(qb4f / q4f / 1e6 / PEAK_HBM_GBS, 4),
            "step_ms": round(q4f + g4f, 4), "step_ms_linear_layout": round(q4 + g4, 4)}
        log(json.dumps(result["mxfp4_frag"]))
        del px4f, sx4f, pw4f, sw4f, x52

    # ---- PyTorch's own memory-bound kernels on the same GPU, for context beside the published
    # 8 TB/s: a 2 GiB device-to-device copy (read:write 1:1) and a 2 GiB fp32 sum (read only), timed
    # with events on torch's stream. They are reference rates, not ceilings: the quantizers
    # (read:write about 3.6:1) run faster than both.
    nb = 1 << 31
    src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    red = src.view(torch.float32)

    def timed(fn, reps=10):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    copy_gbs = 2.0 * nb / timed(lambda: dst.copy_(src)) / 1e6
    read_gbs = 1.0 * nb / timed(lambda: red.sum()) / 1e6
    del src, dst, red
    result["torch_hbm_rates"] = {
        "copy_GBs": round(copy_gbs, 1), "sum_GBs": round(read_gbs, 1),
        "quantize_x_over_copy": round(kernels["quantize_x"]["GB/s"] / copy_gbs, 4),
        "quantize_h_over_copy": round(kernels["quantize_h"]["GB/s"] / copy_gbs, 4)}
    log(json.dumps(result["torch_hbm_rates"]))

    # ---- the other configurations' layer shapes (Wan-1.3B attention and FFN, Wan-14B to_q)
    if not args.no_shapes:
        result["shapes"] = measure_shapes(args.steps)
        log(json.dumps(result["shapes"]))

    # ---- measured-achievable ceilings on this GPU (MFMA-only loops, streaming kernels), and each
    # headline kernel's fraction of them
    if not args.no_ceilings:
        mp = measure_ceilings()
        result["measured_peak"] = mp
        f16 = mp["mfma_f16_nvfp4_operands_TFLOPS"]
        result["roofline"]["frac_of_measured_f16_mfma_loop"] = round(dom_tf / f16, 4)
        kernels_frac = {
            "mm_fp4_fc_in_of_f16_mfma_loop": kernels["mm_fp4_fc_in"]["TFLOPS"] / f16,
            "mm_fp4_fc_out_of_f16_mfma_loop": kernels["mm_fp4_fc_out"]["TFLOPS"] / f16,
            "mm_fp4_fc_in_row_major_of_f16_mfma_loop": kernels["mm_fp4_fc_in_row_major"]["TFLOPS"] / f16,
            "quantize_x_of_stream_4to1": kernels["quantize_x"]["GB/s"] / mp["hbm_read4_write1_GBs"],
            "quantize_x_in_step_of_stream_4to1": kernels["quantize_x_in_step"]["GB/s"] / mp["hbm_read4_write1_GBs"],
            "gelu_quantize_h_of_stream_4to1": kernels["gelu_quantize_h"]["GB/s"] / mp["hbm_read4_write1_GBs"],
            "quantize_h_of_stream_4to1": kernels["quantize_h"]["GB/s"] / mp["hbm_read4_write1_GBs"],
        }
        if "mxfp8" in result:
            kernels_frac["mm_mxfp8_of_fp8_mfma_loop"] = result["mxfp8"]["TFLOPS"] / mp["mfma_fp8_scaled_TFLOPS"]
        if "mxfp4" in result:
            kernels_frac["mm_mxfp4_of_fp4_mfma_loop"] = result["mxfp4"]["TFLOPS"] / mp["mfma_fp4_scaled_TFLOPS"]
        if "mxfp8_frag" in result:
            kernels_frac["mm_mxfp8_frag_of_fp8_mfma_loop"] = (result["mxfp8_frag"]["TFLOPS"]
                                                              / mp["mfma_fp8_scaled_TFLOPS"])
        if "mxfp4_frag" in result:
            kernels_frac["mm_mxfp4_frag_of_fp4_mfma_loop"] = (result["mxfp4_frag"]["TFLOPS"]
                                                              / mp["mfma_fp4_scaled_TFLOPS"])
        result["frac_of_measured_peak"] = {k_: round(v, 4) for k_, v in kernels_frac.items()}
        log(json.dumps(result["measured_peak"]), json.dumps(result["frac_of_measured_peak"]))

    # ---- CPU oracle on a bounded sample of the same workload
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_rows)
        r = result["cpu_baseline"]
        log(f"cpu baseline: {r['value']:.4f} {r['unit']} on {r['cores']} threads")

    print(json.dumps(result), flush=True)


def _event_ms(fns, reps: int) -> float:
    """Mean event time per call of fns (called in turn, each once untimed first) on torch's stream."""
    import torch
    for f in fns:
        f()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fns[i % len(fns)]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure_shapes(steps: int) -> dict:
    """The layer shapes of the Wan-1.3B attention projection (32760x1536x1536), the Wan-1.3B FFN
    (fc_in 32760x8960x1536, GELU fused into the quantize of H, fc_out 32760x1536x8960) and the
    Wan-14B to_q projection (32760x5120x5120): each GEMM and activation quantize timed on its own
    on the configuration's seeded inputs, weights prequantized first. Quantizes cycle over enough
    input and output copies that no buffer is reused within 768 MB of traffic."""
    import numpy as np
    import torch

    import block_scaled_precision_nvfp4_amd as bsp
    import workloads as W
    dev = torch.device("cuda:0")
    one = torch.ones(1, dtype=torch.float32, device=dev)
    reps = max(6, steps)

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    def qtime(x, gelu=False):
        m, k = x.shape
        per = 2 * m * k + m * k // 2
        n = max(2, -(-(768 << 20) // per))
        xs = [x] + [x.clone() for _ in range(n - 1)]
        outs = [(torch.empty((m, k // 2), dtype=torch.uint8, device=dev),
                 torch.empty(nvfp4_sf_shape(m, k), dtype=torch.uint8, device=dev)) for _ in range(n)]
        fn = bsp.bsp_nvfp4_quantize_gelu if gelu else bsp.bsp_nvfp4_quantize
        ms = _event_ms([lambda i=i: fn(xs[i], one, *outs[i]) for i in range(n)], max(reps, 2 * n))
        gbs = (2 * m * k + m * k // 2 + nvfp4_sf_shape(m, k)[0] * k // 16) / ms / 1e6
        return {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}

    def gtime(px, sx, pw, sw, alpha, out):
        m, n, k = px.shape[0], pw.shape[0], px.shape[1] * 2
        ms = _event_ms([lambda: bsp.bsp_mm_fp4(px, sx, pw, sw, alpha, out=out)], reps)
        tf = 2.0 * m * n * k / ms / 1e9
        return {"ms": round(ms, 4), "TFLOPS": round(tf, 2), "frac_fp4_peak": round(tf / PEAK_FP4_TFLOPS, 4),
                "frac_f16_mfma_peak": round(tf / PEAK_F16_TFLOPS, 4)}

    def gtime_frag(xq, wq, m, n, alpha, out):
        (pxf, sx), (pwf, sw) = xq, wq
        ms = _event_ms([lambda: bsp.bsp_mm_fp4_frag(pxf, sx, pwf, sw, m, n, alpha, out=out)], reps)
        tf = 2.0 * m * n * pxf.shape[1] * 64 / ms / 1e9
        return {"ms": round(ms, 4), "TFLOPS": round(tf, 2), "frac_fp4_peak": round(tf / PEAK_FP4_TFLOPS, 4),
                "frac_f16_mfma_peak": round(tf / PEAK_F16_TFLOPS, 4)}

    def weights(bits):
        w = up(bits)
        pw, sw, g, _, _ = bsp.bsp_nvfp4_prequantize_weight(w)
        return (pw, sw), bsp.bsp_nvfp4_quantize_frag(w, g), bsp.bsp_nvfp4_alpha(one, g)

    res = {}
    # Wan-1.3B attention projection
    c2 = W.config(2)
    x = up(W.generate(c2.tensor("X")))
    (pw, sw), wf, al = weights(W.generate(c2.tensor("W")))
    m = x.shape[0]
    res["wan1.3b_attn_quantize_x_32760x1536"] = qtime(x)
    px, sx = bsp.bsp_nvfp4_quantize(x, one)
    out = torch.empty((m, pw.shape[0]), dtype=torch.bfloat16, device=dev)
    res["wan1.3b_attn_mm_fp4_32760x1536x1536"] = gtime(px, sx, pw, sw, al, out)
    res["wan1.3b_attn_mm_fp4_frag_32760x1536x1536"] = gtime_frag(
        bsp.bsp_nvfp4_quantize_frag(x, one), wf, m, pw.shape[0], al, out)
    # Wan-1.3B FFN
    c3 = W.config(3)
    x = up(W.generate(c3.tensor("X")))
    (pw1, sw1), w1f, al1 = weights(W.generate(c3.tensor("W")))
    (pw2, sw2), w2f, al2 = weights(W.generate(c3.tensor("W2")))
    n1, n2 = pw1.shape[0], pw2.shape[0]
    res["wan1.3b_ffn_quantize_x_32760x1536"] = qtime(x)
    px, sx = bsp.bsp_nvfp4_quantize(x, one)
    y = torch.empty((m, n1), dtype=torch.bfloat16, device=dev)
    res["wan1.3b_ffn_mm_fp4_fc_in_32760x8960x1536"] = gtime(px, sx, pw1, sw1, al1, y)
    res["wan1.3b_ffn_mm_fp4_frag_fc_in_32760x8960x1536"] = gtime_frag(
        bsp.bsp_nvfp4_quantize_frag(x, one), w1f, m, n1, al1, y)
    res["wan1.3b_ffn_gelu_quantize_h_32760x8960"] = qtime(y, gelu=True)
    ph, sh = bsp.bsp_nvfp4_quantize_gelu(y, one)
    out = torch.empty((m, n2), dtype=torch.bfloat16, device=dev)
    res["wan1.3b_ffn_mm_fp4_fc_out_32760x1536x8960"] = gtime(ph, sh, pw2, sw2, al2, out)
    res["wan1.3b_ffn_mm_fp4_frag_fc_out_32760x1536x8960"] = gtime_frag(
        bsp.bsp_nvfp4_quantize_gelu_frag(y, one), w2f, m, n2, al2, out)
    del y, ph, sh, out
    # Wan-14B to_q
    c4 = W.config(4)
    x = up(W.generate(c4.tensor("X")))
    (pw, sw), wf, al = weights(W.generate(c4.tensor("W3")))
    px, sx = bsp.bsp_nvfp4_quantize(x, one)
    out = torch.empty((m, pw.shape[0]), dtype=torch.bfloat16, device=dev)
    res["wan14b_to_q_mm_fp4_32760x5120x5120"] = gtime(px, sx, pw, sw, al, out)
    res["wan14b_to_q_mm_fp4_frag_32760x5120x5120"] = gtime_frag(
        bsp.bsp_nvfp4_quantize_frag(x, one), wf, m, pw.shape[0], al, out)
    return res


def measure_ceilings() -> dict:
    """What this GPU sustains, measured with libbsp_probe: MFMA-only loops of each GEMM's matrix
    instruction on operands like its own (4 waves per SIMD, no memory traffic), and nontemporal
    streaming kernels over 2 GiB (read only, copy, and read:write 4:1 like the NVFP4 quantizers)."""
    import ctypes

    import torch
    here = os.path.join(ROOT, "block_scaled_precision_nvfp4_amd", "libbsp_probe.so")
    lib = ctypes.CDLL(here)
    lib.bsp_probe_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.bsp_probe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev).cuda_stream
    wgs = 1024
    sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    res = {}
    for fmt, name, iters, flops in ((0, "mfma_f16_nvfp4_operands_TFLOPS", 10000, 32768.0),
                                    (1, "mfma_fp8_scaled_TFLOPS", 5000, 131072.0),
                                    (2, "mfma_fp4_scaled_TFLOPS", 10000, 131072.0),
                                    (3, "mfma_fp8_scaled_16x16x128_TFLOPS", 10000, 65536.0)):
        def run(fmt=fmt, iters=iters):
            if lib.bsp_probe_mfma_loop(fmt, wgs, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st)) != 0:
                raise RuntimeError("bsp_probe_mfma_loop failed")
        ms = _event_ms([run], 3)
        res[name] = round(wgs * 4 * iters * 8 * flops / ms / 1e9, 1)
    nb = 1 << 31
    src = torch.ones(nb // 4, dtype=torch.int32, device=dev)
    dst = torch.empty(nb // 4, dtype=torch.int32, device=dev)
    for wd, name, nread, nwrite in ((0, "hbm_read_GBs", nb, 0), (1, "hbm_copy_GBs", nb // 2, nb // 2),
                                   (4, "hbm_read4_write1_GBs", nb, nb // 4)):
        def run(wd=wd, nread=nread):
            if lib.bsp_probe_stream(wd, ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                    nread // 16, 2048, ctypes.c_void_p(st)) != 0:
                raise RuntimeError("bsp_probe_stream failed")
        ms = _event_ms([run], 5)
        res[name] = round((nread + nwrite) / ms / 1e6, 1)
    del src, dst
    res["note"] = ("MFMA-only loops: 1024 workgroups x 4 waves, eight independent accumulator chains per "
                   "wave (one wave per SIMD, as in the GEMMs); streams: 2 GiB read, nontemporal, 16 loads "
                   "in flight per thread, 2048 workgroups")
    return res


def cpu_baseline(rows: int) -> dict:
    """The oracle (as it stands) runs the same FFN on the first `rows` tokens of X."""
    import numpy as np

    import workloads as W
    from oracle import activations as A
    from oracle import nvfp4 as N
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = os.cpu_count() or 1
    cfg = W.config(4)
    xb = W.generate(cfg.tensor("X"), rows=rows)
    w1 = W.generate(cfg.tensor("W"))
    w2 = W.generate(cfg.tensor("W2"))
    k1, n1, n2 = xb.shape[1], w1.shape[0], w2.shape[0]
    t0 = time.perf_counter()
    g1 = N.global_sf(w1)[0]
    g2 = N.global_sf(w2)[0]
    pw1, sw1 = N.quantize(w1, g1)
    pw2, sw2 = N.quantize(w2, g2)
    t_load = time.perf_counter() - t0
    ops = {}
    t_all = time.perf_counter()
    t0 = time.perf_counter()
    px, sx = N.quantize(xb, np.float32(1.0))
    ops["quantize_x_s"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    y = N.mm_fp4(px, sx, pw1, sw1, N.alpha(1.0, g1), rows, n1, k1)
    ops["mm_fp4_fc_in_s"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    yb = A.f64_to_bf16_bits(y)
    hb = A.gelu_tanh_bf16_bits(yb)
    ops["bf16_round_and_gelu_s"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    ph, sh = N.quantize(hb, np.float32(1.0))
    ops["quantize_h_s"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    _ = N.mm_fp4(ph, sh, pw2, sw2, N.alpha(1.0, g2), rows, n2, n1)
    ops["mm_fp4_fc_out_s"] = time.perf_counter() - t0
    dt = time.perf_counter() - t_all
    flops = 2.0 * rows * n1 * k1 + 2.0 * rows * n2 * n1
    qbytes_x = 2 * rows * k1 + rows * k1 // 2 + nvfp4_sf_shape(rows, k1)[0] * k1 // 16
    qbytes_h = 2 * rows * n1 + rows * n1 // 2 + nvfp4_sf_shape(rows, n1)[0] * n1 // 16
    rates = {"mm_fp4_fc_in_TFLOPS": 2.0 * rows * n1 * k1 / ops["mm_fp4_fc_in_s"] / 1e12,
             "mm_fp4_fc_out_TFLOPS": 2.0 * rows * n2 * n1 / ops["mm_fp4_fc_out_s"] / 1e12,
             "quantize_x_GBs": qbytes_x / ops["quantize_x_s"] / 1e9,
             "quantize_h_GBs": qbytes_h / ops["quantize_h_s"] / 1e9}
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOPS", "cores": int(blas_threads),
            "kind": "oracle", "seconds": round(dt, 2), "weight_prequant_seconds": round(t_load, 2),
            "per_op_seconds": {k: round(v, 3) for k, v in ops.items()},
            "per_op_rates": {k: round(v, 6) for k, v in rates.items()},
            "cpu_model": cpu_model, "blas_threads": int(blas_threads),
            "quantize_threads": 1,
            "host_cpus": os.cpu_count(),
            "sample": f"first {rows} of 32760 tokens through the same NVFP4 FFN (quantize X, fc_in, "
                      f"GELU, quantize H, fc_out) with the numpy oracle (fp64 GEMM of dequantized "
                      f"operands on the BLAS threads; the quantizes are single-threaded numpy); "
                      f"weight prequantization excluded"}


if __name__ == "__main__":
    main()
