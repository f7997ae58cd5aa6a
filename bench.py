#!/usr/bin/env python3
"""Benchmark of the NVFP4 prefill path on one MI355X.

One step = the W4A4 prefill of the four Qwen3-8B linear layers at 8192 tokens
(QKV 4096->6144, O 4096->4096, gate_up 4096->24576, down 12288->4096): for
each layer, the dynamic-alpha activation quantizer (amax pass + quantize
pass) followed by the NVFP4 GEMM with BF16 output.  Weights are quantized
once before timing (offline, as in a deployed prefill worker).  Three copies
of the activations and weights rotate from step to step, so no step finds
its operands in the 256 MB Infinity Cache.

The headline value is TFLOP/s including activation quantization:
sum(2*M*N*K) / (time of the four quantize+GEMM pairs).  Alongside it the
script times, outside the headline: the in-library BF16 GEMM at the same
shapes (speedup), the same comparison at 512 / 2048 / 32768 tokens, the fused
quantize-in-GEMM path, the NVFP4-output GEMM, the MXFP4 path, the BF16 and
NVFP4 decode GEMMs at batch 1/8/64 on the same weights, and the oracle on the
host cores on a bounded slice of the same workload.  Prints one JSON line.

--workload selects other prefill shapes for the same measurement: Qwen3-8B
at 32768 tokens with Student-t(4) activations, or Qwen3-32B at 16384 tokens.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP4_PEAK_TFLOPS = 10100.0   # MI355X dense FP4/FP6 MFMA
F16_PEAK_TFLOPS = 2500.0    # MI355X dense FP16/BF16 MFMA
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
ROT = 3                     # rotated input sets of the prefill step
METRIC = "NVFP4 prefill GEMM TFLOPS (incl. act quant), % FP4 MFMA peak, speedup vs BF16"
EXTRAS = ("bf16", "sweep", "fused", "quant_out", "mxfp4", "decode")
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "nvfp4_gemm_qwen3_8b_m8192_gate_up_counters.md")
# the tile GEMM's sources: a counter summary describes the kernel built from these
GEMM_SOURCES = ("gemm.hip", "nvfp4_device.hpp", "epilogue.hpp", "tiling.hpp")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    p.add_argument("--no-extras", action="store_true", help="only the headline NVFP4 prefill timing")
    p.add_argument("--extras", default=",".join(EXTRAS),
                   help="comma-separated subset of the timings beside the headline: " + ", ".join(EXTRAS))
    p.add_argument("--workload", default="qwen3_8b_m8192",
                   choices=["qwen3_8b_m8192", "qwen3_8b_m32768_t4", "qwen3_32b_m16384"],
                   help="prefill linears to time (default: Qwen3-8B at 8192 tokens, the headline)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target duration of the oracle leg")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one plain 1 GiB device copy (reference kernel for HBM byte counters)")
    return p.parse_args()


def _bf16_tensor(bits):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "nvfp4_prefill_gemm_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic_from_profile():
    """HBM bytes per gate_up GEMM launch from the committed counter summary, if
    it was taken on the current kernel source (else None)."""
    try:
        txt = open(PROFILE_COUNTERS).read()
    except OSError:
        return None
    vals = {}
    for line in txt.splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("gemm_source_sha256_16") != _source_hash(*GEMM_SOURCES):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events on torch's current stream (the stream every entry point is given)."""

    def __init__(self):
        import torch

        self.torch = torch
        self.pairs = {}

    def span(self, key):
        torch = self.torch
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        self.pairs.setdefault(key, []).append((s, e))
        return s, e

    def total_ms(self, key):
        return sum(s.elapsed_time(e) for s, e in self.pairs.get(key, []))

    def count(self, key):
        return len(self.pairs.get(key, []))

    def median_ms(self, key):
        v = sorted(s.elapsed_time(e) for s, e in self.pairs.get(key, []))
        return (v[(len(v) - 1) // 2] + v[len(v) // 2]) / 2 if v else float("nan")


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the NVFP4 prefill path here has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from nvfp4_prefill_gemm_amd import binding as nv
    from nvfp4_prefill_gemm_amd import workloads as wl

    nv.lib()  # fails loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda", 0)
    w = wl.WORKLOADS[args.workload]
    headline = args.workload == "qwen3_8b_m8192"
    M = w.M
    t_setup = time.time()

    # ---------------------------------------------------------------- inputs
    layers = []
    for li, (name, K, N) in enumerate(w.linears):
        a_bits, w_bits = wl.layer_inputs(w, li)
        x = _bf16_tensor(a_bits)
        wb = _bf16_tensor(w_bits)
        wc, ws, wa = nv.nvfp4_quantize(wb)  # offline weight quantization (untimed)
        layers.append(dict(
            name=name, K=K, N=N, x=x, w_bf16=wb, wc=wc, ws=ws, wa=wa,
            ac=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
            asc=torch.empty((M, K // 16), dtype=torch.uint8, device=dev),
            aal=torch.empty(1, dtype=torch.float32, device=dev),
            ws_buf=torch.empty(max(nv.quantize_workspace_size(M, K), 4), dtype=torch.uint8, device=dev),
            y=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
        del a_bits, w_bits
    # Input sets rotated from step to step (copies of the activations and of
    # both weight forms): consecutive steps never find their operands in the
    # 256 MB Infinity Cache (three sets of the Qwen3-8B layers at 8192 tokens
    # hold 2.6 GB).  Quantizer outputs and GEMM outputs are shared.
    sets = [layers] + [[dict(L, x=L["x"].clone(), w_bf16=L["w_bf16"].clone(), wc=L["wc"].clone(),
                             ws=L["ws"].clone()) for L in layers] for _ in range(ROT - 1)]
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    print(f"bench: {w.name} inputs ready in {setup_s:.1f} s", file=sys.stderr, flush=True)
    flops_step = sum(wl.flops(M, L["N"], L["K"]) for L in layers)

    # ------------------------------------------------------- headline: NVFP4
    def nvfp4_step(i, timer=None):
        for L in sets[i % ROT]:
            if timer:
                sq, eq = timer.span(("quant", L["name"]))
                sq.record()
            nv.nvfp4_quantize(L["x"], L["ac"], L["asc"], L["aal"], workspace=L["ws_buf"])
            if timer:
                eq.record()
                sg, eg = timer.span(("gemm", L["name"]))
                sg.record()
            nv.nvfp4_gemm(L["ac"], L["asc"], L["aal"], L["wc"], L["ws"], L["wa"], out=L["y"])
            if timer:
                eg.record()

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        nvfp4_step(i)
    torch.cuda.synchronize()
    timer = Timer()
    t0 = time.perf_counter()
    s_all, e_all = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_all.record()
    for i in range(args.steps):
        ss, es = timer.span("step")
        ss.record()
        nvfp4_step(i, timer)
        es.record()
    e_all.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    step_ms = s_all.elapsed_time(e_all) / args.steps
    step_median_ms = timer.median_ms("step")
    per_layer = {}
    for L in layers:
        q = timer.total_ms(("quant", L["name"])) / args.steps
        g = timer.total_ms(("gemm", L["name"])) / args.steps
        per_layer[L["name"]] = dict(M=M, N=L["N"], K=L["K"], quant_us=round(q * 1e3, 2), gemm_us=round(g * 1e3, 2),
                                    gemm_tflops=round(wl.flops(M, L["N"], L["K"]) / (g * 1e-3) / 1e12, 1),
                                    quant_gbps=round(M * L["K"] * 4.5625 / (q * 1e-3) / 1e9, 1))
    kern_ms = sum(v["quant_us"] + v["gemm_us"] for v in per_layer.values()) / 1e3
    value = flops_step / (step_ms * 1e-3) / 1e12
    gemm_ms_total = sum(v["gemm_us"] for v in per_layer.values()) / 1e3
    quant_ms_total = sum(v["quant_us"] for v in per_layer.values()) / 1e3
    quant_bytes = sum(M * L["K"] * 4.5625 for L in layers)

    # practical HBM yardstick for the quantizer: a plain 1 GiB device copy
    # (reads 1 GiB, writes 1 GiB; larger than the 256 MB Infinity Cache)
    csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    torch.cuda.synchronize()
    cs_, ce_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cs_.record()
    for _ in range(5):
        cdst.copy_(csrc)
    ce_.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 5 / (cs_.elapsed_time(ce_) * 1e-3) / 1e9
    del csrc, cdst

    # dominant kernel: the gate_up NVFP4 GEMM launch
    gu = per_layer["gate_up"]
    gu_flops = wl.flops(M, gu["N"], gu["K"])
    gu_tflops = gu_flops / (gu["gemm_us"] * 1e-6) / 1e12
    roofline = {"bound": "mfma", "achieved": round(gu_tflops, 1), "peak": F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gu_tflops / F16_PEAK_TFLOPS, 4),
                "traffic": _traffic_from_profile() if headline else None,
                "kernel": f"gemm_kernel<NVFP4> gate_up {M}x{gu['N']}x{gu['K']} (FP16 MFMA on exact q*sigma)",
                "frac_of_fp4_peak": round(gu_tflops / FP4_PEAK_TFLOPS, 4)}

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "ms_per_step_median": round(step_median_ms, 4),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": w.name, "M": M, "linears": [[n, k, nn] for n, k, nn in w.linears],
                   "activations": ("Student-t(nu=4), BF16" if w.act_dist == "student_t4"
                                   else "N(0,1) with 0.5% channels x20, BF16"),
                   "weights": "N(0,0.02) BF16 -> NVFP4 offline",
                   "alpha": "dynamic", "out_dtype": "bf16", "storage": "nvfp4 (e2m1 codes + e4m3 per 16 + fp32)",
                   "input_sets": f"{ROT}, rotated per step (activations and weights)"},
        "frac_fp4_peak": round(value / FP4_PEAK_TFLOPS, 4),
        "frac_f16_mfma_peak": round(value / F16_PEAK_TFLOPS, 4),
        "gemm_only_tflops": round(flops_step / (gemm_ms_total * 1e-3) / 1e12, 2),
        "quantizer_gbps": round(quant_bytes / (quant_ms_total * 1e-3) / 1e9, 1),
        "hbm_copy_gbps": round(copy_gbps, 1),
        "quantizer_frac_of_copy": round(quant_bytes / (quant_ms_total * 1e-3) / 1e9 / copy_gbps, 3),
        "per_layer": per_layer,
        "wall_ms_per_step": round(wall_ms / args.steps, 4),
        "kernel_ms_per_step": round(kern_ms, 4),
        "roofline": roofline,
        "setup_s": round(setup_s, 1),
    }

    print(f"bench: headline {value:.1f} TFLOP/s", file=sys.stderr, flush=True)
    parts = set() if args.no_extras else {x.strip() for x in args.extras.split(",") if x.strip()}
    if parts - set(EXTRAS):
        print(f"bench.py: unknown --extras {sorted(parts - set(EXTRAS))}", file=sys.stderr)
        return 2
    if parts:
        result.update(extras(args, nv, wl, layers, sets, M, flops_step, step_ms, parts, sweep=headline))
        print("bench: extras done", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, wl, w)
    print(json.dumps(result), flush=True)
    return 0


def extras(args, nv, wl, layers, sets, M, flops_step, nvfp4_step_ms, parts, sweep=False):
    import torch

    dev = torch.device("cuda", 0)
    out = {}
    reps = max(3, min(args.steps, 20) // 2)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    bf16_ms = None
    if "bf16" in parts:
        bf16_ms = _bf16_prefill(nv, sets, reps, s, e)
        out["bf16_tflops"] = round(flops_step / (bf16_ms * 1e-3) / 1e12, 2)
        out["speedup_vs_bf16"] = round(bf16_ms / nvfp4_step_ms, 3)
    if sweep and "sweep" in parts:
        out["prefill_sweep"] = _phase_split_sweep(nv, wl, layers, sets, M, reps, s, e, nvfp4_step_ms, bf16_ms)
    if "fused" in parts:
        out.update(_fused(nv, layers, sets, M, flops_step, reps, s, e))
    if "quant_out" in parts:
        out.update(_quant_out(nv, layers, M, flops_step, reps, s, e))
    if "mxfp4" in parts:
        out.update(_mxfp4(nv, wl, layers, M, flops_step, reps, s, e, bf16_ms))
    if "decode" in parts:
        out.update(_decode(nv, wl, layers, s, e))
    return out


def _bf16_prefill(nv, sets, reps, s, e):
    import torch

    # BF16 prefill GEMMs at the same shapes (the speedup denominator), on the
    # same rotated input sets as the NVFP4 steps
    def bf16_step(i):
        for L in sets[i % ROT]:
            nv.bf16_gemm(L["x"], L["w_bf16"], out=L["y"])
    for i in range(ROT):
        bf16_step(i)
    torch.cuda.synchronize()
    s.record()
    for i in range(reps):
        bf16_step(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def _phase_split_sweep(nv, wl, layers, sets, M, reps, s, e, nvfp4_step_ms, bf16_ms):
    """NVFP4 prefill (dynamic-alpha quantizer + GEMM, BF16 out) against the
    BF16 GEMM at other token counts, same weights; the activations are the
    first rows of the headline ones, or those rows repeated."""
    import torch

    dev = torch.device("cuda", 0)

    def timed_ms(step):
        for i in range(ROT):
            step(i)
        torch.cuda.synchronize()
        s.record()
        for i in range(reps):
            step(i)
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    sw = {}
    for Ms in wl.PHASE_SPLIT_PREFILL_M:
        fl = sum(wl.flops(Ms, L["N"], L["K"]) for L in layers)
        if Ms == M and bf16_ms is not None:
            t4, t16 = nvfp4_step_ms, bf16_ms
        else:
            if Ms > M and Ms % M:
                continue
            bufs = []
            for L in layers:
                x = (L["x"][:Ms] if Ms <= M else L["x"].repeat(Ms // M, 1)).contiguous()
                bufs.append(dict(x=x, ac=torch.empty((Ms, L["K"] // 2), dtype=torch.uint8, device=dev),
                                 asc=torch.empty((Ms, L["K"] // 16), dtype=torch.uint8, device=dev),
                                 aal=torch.empty(1, dtype=torch.float32, device=dev),
                                 wsb=torch.empty(max(nv.quantize_workspace_size(Ms, L["K"]), 4),
                                                 dtype=torch.uint8, device=dev),
                                 y=torch.empty((Ms, L["N"]), dtype=torch.bfloat16, device=dev)))

            # the weights rotate over the same copies as in the headline
            # step (three sets: the NVFP4 weights of one set would
            # otherwise stay in the Infinity Cache from rep to rep)
            def nv_step(i):
                for L, B in zip(sets[i % ROT], bufs):
                    nv.nvfp4_quantize(B["x"], B["ac"], B["asc"], B["aal"], workspace=B["wsb"])
                    nv.nvfp4_gemm(B["ac"], B["asc"], B["aal"], L["wc"], L["ws"], L["wa"], out=B["y"],
                                  workspace=False)

            def bf_step(i):
                for L, B in zip(sets[i % ROT], bufs):
                    nv.bf16_gemm(B["x"], L["w_bf16"], out=B["y"], workspace=False)
            t4, t16 = timed_ms(nv_step), timed_ms(bf_step)
            del bufs
        sw[str(Ms)] = {"nvfp4_tflops": round(fl / (t4 * 1e-3) / 1e12, 1),
                       "bf16_tflops": round(fl / (t16 * 1e-3) / 1e12, 1), "speedup_vs_bf16": round(t16 / t4, 3)}
    return sw


def _fused(nv, layers, sets, M, flops_step, reps, s, e):
    import torch

    dev = torch.device("cuda", 0)
    out = {}

    # nvfp4_quant_gemm (BF16 activations in, dynamic alpha), on the same
    # rotated sets: with its full workspace it quantizes once into the
    # workspace and runs the NVFP4 GEMM; with only the amax partials' workspace
    # the tile kernel quantizes in its operand staging (every column tile
    # again), reported as fused_prologue_tflops
    qg_ws = [torch.empty(nv.quant_gemm_workspace_size(M, L["N"], L["K"]), dtype=torch.uint8, device=dev)
             for L in layers]

    def fused_step(i, full=True):
        for j, L in enumerate(sets[i % ROT]):
            nv.nvfp4_quant_gemm(L["x"], L["wc"], L["ws"], L["wa"], a_alpha=L["aal"], out=L["y"],
                                workspace=qg_ws[j] if full else L["ws_buf"])

    def fused_ms_of(full):
        for i in range(ROT):
            fused_step(i, full)
        torch.cuda.synchronize()
        s.record()
        for i in range(reps):
            fused_step(i, full)
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps
    out["fused_tflops"] = round(flops_step / (fused_ms_of(True) * 1e-3) / 1e12, 2)
    out["fused_prologue_tflops"] = round(flops_step / (fused_ms_of(False) * 1e-3) / 1e12, 2)
    del qg_ws
    return out


def _quant_out(nv, layers, M, flops_step, reps, s, e):
    """NVFP4 GEMM whose epilogue quantizes Y to NVFP4 for the next layer
    (static output scale), and the same with a dynamic output scale; same
    layers and activations."""
    import torch

    dev = torch.device("cuda", 0)
    out = {}
    yq = [(torch.empty((M, L["N"] // 2), dtype=torch.uint8, device=dev),
           torch.empty((M, L["N"] // 16), dtype=torch.uint8, device=dev)) for L in layers]
    y_alpha = torch.tensor([0.02], dtype=torch.float32, device=dev)

    def qo_step():
        for L, (yc, ysc) in zip(layers, yq):
            nv.nvfp4_gemm_quant_out(L["ac"], L["asc"], L["aal"], L["wc"], L["ws"], L["wa"], y_alpha, yc, ysc)
    for _ in range(2):
        qo_step()
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        qo_step()
    e.record()
    torch.cuda.synchronize()
    out["quant_out_gemm_tflops"] = round(flops_step / (s.elapsed_time(e) / reps * 1e-3) / 1e12, 2)
    # the same with the output tensor scale from Y's own amax (FP32 Y through
    # a workspace, then the FP32 quantizer)
    ya = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(max(nv.gemm_quant_out_dynamic_workspace_size(M, L["N"], L["K"]) for L in layers),
                     dtype=torch.uint8, device=dev)

    def qd_step():
        for L, (yc, ysc) in zip(layers, yq):
            nv.nvfp4_gemm_quant_out_dynamic(L["ac"], L["asc"], L["aal"], L["wc"], L["ws"], L["wa"], yc, ysc, ya, ws)
    for _ in range(2):
        qd_step()
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        qd_step()
    e.record()
    torch.cuda.synchronize()
    out["quant_out_dynamic_gemm_tflops"] = round(flops_step / (s.elapsed_time(e) / reps * 1e-3) / 1e12, 2)
    del yq, ws
    return out


def _mxfp4(nv, wl, layers, M, flops_step, reps, s, e, bf16_ms):
    """MXFP4 (E2M1 + E8M0 per 32) prefill of the same layers on the
    block-scaled FP4 MFMA: activation quantizer + GEMM, weights quantized once."""
    import torch

    dev = torch.device("cuda", 0)
    out = {}
    mx = []
    for L in layers:
        wc, ws = nv.mxfp4_quantize(L["w_bf16"])
        mx.append((torch.empty((M, L["K"] // 2), dtype=torch.uint8, device=dev),
                   torch.empty((M, L["K"] // 32), dtype=torch.uint8, device=dev), wc, ws))

    def mx_step(timer=None):
        for L, (ac, asc, wc, ws) in zip(layers, mx):
            nv.mxfp4_quantize(L["x"], ac, asc)
            if timer:
                sg, eg = timer.span(("mxgemm", L["name"]))
                sg.record()
            nv.mxfp4_gemm(ac, asc, wc, ws, out=L["y"])
            if timer:
                eg.record()
    for _ in range(2):
        mx_step()
    torch.cuda.synchronize()
    mt = Timer()
    s.record()
    for _ in range(reps):
        mx_step(mt)
    e.record()
    torch.cuda.synchronize()
    mx_ms = s.elapsed_time(e) / reps
    out["mxfp4_prefill_tflops"] = round(flops_step / (mx_ms * 1e-3) / 1e12, 2)
    out["mxfp4_frac_fp4_peak"] = round(flops_step / (mx_ms * 1e-3) / 1e12 / FP4_PEAK_TFLOPS, 4)
    if bf16_ms is not None:
        out["mxfp4_speedup_vs_bf16"] = round(bf16_ms / mx_ms, 3)
    out["mxfp4_gemm_tflops"] = {L["name"]: round(wl.flops(M, L["N"], L["K"]) / (mt.total_ms(("mxgemm", L["name"])) / reps
                                                                              * 1e-3) / 1e12, 1) for L in layers}
    return out


def _decode(nv, wl, layers, s, e):
    import torch

    dev = torch.device("cuda", 0)
    out = {}
    # Decode steps (one token batch through the four layers) are replayed from
    # HIP graphs, as a serving loop runs them: per-call host overhead would
    # otherwise exceed these kernels' GPU time.  Weights rotate over copies
    # that together exceed the 256 MB Infinity Cache.
    def graph_us(step, copies, n):
        graphs = []
        for c in range(copies):
            step(c)  # warm-up: first-launch attribute setup stays out of the graph
        torch.cuda.synchronize()
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        s.record()
        for r in range(n):
            graphs[r % copies].replay()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / n * 1e3

    # BF16 decode GEMMs (the method's decode precision): two weight copies,
    # decode-packed (bf16_decode_pack, once at load); the row-major weights'
    # step is timed beside it
    copies = [[L["w_bf16"] for L in layers], [L["w_bf16"].clone() for L in layers]]
    packed = [[nv.bf16_decode_pack(w) for w in cp] for cp in copies]
    decode = {}
    for Md in wl.PHASE_SPLIT_DECODE_M:
        xs = [torch.randn((Md, L["K"]), device=dev).to(torch.bfloat16) for L in layers]
        ys = [torch.empty((Md, L["N"]), dtype=torch.bfloat16, device=dev) for L in layers]
        wsd = [torch.empty(max(nv.bf16_gemm_workspace_size(Md, L["N"], L["K"]), 16), dtype=torch.uint8, device=dev)
               for L in layers]

        def dec_step(c):
            for i, L in enumerate(layers):
                nv.bf16_gemm_packed(xs[i], packed[c][i], out=ys[i], workspace=wsd[i])

        def dec_step_row_major(c):
            for i, L in enumerate(layers):
                nv.bf16_gemm(xs[i], copies[c][i], out=ys[i], workspace=wsd[i])
        us = graph_us(dec_step, 2, 20)
        us_rm = graph_us(dec_step_row_major, 2, 20)
        nbytes = sum(2 * L["N"] * L["K"] + 2 * Md * L["K"] + 2 * Md * L["N"] for L in layers)
        decode[str(Md)] = {"us_per_step": round(us, 1), "hbm_gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                           "frac_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 3),
                           "weights": "decode-packed", "row_major_us_per_step": round(us_rm, 1)}
    out["decode_bf16"] = decode
    del copies, packed

    # NVFP4 x NVFP4 decode (the uniform-NVFP4 / FP4-decode ablation variants):
    # dynamic-alpha activation quantizer + decode GEMM per layer; a step's
    # NVFP4 weights (109 MB) fit the Infinity Cache, so four copies rotate.
    # The step runs on decode-packed weights (nvfp4_decode_pack, packed once
    # like the offline quantization); the row-major weights' step is timed
    # beside it.
    wq = [[(L["wc"], L["ws"], L["wa"]) for L in layers]]
    for _ in range(3):
        wq.append([(L["wc"].clone(), L["ws"].clone(), L["wa"]) for L in layers])
    wpk = [[nv.nvfp4_decode_pack(*w) for w in cp] for cp in wq]
    dec4 = {}
    for Md in wl.PHASE_SPLIT_DECODE_M:
        xs = [torch.randn((Md, L["K"]), device=dev).to(torch.bfloat16) for L in layers]
        ys = [torch.empty((Md, L["N"]), dtype=torch.bfloat16, device=dev) for L in layers]
        # one nvfp4_quant_gemm per layer: BF16 activations in, dynamic alpha;
        # the library quantizes the batch inside the decode kernel (small
        # batches) or into the workspace before it
        qa = [(torch.empty(1, dtype=torch.float32, device=dev),
               torch.empty(max(nv.quant_gemm_workspace_size(Md, L["N"], L["K"]), 16), dtype=torch.uint8,
                           device=dev)) for L in layers]
        # the library's route (include/nvfp4.h, nvfp4_quant_gemm): which layers quantize in the decode kernel
        fused = [L["K"] % 32 == 0 and Md * L["K"] <= 196608 and
                 (Md <= 2 or (Md <= 6 and L["N"] <= 8192 and Md * L["K"] <= 32768)) for L in layers]

        def dec4_step(c):
            for i, L in enumerate(layers):
                aal, wsb = qa[i]
                nv.nvfp4_quant_gemm_packed(xs[i], wpk[c][i], a_alpha=aal, out=ys[i], workspace=wsb)

        def dec4_step_row_major(c):
            for i, L in enumerate(layers):
                aal, wsb = qa[i]
                nv.nvfp4_quant_gemm(xs[i], *wq[c][i], a_alpha=aal, out=ys[i], workspace=wsb)
        us = graph_us(dec4_step, 4, 20)
        us_rm = graph_us(dec4_step_row_major, 4, 20)
        nbytes = sum(L["N"] * L["K"] * 9 // 16 + 2 * Md * L["K"] + Md * L["K"] * 9 // 16 + 2 * Md * L["N"]
                     for L in layers)
        dec4[str(Md)] = {"us_per_step": round(us, 1), "hbm_gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                         "frac_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 3),
                         "speedup_vs_bf16_decode": round(decode[str(Md)]["us_per_step"] / us, 3),
                         "weights": "decode-packed", "row_major_us_per_step": round(us_rm, 1),
                         "fused_layers": [L["name"] for L, f in zip(layers, fused) if f]}
    out["decode_nvfp4"] = dec4
    del wq, wpk
    return out


def cpu_baseline(args, wl, w):
    """The oracle (plain C, threads over rows) on the host cores: activation
    quantization plus exact GEMM for a slab of rows of every layer, scaled to
    TFLOP/s.  Weights are quantized outside the timed region, as on the GPU."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    wq = []
    for li, (name, K, N) in enumerate(w.linears):
        wb = wl.weights(N, K, wl.rng(w.config_id, li, 1))
        wq.append(oracle.quantize(wb, nthreads=threads))

    # time only quantize + GEMM (input generation excluded)
    def timed(rows):
        flops, spent = 0, 0.0
        for li, (name, K, N) in enumerate(w.linears):
            a = wl.activations(rows, K, wl.rng(w.config_id, li, 0))
            ta = time.perf_counter()
            A = oracle.quantize(a, nthreads=threads)
            oracle.gemm_exact(*A, *wq[li], nthreads=threads)
            spent += time.perf_counter() - ta
            flops += wl.flops(rows, N, K)
        return flops, spent

    # grow the slab until the timed work reaches about half the target (the
    # first, smallest pass also absorbs one-time costs such as page faults)
    rows = max(threads, 16)
    flops, spent = timed(rows)
    for _ in range(3):
        if spent >= args.cpu_seconds / 2 or rows >= w.M:
            break
        rows = int(min(w.M, max(rows * 2, rows * args.cpu_seconds / max(spent, 1e-3))))
        rows = max(threads, (rows // threads) * threads)
        flops, spent = timed(rows)
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} of {w.M} token rows of each of the 4 Qwen3-8B linears: oracle quantize "
                      f"(dynamic alpha over the slab) + exact int64 GEMM against the full NVFP4 weights; "
                      f"{spent:.1f} s", "seconds": round(spent, 2)}


if __name__ == "__main__":
    sys.exit(main())
