"""Benchmark of the fused weight-gradient GEMM + optimizer step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload mlp_down] [--no-cpu]

One step = one fused call over one batch of seeded synthetic input already
resident in HBM: dW = X^T dY (bf16 in, fp32 accumulate, all tokens) consumed by
AdamW in the epilogue, W/m/v updated in place. The default workload is a
Llama-3-8B MLP down projection (X [8192, 14336], dY [8192, 4096], fp32 W/m/v
[4096, 14336]). The unfused pair (fp32 gradient stored, then elementwise AdamW)
is timed beside it, then (dense AdamW workloads) three precision variants: fused
AdamW with bf16 moments, and the bf16-rounded gradient stored and followed by
elementwise AdamW, and fused AdamW from fp8 inputs; the layer's input gradient
dX = dY W and the whole backward (dX from the weight before the step, then the
fused step), each from the float32 weight and from the bf16 copy the fused step
refreshes; and the CPU oracle on a bounded sample.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_FP8_TFLOPS = 5033.2       # dense fp8 MFMA, twice the bf16 rate
PEAK_HBM_GBS = 8000.0
METRIC = "fused dW-GEMM+AdamW TFLOP/s & ms/step, MFMA util %, HBM bytes vs unfused"

WORKLOADS = {
    # name: (config index, optimizer)
    "tiny": (0, "adamw"),
    "mlp_down": (1, "adamw"),
    "qkv": (2, "adamw"),
    "qkv_sgdm": (2, "sgdm"),
    "lm_head": (3, "adamw"),
    "moe": (4, "adamw"),
}
KERNEL_SOURCES = ("wgrad_kernels.hpp", "elementwise_kernels.hpp", "optim_math.hpp", "forge.hip",
                  "host.hpp", "host.hip", "fp8_kernels.hpp", "forge_fp8.hip", "dgrad_kernels.hpp",
                  "forge_dgrad.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """Hash of the kernel sources' code: comments, trailing blanks and empty
    lines are dropped, so only a change to the code itself invalidates the
    committed counter summaries."""
    h = hashlib.sha256()
    for fn in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "weight_gradient_gemm_amd", "csrc", fn)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str, sha: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"pmc_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        text = f.read()
    m_sha = re.search(r"^kernel_source_sha:\s*(\w+)", text, re.M)
    m_b = re.search(r"^fused_hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not (m_sha and m_b) or m_sha.group(1) != sha:
        return None
    return float(m_b.group(1))


def read_counters(workload: str, sha: str, n_param: int):
    """The rest of the committed counter summaries for the fused kernel, where
    they were taken on the current kernel sources: HBM bytes written per
    parameter (the optimizer state only, if the gradient never reaches HBM),
    the unfused pair's bytes per step, and the matrix cores' busy fraction."""
    out = {}
    path = os.path.join(ROOT, "profiles", f"pmc_{workload}.txt")
    if os.path.exists(path):
        with open(path) as f:
            text = f.read()
        m_sha = re.search(r"^kernel_source_sha:\s*(\w+)", text, re.M)
        m_w = re.search(r"^fused_write_bytes:\s*([0-9.eE+]+)", text, re.M)
        m_u = re.search(r"^unfused_pair_hbm_bytes_per_step:\s*([0-9.eE+]+)", text, re.M)
        if m_sha and m_sha.group(1) == sha:
            if m_w:
                out["fused_write_bytes_per_param"] = round(float(m_w.group(1)) / n_param, 3)
            if m_u:
                out["unfused_pair_hbm_bytes"] = float(m_u.group(1))
    path = os.path.join(ROOT, "profiles", f"pmc_mfma_{workload}.txt")
    if os.path.exists(path):
        with open(path) as f:
            text = f.read()
        m_sha = re.search(r"^kernel_source_sha:\s*(\w+)", text, re.M)
        # the plain fused kernel's row: | fused AdamW (persistent) [epi 0] | dispatches | busy |
        # cycles per XCD | mean us | clock GHz | ...
        m_b = re.search(r"^\| fused (?:AdamW|SGD-m) \(\w+\) \[epi \d+\] \|\s*\d+\s*\|"
                        r"\s*([0-9.]+)\s*\|(?:\s*[0-9.eE+]+\s*\|\s*[0-9.]+\s*\|\s*([0-9.]+)\s*\|)?",
                        text, re.M)
        if m_sha and m_sha.group(1) == sha and m_b:
            # busy cycles over the kernel's cycles at the clock it ran in the
            # profiled run (the board holds it at its power limit); the bench's
            # roofline fraction stays against the published peak
            out["mfma_busy_fraction"] = float(m_b.group(1))
            if m_b.group(2):
                out["profiled_clock_ghz"] = float(m_b.group(2))
    if out:
        out["from"] = f"profiles/pmc_{workload}.txt, pmc_mfma_{workload}.txt (committed)"
    return out or None


def with_tokens(case, tokens: int):
    """The dense workload `case` with `tokens` rows of X and dY (same layer,
    same seeds and distributions); its name carries the new count."""
    name = re.sub(r"_T\d+$", "", case.name) + f"_T{tokens}"
    return dataclasses.replace(case, T=int(tokens), name=name)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mlp_down", choices=sorted(WORKLOADS))
    ap.add_argument("--tile", type=int, default=0)
    ap.add_argument("--pool", type=int, default=2, help="distinct input batches cycled")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="untimed fused steps for at least this long before the warm-up steps "
                         "(the clock ramps for ~0.2 s after an idle period)")
    ap.add_argument("--leg-settle-s", type=float, default=0.1,
                    help="untimed steps of each comparison leg (unfused pair, precision "
                         "variants, backward) for at least this long before its warm-up steps "
                         "(the clock moves when the load changes kind)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the precision-variant legs (dense AdamW workloads)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the input-gradient and whole-backward legs (dense AdamW)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="dense workloads: run the layer with this many tokens instead of "
                         "the workload's own (a token-count sweep; not the headline line)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the fused step needs no collective and no multi-GPU "
              "path exists (run it with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import weight_gradient_gemm_amd as wg

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    k, opt = WORKLOADS[args.workload]
    case = synth.CONFIGS[k]
    grouped = isinstance(case, synth.GroupedCase)
    if args.tokens:
        if grouped or args.tokens < 1:
            print("--tokens takes a positive count and applies to dense workloads only",
                  file=sys.stderr)
            sys.exit(2)
        case = with_tokens(case, args.tokens)

    def up_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
            torch.bfloat16)

    log(f"[bench] workload {args.workload}: {case}")
    t0 = time.perf_counter()
    batches = []
    for s in range(1, args.pool + 1):
        if grouped:
            Xp, Yp, offs = synth.grouped_inputs(case, s)
            batches.append((up_bf16(Xp), up_bf16(Yp), [int(x) for x in offs], (Xp, Yp, offs)))
        else:
            Xb, Yb = synth.dense_inputs(case, s)
            batches.append((up_bf16(Xb), up_bf16(Yb), None, (Xb, Yb, None)))
        log(f"[bench] batch {s} ready ({time.perf_counter() - t0:.1f}s)")
    W0, m0, v0 = synth.grouped_state(case) if grouped else synth.dense_state(case)
    W = torch.from_numpy(W0).to(dev)
    m = torch.from_numpy(m0).to(dev)
    v = torch.from_numpy(v0).to(dev)
    if grouped:
        rows = int(batches[0][2][-1])
        flops = 2 * rows * case.d_in * case.d_out
        n_param = case.E * case.d_in * case.d_out
        x_bytes = 2 * rows * (case.d_in + case.d_out)
    else:
        flops = 2 * case.T * case.d_in * case.d_out
        n_param = case.d_in * case.d_out
        x_bytes = 2 * case.T * (case.d_in + case.d_out)
    state_bytes = (24 if opt == "adamw" else 16) * n_param
    alg_bytes = x_bytes + state_bytes
    hp = dict(lr=case.lr, weight_decay=case.weight_decay)
    if opt == "adamw":
        hp.update(beta1=case.beta1, beta2=case.beta2, eps=case.eps)
    else:
        hp.update(momentum=case.momentum)
        hp["weight_decay"] = 0.0

    def fused(step, batch):
        X, dY, offs, _ = batch
        if grouped:
            wg.forge_grouped_wgrad_adamw(X, dY, offs, W, m, v, step=step, tile=args.tile, **hp)
        elif opt == "adamw":
            wg.forge_wgrad_adamw(X, dY, W, m, v, step=step, tile=args.tile, **hp)
        else:
            wg.forge_wgrad_sgdm(X, dY, W, m, tile=args.tile, **hp)

    stream = torch.cuda.current_stream()

    def timed(fn, steps, warmup, settle_s=0.0):
        n, t_s = 0, time.perf_counter()
        while time.perf_counter() - t_s < settle_s:
            for _ in range(4):
                fn(n + 1, batches[n % len(batches)])
                n += 1
            torch.cuda.synchronize()
        for s in range(warmup):
            fn(s + 1, batches[s % len(batches)])
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record(stream)
        for s in range(steps):
            ev[s][0].record(stream)
            fn(warmup + s + 1, batches[(warmup + s) % len(batches)])
            ev[s][1].record(stream)
        t_end.record(stream)
        torch.cuda.synchronize()
        total = t_start.elapsed_time(t_end)
        per = [a.elapsed_time(b) for a, b in ev]
        return total / steps, float(np.mean(per)), per

    # After an idle period (input generation) the clock ramps for about 0.2 s
    # under this load; untimed steps until it has settled, so the timed steps
    # see the clock a continuously running training loop sees. Reported.
    n_settle, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < args.settle_s:
        for _ in range(8):
            fused(n_settle + 1, batches[n_settle % len(batches)])
            n_settle += 1
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t0
    ms_step, ms_kernel, per = timed(fused, args.steps, args.warmup)
    log(f"[bench] fused: {ms_step:.4f} ms/step, kernel avg {ms_kernel:.4f} ms "
        f"(min {min(per):.4f} max {max(per):.4f})")

    unfused = None
    if not args.no_unfused:
        grad = torch.empty_like(W)

        def unfused_step(step, batch):
            X, dY, offs, _ = batch
            if grouped:
                # Per-expert fp32 gradient stores (an empty expert stores zeros),
                # then one elementwise AdamW over every expert's state.
                for e in range(case.E):
                    r0, r1 = offs[e], offs[e + 1]
                    wg.forge_wgrad(X[r0:r1], dY[r0:r1], grad[e], tile=args.tile)
            else:
                wg.forge_wgrad(X, dY, grad, tile=args.tile)
            if opt == "adamw":
                wg.forge_adamw(grad, W, m, v, step=step, **hp)
            else:
                wg.forge_sgdm(grad, W, m, **hp)

        u_step, u_kernel, _ = timed(unfused_step, args.steps, args.warmup, args.leg_settle_s)
        unfused = {"ms_per_step": round(u_step, 5), "tflops": round(flops / u_step / 1e9, 2),
                   "alg_hbm_bytes": alg_bytes + 8 * n_param,
                   "fused_speedup": round(u_step / ms_step, 4)}
        log(f"[bench] unfused: {u_step:.4f} ms/step")
        del grad

    variants = None
    if not args.no_variants and opt == "adamw" and not grouped:
        # Precision variants on the same workload: fused AdamW with bf16 moments,
        # and the lowering the fusion replaces (gradient rounded to bf16 and
        # stored, then elementwise AdamW on float32 state).
        mb = torch.zeros(W.shape, device=dev, dtype=torch.bfloat16)
        vb = torch.zeros_like(mb)
        gb = torch.empty(W.shape, device=dev, dtype=torch.bfloat16)

        def fused_bf16_state(step, batch):
            X, dY, _, _ = batch
            wg.forge_wgrad_adamw_bf16state(X, dY, W, mb, vb, step=step, tile=args.tile, **hp)

        def bf16_grad_unfused(step, batch):
            X, dY, _, _ = batch
            wg.forge_wgrad_bf16(X, dY, gb, tile=args.tile)
            wg.forge_adamw_mixed(gb, W, m, v, step=step, **hp)

        # fp8 inputs (X E4M3, dY E5M2, power-of-two per-tensor scales) from the
        # same float32 draws as the bf16 batches.
        fp8_batches = []
        for s_ in range(1, args.pool + 1):
            X8, sx, dY8, sdy = synth.dense_inputs_fp8(case, s_)
            fp8_batches.append((torch.from_numpy(X8).to(dev), sx, torch.from_numpy(dY8).to(dev),
                                sdy))

        def fused_fp8(step, batch):
            X8, sx, dY8, sdy = fp8_batches[(step - 1) % len(fp8_batches)]
            wg.forge_wgrad_adamw_fp8(X8, "e4m3", sx, dY8, "e5m2", sdy, W, m, v, step=step,
                                     tile=args.tile, **hp)

        variants = {}
        for name, fn, nbytes in (("fused_adamw_bf16_state", fused_bf16_state,
                                  x_bytes + 16 * n_param),
                                 ("bf16_gradient_then_adamw", bf16_grad_unfused,
                                  x_bytes + 28 * n_param),
                                 ("fused_adamw_fp8_inputs", fused_fp8,
                                  x_bytes // 2 + 24 * n_param)):
            v_step, v_kernel, _ = timed(fn, args.steps, args.warmup, args.leg_settle_s)
            variants[name] = {"ms_per_step": round(v_step, 5),
                              "tflops": round(flops / v_step / 1e9, 2),
                              "alg_hbm_bytes": nbytes,
                              }
            # each variant against the peak of the arithmetic it runs
            if "fp8" in name:
                variants[name]["frac_fp8_peak"] = round(flops / v_step / 1e9 / PEAK_FP8_TFLOPS,
                                                        4)
            else:
                variants[name]["frac_bf16_peak"] = round(flops / v_step / 1e9 / PEAK_BF16_TFLOPS,
                                                         4)
            log(f"[bench] {name}: {v_step:.4f} ms/step")
        del mb, vb, gb, fp8_batches

    backward = None
    if not args.no_backward and opt == "adamw" and not grouped:
        # The layer's input gradient dX = dY W_b (bf16 out) on its own, then the
        # whole backward: dX from the weight before the step, then the fused step.
        # Each from the float32 weight and from its bf16 copy (rounded once here;
        # the fused step keeps it current).
        dX = torch.empty((case.T, case.d_in), device=dev, dtype=torch.bfloat16)
        Wb = W.to(torch.bfloat16)

        def dgrad_only(step, batch):
            wg.forge_dgrad(batch[1], W, dX, tile=0)

        def dgrad_copy(step, batch):
            wg.forge_dgrad_bf16w(batch[1], Wb, dX, tile=0)

        def linear_backward(step, batch):
            X, dY, _, _ = batch
            wg.forge_linear_backward_adamw(X, dY, W, m, v, dX, step=step, tile=args.tile, **hp)

        def linear_backward_copy(step, batch):
            X, dY, _, _ = batch
            wg.forge_linear_backward_adamw_bf16w(X, dY, W, m, v, Wb, dX, step=step,
                                                 tile=args.tile, **hp)

        dx_bytes = 2 * case.T * case.d_out + 2 * case.T * case.d_in
        backward = {}
        for name, fn, nbytes in (("dgrad", dgrad_only, dx_bytes + 4 * n_param),
                                 ("dgrad_bf16_copy", dgrad_copy, dx_bytes + 2 * n_param)):
            d_step, d_kernel, _ = timed(fn, args.steps, args.warmup, args.leg_settle_s)
            backward[name] = {"ms_per_step": round(d_step, 5), "kernel_ms": round(d_kernel, 5),
                              "tflops": round(flops / d_kernel / 1e9, 2),
                              "frac_bf16_peak": round(flops / d_kernel / 1e9 / PEAK_BF16_TFLOPS,
                                                      4),
                              "alg_hbm_bytes": nbytes}
            log(f"[bench] {name}: {d_step:.4f} ms/step")
        for name, fn in (("linear_backward_adamw", linear_backward),
                         ("linear_backward_adamw_bf16_copy", linear_backward_copy)):
            b_step, _, _ = timed(fn, args.steps, args.warmup, args.leg_settle_s)
            backward[name] = {"ms_per_step": round(b_step, 5),
                              "tflops": round(2 * flops / b_step / 1e9, 2)}
            log(f"[bench] {name}: {b_step:.4f} ms/step")
        del dX, Wb

    if args.copy_calib_mib:
        n = args.copy_calib_mib * (1 << 20) // 4
        a = torch.ones(n, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {args.copy_calib_mib} MiB copied")

    value = flops / ms_step / 1e9
    achieved = flops / ms_kernel / 1e9
    # Roofline of the fused kernel: the bound is whichever of the MFMA time and
    # the HBM time of the algorithmic work is longer at the spec peaks; the
    # combined fraction max(t_mfma, t_hbm) / t applies to either bound.
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    t_hbm = alg_bytes / (PEAK_HBM_GBS * 1e9) * 1e3
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        gbs = alg_bytes / ms_kernel / 1e6
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}
    sha = kernel_source_sha()
    traffic = read_traffic(args.workload, sha)
    counters = read_counters(args.workload, sha, n_param)

    cpu = None
    if not args.no_cpu:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max([p.get("num_threads", 1) for p in threadpool_info()
                           if p.get("user_api") == "blas"] or [1])
        except Exception:  # pragma: no cover
            threads = os.cpu_count() or 1
        Xb, Yb, offs = batches[0][3]
        Wc, mc, vc = W0.copy(), m0.copy(), v0.copy()
        ahp = dict(lr=case.lr, beta1=case.beta1, beta2=case.beta2, eps=case.eps,
                   weight_decay=case.weight_decay)
        log("[bench] CPU oracle leg ...")
        # Whole oracle steps on the host (fp64 contraction + fp32 optimizer), repeated
        # until about 10 s have elapsed; the value is their mean throughput.
        n_done, c_s = 0, 0.0
        while n_done < 1 or (c_s < 10.0 and n_done < 20):
            c0 = time.perf_counter()
            if grouped:
                grads = oracle.grouped_wgrad(Xb, Yb, offs)
                oracle.grouped_adamw_step(Wc, mc, vc, grads, n_done + 1, **ahp)
            else:
                g = oracle.wgrad(Xb, Yb)
                if opt == "adamw":
                    oracle.adamw_step(Wc, mc, vc, g, n_done + 1, **ahp)
                else:
                    oracle.sgdm_step(Wc, mc, g, lr=case.lr, momentum=case.momentum)
            c_s += time.perf_counter() - c0
            n_done += 1
        what = ("grouped fp64 GEMMs + fp32 AdamW" if grouped else
                f"fp64 GEMM {case.T}x{case.d_in}x{case.d_out} + fp32 {opt}")
        sample = f"{n_done} full oracle steps of {args.workload} ({what}), {c_s:.1f} s"
        cpu = {"value": round(n_done * flops / c_s / 1e12, 5), "unit": "TFLOP/s",
               "cores": int(threads), "kind": "oracle", "sample": sample,
               "seconds": round(c_s, 3), "host_cpus": os.cpu_count()}
        log(f"[bench] CPU oracle: {sample}")

    if grouped:
        wl = (f"{case.name}: {case.E} experts W[{case.d_out},{case.d_in}] fp32, "
              f"{rows} routed rows, AdamW")
        cfg = {"workload": wl, "experts": case.E, "routed_rows": rows, "d_in": case.d_in,
               "d_out": case.d_out, "optimizer": opt, "tile": args.tile}
    else:
        wl = (f"{case.name}: X bf16[{case.T},{case.d_in}] dY bf16[{case.T},{case.d_out}] "
              f"W/m/v fp32[{case.d_out},{case.d_in}], {opt}")
        cfg = {"workload": wl, "T": case.T, "d_in": case.d_in, "d_out": case.d_out,
               "optimizer": opt, "tile": args.tile}
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"steps": n_settle, "seconds": round(settle_s, 3),
                   "per_comparison_leg_s": args.leg_settle_s},
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; inputs resident in HBM)",
        "config": cfg,
        "mfma_util_pct": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": dict(roof, traffic=traffic),
        "combined_roofline": {"t_mfma_ms": round(t_mfma, 5), "t_hbm_ms": round(t_hbm, 5),
                              "frac": round(max(t_mfma, t_hbm) / ms_kernel, 4)},
        "kernel_ms": round(ms_kernel, 5),
        "alg_hbm_bytes": alg_bytes,
        "alg_hbm_gbs": round(alg_bytes / ms_kernel / 1e6, 1),
        "hbm_frac_alg": round(alg_bytes / ms_kernel / 1e6 / PEAK_HBM_GBS, 4),
        "unfused": unfused,
        "precision_variants": variants,
        "backward": backward,
        "kernel_source_sha": sha,
        "counters": counters,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
