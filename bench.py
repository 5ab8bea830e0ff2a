"""Benchmark of the Muon-style optimizer step on one MI355X.

One "step" is one call of muon_step over the whole 124M GPT-2-shaped matrix
set (72 bf16 matrices: 12 layers x {Q, K, V, O 768x768; MLP 768x3072;
MLP 3072x768}), fp32 momentum, five quintic Newton-Schulz iterations, grouped
by effective shape: momentum, norm, 5 x (Gram, polynomial, apply), update.
Inputs are synthetic (seeded low-rank + noise gradients at entry RMS 1e-3,
0.02 N(0,1) parameters) and resident in HBM before the timed region.

`--workload` selects another configuration of the same step for measurement
(the line's metric is the 124M set's; the others are timed the same way):
gpt124m_anvil (fast/slow momentum, six map steps, cautious decay 0.1, EMA),
gpt2p7b (32 layers x {4x 2560^2, 2560x10240, 10240x2560}, wd 1.6) and
moe_share (64 experts x {2048x1408, 1408x2048} + 24 x 4 x 2048^2).

Prints one JSON line.  Extra fields: NS TFLOP/s (symmetric flop count),
per-kernel times, elementwise GB/s, the roofline of the dominant kernel (the
APPLY GEMM, timed live with HIP events around its launches in the timed
region), the step replayed from one captured device graph, `configs` (the
same record for the other matrix sets: the ANVIL option set, the 2.7B set
and the MoE share, each timed the same way after the main line), a single
256x512 matrix eager and replayed, AdamW over the 124M model's other
parameters, and the CPU oracle timed on the host: one whole step for the
124M sets, one matrix per distinct shape (labelled as an estimate for the
whole step) for the 2.7B and MoE sets.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
WORKLOADS = {
    "gpt124m": "gpt124m matrix set: 72 bf16 matrices (48x 768x768, 12x 768x3072, 12x 3072x768), "
               "fp32 momentum, Muon step, 5 quintic Newton-Schulz iterations, grouped by shape",
    "gpt124m_anvil": "gpt124m matrix set, ANVIL-style step: fast (0.9) and slow (0.99) momentum, "
                     "6 quintic map iterations, cautious weight decay 0.1, EMA 0.99 from step 1",
    "gpt2p7b": "2.7B matrix set: 192 bf16 matrices (128x 2560x2560, 32x 2560x10240, "
               "32x 10240x2560), fp32 momentum, wd 1.6, 5 quintic iterations",
    "moe_share": "MoE one-GPU share: 224 bf16 matrices (64x 2048x1408, 64x 1408x2048, "
                 "96x 2048x2048), fp32 momentum, 5 quintic iterations",
}


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_apply_{workload}.json")


def _src_hash() -> str:
    h = hashlib.sha256()
    for f in ("muon_gemm.hip", "muon_common.h"):
        with open(os.path.join(ROOT, "orthogonalising_matrix_optimizer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(workload: str, launch_flops_key: str):
    """HBM bytes per APPLY launch from the committed counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_src_sha256_16") != _src_hash() or t.get("workload") != launch_flops_key:
        return None
    return t.get("hbm_bytes_per_launch")


def apply_flops(shapes) -> float:
    """Algorithmic flops of one APPLY launch: 2 m^2 n per matrix."""
    tot = 0.0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        tot += 2.0 * m * m * n
    return tot


def elementwise_bytes(shapes, ms):
    """Algorithmic HBM bytes of the prepare and finish kernels (bf16
    params/grads/iterate, fp32 state): prepare reads G (2) and M (4), writes
    M (4) and X0 (2), plus S (4 + 4) with slow momentum; finish reads O (2) and
    W (2), writes W (2), plus S (4) with cautious decay and E (4 + 4) with an
    average."""
    n = sum(r * c for r, c in shapes)
    prep = 12.0 + (8.0 if ms.beta_slow >= 0 else 0.0)
    fin = 6.0 + (4.0 if ms.cautious else 0.0) + (8.0 if ms.beta_ema >= 0 else 0.0)
    return prep * n, fin * n


def cpu_baseline(ms, coeffs, whole_step: bool):
    """The CPU oracle (fp64 numpy, the float32 state recurrences) on the same
    step.  whole_step: one whole step of the set, measured.  Otherwise (sets
    whose oracle step takes minutes) one matrix of each distinct shape is
    measured and the step's time is estimated as the sum over shapes of the
    measured time times the shape's matrix count; the record says so."""
    import threadpoolctl
    from oracle import muon_oracle as orc
    from workloads import gen
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    vendor = ",".join(sorted({str(i.get("internal_api")) for i in info
                              if i.get("user_api") == "blas"})) or "unknown"
    shapes = list(ms.shapes)
    if whole_step:
        idx = list(range(len(shapes)))
    else:
        first = {}
        for i, s in enumerate(shapes):
            first.setdefault(s, i)
        idx = list(first.values())
    times = {}
    for i in idx:
        (g, w), = gen.make_inputs(ms, seed=0, indices=[i])
        st = orc.OracleState([shapes[i]], beta_slow=ms.beta_slow, beta_ema=ms.beta_ema,
                             ema_start=ms.ema_start)
        t0 = time.perf_counter()
        orc.muon_step([gen.f32_from_bf16_bits(w).astype(np.float64)], [gen.f32_from_bf16_bits(g)],
                      st, coeffs, ms.lr, ms.wd, ms.beta, param_dtype="bf16",
                      cautious=ms.cautious, keep=False)
        times[i] = time.perf_counter() - t0
    measured = sum(times.values())
    if whole_step:
        est = measured
        sample = (f"one whole step of the same {len(shapes)}-matrix set on the host, measured "
                  f"({measured:.2f} s")
    else:
        count = {}
        for s in shapes:
            count[s] = count.get(s, 0) + 1
        est = sum(times[i] * count[shapes[i]] for i in idx)
        sample = (f"{len(idx)} of the {len(shapes)} matrices measured (one per distinct shape: "
                  + ", ".join(f"{shapes[i][0]}x{shapes[i][1]} {times[i]:.2f} s" for i in idx)
                  + f"); the whole step is an ESTIMATE, each shape's time times its matrix "
                    f"count ({est:.1f} s")
    return {"value": round(1.0 / est, 5), "unit": "optimizer steps/s", "cores": int(threads),
            "kind": "oracle", "measured_s": round(measured, 3), "estimated": not whole_step,
            "sample": sample + f", fp64 numpy, BLAS {vendor})"}


def _events_ms(fn, reps):
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_graph(opt, grads, reps):
    """ms per step of `opt` stepping on `grads` through one captured graph."""
    import torch
    g = opt.graph(grads)
    g.replay()
    torch.cuda.synchronize()
    return round(_events_ms(g.replay, reps), 4)


def single_matrix_times(gen, mo, dev, reps, with_oracle=True):
    """One 256x512 fp32 matrix (five quintic iterations, bf16 operands): ms per
    step eager and as a replayed graph, and the CPU oracle on one thread."""
    import torch
    ms = gen.SETS["single_256x512"]
    (g, w), = gen.make_inputs(ms, seed=0)
    p = [torch.from_numpy(w).to(dev)]
    gr = [torch.from_numpy(g).to(dev)]
    opt = mo.Muon(p, lr=ms.lr, wd=ms.wd, beta=ms.beta, steps=ms.steps,
                  coeffs=gen.coeff_table(ms.coeffs, ms.steps))
    for _ in range(5):
        opt.step(gr)
    eager = _events_ms(lambda: opt.step(gr), max(reps, 20))
    out = {"workload": "one 256x512 fp32 matrix, 5 quintic iterations, bf16 operands",
           "eager_ms_per_step": round(eager, 4),
           "graph_ms_per_step": time_graph(opt, gr, max(reps, 20))}
    if with_oracle:
        # the CPU oracle on the same matrix, BLAS limited to one thread
        import threadpoolctl
        from oracle import muon_oracle as orc
        with threadpoolctl.threadpool_limits(limits=1, user_api="blas"):
            coeffs = gen.coeff_table(ms.coeffs, ms.steps)
            t = []
            for _ in range(5):
                st = orc.OracleState([ms.shapes[0]])
                t0 = time.perf_counter()
                orc.muon_step([w.astype(np.float64)], [g], st, coeffs, ms.lr, ms.wd, ms.beta,
                              param_dtype="f32", keep=False)
                t.append(time.perf_counter() - t0)
        out["cpu_oracle_ms_per_step_1_thread"] = round(1e3 * float(np.median(t)), 3)
    return out


def adamw_times(gen, mo, dev, reps):
    """AdamW over the 124M model's non-matrix parameters (embeddings, LayerNorm
    and bias vectors: 124 bf16 tensors, 39.5M elements), one grouped launch:
    kernel time from HIP events around the launch, and whole-call time."""
    import torch
    sizes = gen.gpt124m_adamw_sizes()
    params = [gen.torch_flat(gen.flat_param(n, 0, i), dev, torch.bfloat16)
              for i, n in enumerate(sizes)]
    grads = [gen.torch_flat(gen.flat_grad(n, 0, 0, i), dev, torch.bfloat16)
             for i, n in enumerate(sizes)]
    opt = mo.AdamW(params, lr=3e-3, betas=(0.9, 0.95), eps=1e-8, wd=0.0)
    for _ in range(3):
        opt.step(grads)
    call_ms = _events_ms(lambda: opt.step(grads), reps)
    mo.probe_arm("adamw", reps)
    for _ in range(reps):
        opt.step(grads)
    torch.cuda.synchronize()
    k = mo.probe_read(reps)
    mo.probe_disarm()
    kernel_ms = float(np.mean(k))
    n = int(sum(sizes))
    nbytes = n * (2 * 2 + 2 + 16)   # p bf16 read+write, g bf16, m and v fp32 read+write
    gbs = nbytes / (kernel_ms * 1e-3) / 1e9
    return {"workload": "gpt124m non-matrix parameters: 124 bf16 tensors (embeddings, "
                        "LayerNorm gains/biases, linear biases), fp32 moments",
            "elements": n, "tensors": len(sizes), "kernel_ms": round(kernel_ms, 4),
            "call_ms": round(call_ms, 4), "bytes_per_element": 22,
            "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def measure(name, steps, warmup, mo, gen, dev, with_graph=False):
    """Time `steps` optimizer steps of matrix set `name` after `warmup` steps
    (inputs resident in HBM), with HIP events around every APPLY launch of the
    timed region, then per-phase kernel times from a short extra run."""
    import torch
    ms = gen.SETS[name]
    shapes = list(ms.shapes)
    coeffs = gen.coeff_table(ms.coeffs, ms.steps)
    if ms.numel <= 200_000_000:
        inputs = gen.make_inputs(ms, seed=0)

        def to_dev(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

        params = [to_dev(w) for _, w in inputs]
        grads = [to_dev(g) for g, _ in inputs]
        del inputs
    else:
        # large sets: the same recipe drawn on the device
        params = [gen.torch_param_matrix(r, c, 0, i, dev, dtype=torch.bfloat16)
                  for i, (r, c) in enumerate(shapes)]
        grads = [gen.torch_grad_matrix(r, c, 0, 0, i, dev, rms=ms.grad_rms, dtype=torch.bfloat16)
                 for i, (r, c) in enumerate(shapes)]
    opt = mo.Muon(params, lr=ms.lr, wd=ms.wd, beta=ms.beta, steps=ms.steps, coeffs=coeffs,
                  ns_dtype="bf16", beta_slow=None if ms.beta_slow < 0 else ms.beta_slow,
                  beta_ema=None if ms.beta_ema < 0 else ms.beta_ema, ema_start=ms.ema_start,
                  cautious=ms.cautious)
    plan = mo.plan_info(shapes, ms.steps, coeffs)
    stream = torch.cuda.current_stream()

    for _ in range(warmup):
        opt.step(grads)
    torch.cuda.synchronize()

    # timed region; the APPLY launches are bracketed with HIP events on the
    # launch stream (a last APPLY that carries the parameter update is a
    # separate kernel and phase, apply_update)
    n_apply = steps * ms.steps
    mo.probe_arm("apply", n_apply)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    t0 = time.perf_counter()
    for k in range(steps):
        opt.step(grads)
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev[0].elapsed_time(ev[-1]) / steps
    per_step = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(steps)])
    apply_ms = mo.probe_read(n_apply)
    mo.probe_disarm()

    # per-phase averages from a short extra run (not part of the timed region)
    phase_ms = {}
    for ph in ("prepare", "gram", "poly", "finish", "apply_update"):
        cap = 5 * (ms.steps if ph in ("gram", "poly") else 1)
        mo.probe_arm(ph, cap)
        for _ in range(5):
            opt.step(grads)
        torch.cuda.synchronize()
        t = mo.probe_read(cap)
        mo.probe_disarm()
        phase_ms[ph] = round(float(np.mean(t)), 4) if t else None
    phase_ms["apply"] = round(float(np.mean(apply_ms)), 4) if apply_ms else None

    graph_ms = None
    if with_graph and (ms.beta_ema < 0 or opt.ema_count > 0):
        graph_ms = time_graph(opt, grads, steps)

    sym, dense = gen.ns_flops(shapes, ms.steps)
    a_flops = apply_flops(shapes)
    a_tf = a_flops / (phase_ms["apply"] * 1e-3) / 1e12
    traffic = _traffic(name, f"{name}:{ms.steps}:{ms.coeffs}")
    prep_b, fin_b = elementwise_bytes(shapes, ms)
    prep_gbs = prep_b / (phase_ms["prepare"] * 1e-3) / 1e9
    fin_gbs = fin_b / (phase_ms["finish"] * 1e-3) / 1e9 if phase_ms["finish"] else None
    rec = {
        "workload": WORKLOADS[name],
        "value": round(1000.0 / ms_step, 3),
        "unit": "optimizer steps/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_p10_median_p90": [round(float(np.percentile(per_step, q)), 4)
                                       for q in (10, 50, 90)],
        "config": {"matrices": len(shapes), "elements": int(sum(r * c for r, c in shapes)),
                   "ns_steps": ms.steps, "coeffs": "quintic (15/8, -10/8, 3/8)",
                   "groups": plan["groups"], "tile": plan["tile"],
                   "launches_per_step": plan["launches_per_step"]},
        "ns_tflops": round(sym / (ms_step * 1e-3) / 1e12, 2),
        "ns_frac_mfma_peak": round(sym / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "ns_flops_per_step": {"symmetric": sym, "dense_equivalent": dense},
        "kernel_ms": phase_ms,
        "elementwise_gbs": {"prepare": round(prep_gbs, 1),
                            "finish": round(fin_gbs, 1) if fin_gbs else None},
        "elementwise_frac_hbm_peak": {"prepare": round(prep_gbs / PEAK_HBM_GBS, 4),
                                      "finish": round(fin_gbs / PEAK_HBM_GBS, 4) if fin_gbs
                                      else None},
        # the plain update runs in the last APPLY launch's epilogue (no finish
        # launch); that launch is timed as apply_update, not in apply/roofline
        "update_in_last_apply": phase_ms["apply_update"] is not None,
        "roofline": {"bound": "mfma", "kernel": "APPLY (X <- aX + BX, bf16 MFMA)",
                     "achieved": round(a_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(a_tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "flops_per_launch": a_flops, "launches_timed": len(apply_ms)},
        "wall_s_timed": round(wall, 4),
        "graph_ms_per_step": graph_ms,
    }
    del opt, params, grads
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="gpt124m", choices=sorted(WORKLOADS),
                    help="matrix set and options of the step (default: the 124M set)")
    ap.add_argument("--no-configs", action="store_true",
                    help="leave out the records of the other matrix sets and the extras "
                         "(single matrix, AdamW, graph replay)")
    ap.add_argument("--single-only", action="store_true",
                    help="only time the single 256x512 matrix step (eager and replayed)")
    ap.add_argument("--adamw-only", action="store_true",
                    help="only time the AdamW step over the 124M model's non-matrix parameters")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("this benchmark runs on one GPU only: the optimizer step is measured on a single "
              "MI355X (the multi-GPU layout is a design note, not a measured path)", file=sys.stderr)
        sys.exit(2)

    import torch
    import orthogonalising_matrix_optimizer_amd as mo
    from workloads import gen

    dev = torch.device("cuda:0")
    if args.copy_calib:
        n = args.copy_calib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_read": n * 4, "copy_calib_bytes_written": n * 4}))
        return

    if args.adamw_only:
        print(json.dumps(adamw_times(gen, mo, dev, max(args.steps, 20))), flush=True)
        return
    if args.single_only:
        print(json.dumps(single_matrix_times(gen, mo, dev, args.steps,
                                             with_oracle=not args.no_cpu_baseline)), flush=True)
        return

    name = args.workload
    main_rec = measure(name, args.steps, args.warmup, mo, gen, dev,
                       with_graph=not args.no_configs)
    out = {
        "metric": "optimizer steps/sec + NS TFLOP/s (% MFMA peak), 124M-GPT matrix set, 1 GPU"
                  if name == "gpt124m" else
                  f"optimizer steps/sec + NS TFLOP/s (% MFMA peak), {name} matrix set, 1 GPU",
        "value": main_rec["value"],
        "unit": "optimizer steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_rec["ms_per_step"],
        "ms_per_step_p10_median_p90": main_rec["ms_per_step_p10_median_p90"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded low-rank+noise gradients, random-init bf16 parameters)",
        "config": dict({"workload": main_rec["workload"]}, **main_rec["config"]),
    }
    for k in ("ns_tflops", "ns_frac_mfma_peak", "ns_flops_per_step", "kernel_ms",
              "elementwise_gbs", "elementwise_frac_hbm_peak", "update_in_last_apply",
              "roofline", "wall_s_timed", "graph_ms_per_step"):
        out[k] = main_rec[k]
    if not args.no_configs:
        # the other matrix sets of the same step, each timed the same way
        # (fewer steps for the 2.7B set, whose step takes ~0.1 s)
        others = {}
        for other in ("gpt124m_anvil", "gpt2p7b", "moe_share"):
            if other == name:
                continue
            st = min(args.steps, 10) if other == "gpt2p7b" else args.steps
            wu = min(args.warmup, 3) if other == "gpt2p7b" else args.warmup
            others[other] = measure(other, st, wu, mo, gen, dev)
            print(f"measured {other}: {others[other]['ms_per_step']} ms per step",
                  file=sys.stderr, flush=True)
        out["configs"] = others
        out["single_matrix"] = single_matrix_times(gen, mo, dev, args.steps,
                                                   with_oracle=not args.no_cpu_baseline)
        out["adamw"] = adamw_times(gen, mo, dev, max(args.steps, 20))
    if not args.no_cpu_baseline:
        coeffs = gen.coeff_table(gen.SETS[name].coeffs, gen.SETS[name].steps)
        out["cpu_baseline"] = cpu_baseline(gen.SETS[name], coeffs,
                                           whole_step=gen.SETS[name].numel <= 200_000_000)
        if not args.no_configs:
            for other, rec in out["configs"].items():
                ms = gen.SETS[other]
                rec["cpu_baseline"] = cpu_baseline(ms, gen.coeff_table(ms.coeffs, ms.steps),
                                                   whole_step=ms.numel <= 200_000_000)
                print(f"oracle {other}: {rec['cpu_baseline']['measured_s']} s measured",
                      file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
