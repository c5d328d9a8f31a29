#!/usr/bin/env python3
"""Benchmark of the Hyena operator hot path on one MI355X.

A step is one call of the order-N operator (every order: load, zero-padded forward transform,
product with the cached filter spectrum, inverse transform, cut to the output window, gate, store)
over one batch of seeded synthetic input already resident in HBM.  The filter spectra depend only on
the filter parameters and the grid, so they are built once (hyena_filter_gen) before the timed region;
that build is reported separately as ``filter_gen_ms``.

Prints ONE JSON line.  Default workload: order 2, B=4, D=768, L=8192, bf16 storage (workload 1), whose
convolution runs on the matrix cores;
``--workload i`` times another of hyena_inputs.WORKLOADS (parity configurations are not bench lines).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import hyena_inputs as hi  # noqa: E402

PEAK_HBM_GBPS = 8000.0
METRIC = "Hyena op tokens·channels/s + HBM GB/s (% peak), order 2, L=8K..1M, 1 GPU"


def algorithmic_bytes_per_order(w) -> int:
    """One HBM round trip per order: read u, read x_i, write u_i (s bytes each per token-channel),
    plus the filter read once in its smallest exact form (fp32 taps), shared by the B rows of a channel."""
    return 3 * w.elem_bytes * w.tokens_channels + 4 * w.D * w.support


def floor_bytes_per_step(w) -> int:
    """All orders fused on chip: read v and the N gates, write y, plus the N filters (fp32 taps)."""
    return (w.order + 2) * w.elem_bytes * w.tokens_channels + 4 * w.order * w.D * w.support


def uses_matrix_cores(w) -> bool:
    """Causal, bf16 storage, L = 8192, rows in pairs of one channel: the library's matrix-core kernel."""
    return w.mode == "causal" and w.dtype == "bf16" and w.dims[0] == 8192 and w.B % 2 == 0


def single_launch_per_order(w) -> bool:
    """1-D lengths whose transform fits one workgroup: one fused kernel per order."""
    return w.ndim == 1 and (w.dims[0] <= 16384 or w.mode == "circular")


def kernel_key(w) -> str:
    circ = "_periodic" if w.mode == "circular" else ""
    if w.ndim == 3:
        return f"conv3d_{w.dims[0]}cubed_{w.dtype}{circ}"
    L = w.dims[0]
    if uses_matrix_cores(w):
        return f"conv_mfma_L{L}_bf16_pairs"
    return f"conv1d_L{L}_{w.dtype}_gate{circ}" if single_launch_per_order(w) else f"fourstep_L{L}_{w.dtype}"


def arithmetic(w) -> str:
    if uses_matrix_cores(w):
        return "bf16 matrix-core products, fp32 accumulation and twiddles"
    return "fp32"


def load_traffic(key: str):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel sources (matched by hash); else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.load(f)
        ent = data.get(key)
        if not ent:
            return None
        from attention_free_long_implicit_amd.build import source_hash
        if ent.get("source_hash") != source_hash():
            return None
        return ent.get("bytes_per_launch")
    except Exception:
        return None


def cpu_baseline(w, v, xs, params, budget_s: float):
    """The oracle as it stands on whole (b, d) rows (volumes) of the same workload, until about
    budget_s seconds of oracle time; the filters of the sampled channels are built outside the
    timed part (as the GPU's spectra are), and building stops once it has taken 3 x budget_s."""
    from oracle import hyena_oracle as orc
    rows = hi.sample_rows(w, 4096, seed=99)
    circ = w.mode == "circular"
    filt = {}
    n_done, t_used, t_build = 0, 0.0, 0.0
    for b, d in rows:
        if d not in filt:
            if t_build > 3 * budget_s and n_done > 0:
                break
            tb = time.perf_counter()
            if w.ndim == 1:
                filt[d] = [orc.implicit_filter_1d(p, w.dims[0], channels=[d]) for p in params]
            elif circ:
                filt[d] = [orc.implicit_filter_3d_circular(p, w.dims[0], channels=[d]) for p in params]
            else:
                filt[d] = [orc.implicit_filter_3d(p, w.dims[0], channels=[d]) for p in params]
            t_build += time.perf_counter() - tb
            print(f"cpu baseline: filters for channel {d} built ({t_build:.1f} s so far)", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        if w.ndim == 1:
            orc.hyena_operator_rows(v[b, d][None], [x[b, d][None] for x in xs], filt[d], circular=circ)
        else:
            orc.hyena_operator_3d(v[b, d][None], [x[b, d][None] for x in xs], filt[d], circular=circ)
        t_used += time.perf_counter() - t0
        n_done += 1
        if t_used >= budget_s:
            break
    return {"value": n_done * w.points / t_used, "unit": "tokens·channels/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_done} of {w.B * w.D} (b,d) rows of the same workload, order {w.order}, float64 numpy FFT "
                      f"convolution on one core (numpy.fft is single-threaded), filters prebuilt; {t_used:.1f} s"}


def copy_bandwidth(torch, dev, nbytes=1 << 30, reps=10):
    """Device-to-device copy of nbytes (read + write) as the practical bandwidth ceiling."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return 2 * nbytes / (ms / 1e3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU reaches steady-state clocks only under sustained load: 0.1 s of warm-up and timed work
    # (workload 1) measures that state; 50 steps after 5 read about 15 % slower
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", type=int, default=1, help="index into hyena_inputs.WORKLOADS")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy", action="store_true", help="skip the device copy-bandwidth probe")
    ap.add_argument("--cold-steps", type=int, default=50,
                    help="after the timed region, this many more steps, each after a scratch write that evicts the "
                         "256 MB memory-side cache, timed one by one (reported as cold_cache; 0 skips them)")
    ap.add_argument("--evict-mb", type=int, default=1024, help="size of that scratch write")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the operator's (b, d) rows are independent, "
                                   "so a multi-GPU run would shard channels with no communication; use --gpus 1"}))
        sys.exit(2)

    import torch
    import attention_free_long_implicit_amd as hy
    from attention_free_long_implicit_amd import _lib

    w = hi.WORKLOADS[args.workload]
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    vd = torch.from_numpy(v).to(dev).to(dt)
    xd = [torch.from_numpy(x).to(dev).to(dt) for x in xs]
    pd = [{k: torch.from_numpy(a).to(dev) for k, a in p.items()} for p in params]
    y = torch.empty_like(vd)
    mode = {"causal": _lib.CAUSAL, "linear": _lib.LINEAR, "circular": _lib.CIRCULAR}[w.mode]
    ws_n = _lib.workspace_bytes(w.order, w.B, w.D, w.dims, _lib.BF16 if w.dtype == "bf16" else _lib.F32, mode)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None

    # filter spectra (cached per grid): timed separately
    spectra = [hy.filter_gen(p, w.dims, mode=mode) for p in pd]
    torch.cuda.synchronize()
    fg = []
    for _ in range(3):
        t0 = time.perf_counter()
        spectra = [hy.filter_gen(p, w.dims, mode=mode) for p in pd]
        torch.cuda.synchronize()
        fg.append(time.perf_counter() - t0)
    filter_gen_ms = 1e3 * min(fg)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        hy.operator(vd, xd, spectra, y=y, ws=ws, mode=mode)
    torch.cuda.synchronize()

    # two events on the launch stream bracket the timed region (an event after every step would add
    # its own few microseconds to each step)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for k in range(args.steps):
        hy.operator(vd, xd, spectra, y=y, ws=ws, mode=mode)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.full(args.steps, ev0.elapsed_time(ev1) / args.steps)
    ms_per_step = 1e3 * wall / args.steps

    # Back-to-back steps reread the same buffers, part of which the memory-side cache still holds.  The
    # cold figure evicts it before every step (a scratch write several times its size) and times each
    # step by its own events (which add a few microseconds per step).
    cold = None
    if args.cold_steps > 0:
        scratch = torch.empty(args.evict_mb << 18, dtype=torch.float32, device=dev)
        marks = []
        torch.cuda.synchronize()
        for k in range(args.cold_steps):
            scratch.fill_(float(k))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            hy.operator(vd, xd, spectra, y=y, ws=ws, mode=mode)
            e1.record(stream)
            marks.append((e0, e1))
        torch.cuda.synchronize()
        cold_ms = float(np.median([a.elapsed_time(b) for a, b in marks]))
        del scratch
        cold = {"ms_per_step": cold_ms, "steps": args.cold_steps, "evict_mb": args.evict_mb,
                "value": w.tokens_channels / (cold_ms / 1e3),
                "hbm_frac_alg": algorithmic_bytes_per_order(w) * w.order / (cold_ms / 1e3) / 1e9 / PEAK_HBM_GBPS}
    T = w.tokens_channels
    value = T / (ms_per_step / 1e3)
    alg_step = algorithmic_bytes_per_order(w) * w.order
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens·channels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded activations, Xavier-uniform filter networks; see hyena_inputs)",
        "config": {"workload": w.name, "order": w.order, "B": w.B, "D": w.D, "grid": list(w.dims),
                   "boundary": w.mode, "storage": w.dtype, "arithmetic": arithmetic(w),
                   "alpha_range": [w.alpha_lo, w.alpha_hi],
                   "inputs": f"numpy default_rng([{w.index}, stream]): stream 0 activations, stream 1 filter parameters"},
        "hbm_gbps_alg": alg_step / (ms_per_step / 1e3) / 1e9,
        "hbm_frac_alg": alg_step / (ms_per_step / 1e3) / 1e9 / PEAK_HBM_GBPS,
        "event_ms_per_step": float(np.mean(step_ms)),
        "filter_gen_ms": filter_gen_ms,
    }
    if cold is not None:
        out["cold_cache"] = cold
    # filter network (a GEMM pair per position) for all orders; the time includes the spectrum build
    net_flop = 2.0 * w.order * w.support * w.hidden * (w.features + w.D)
    out["filter_gen"] = {"ms": filter_gen_ms, "network_gflop": net_flop / 1e9,
                         "achieved_tflops": net_flop / (filter_gen_ms / 1e3) / 1e12, "peak_tflops": 157.3,
                         "note": "all orders; network flops over the whole filter build (spectra included)"}
    key = kernel_key(w)
    if uses_matrix_cores(w) and w.order <= 8:
        # the whole step is one launch of the matrix-core kernel: all orders, u_i kept on chip
        launch_ms = float(np.mean(step_ms))
        achieved = alg_step / (launch_ms / 1e3) / 1e9
        floor = floor_bytes_per_step(w)
        out["roofline"] = {"bound": "hbm", "kernel": key, "achieved": achieved, "peak": PEAK_HBM_GBPS,
                           "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS, "traffic": load_traffic(key),
                           "launch_ms": launch_ms, "alg_bytes_per_launch": alg_step,
                           "floor_bytes_per_launch": floor,
                           "floor_frac": floor / (launch_ms / 1e3) / 1e9 / PEAK_HBM_GBPS}
    elif single_launch_per_order(w):
        # the whole step is `order` launches of one fused kernel: its average launch duration
        launch_ms = float(np.mean(step_ms)) / w.order
        bytes_launch = algorithmic_bytes_per_order(w)
        achieved = bytes_launch / (launch_ms / 1e3) / 1e9
        out["roofline"] = {"bound": "hbm", "kernel": key, "achieved": achieved, "peak": PEAK_HBM_GBPS,
                           "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS, "traffic": load_traffic(key),
                           "launch_ms": launch_ms, "alg_bytes_per_launch": bytes_launch}
    else:
        # several kernels per order: the whole step against the algorithmic bytes of the step
        achieved = alg_step / (float(np.mean(step_ms)) / 1e3) / 1e9
        out["roofline"] = {"bound": "hbm", "kernel": key + " (whole step)", "achieved": achieved,
                           "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                           "traffic": load_traffic(key), "alg_bytes_per_step": alg_step}
    if not args.no_copy:
        out["copy_gbps"] = copy_bandwidth(torch, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, v, xs, params, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
