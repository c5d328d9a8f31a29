"""Helpers shared by the GPU parity tests: seeded workloads onto the device, the HIP operator, and
the oracle on selected rows or on every row of a workload."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import hyena_inputs as hi
from oracle import hyena_oracle as orc

FP32_TOL = 1e-4      # per-row relative L2, fp32 storage
BF16_TOL = 2e-2      # per-row relative L2, bf16 storage (bf16 operands allowed inside the transforms)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(w):
    import torch
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def to_dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dtype).contiguous()


def params_to_dev(p):
    import torch
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda") for k, v in p.items()}


def run_hip_operator(w, v, xs, params, mode=None, host_dtype=np.float64):
    """Filter spectra + operator through the C ABI; returns y on the host (float64 by default)."""
    import torch
    import attention_free_long_implicit_amd as hy
    dt = torch_dtype(w)
    vd = to_dev(v, dt)
    xd = [to_dev(x, dt) for x in xs]
    spectra = [hy.filter_gen(params_to_dev(p), w.dims, mode=mode) for p in params]
    y = hy.operator(vd, xd, spectra, mode=mode)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(host_dtype, copy=False)


def oracle_rows_1d(w, v, xs, params, rows, circular=False):
    """Oracle output for the given (b, d) rows: [len(rows), L] float64 (periodic with ``circular``)."""
    L = w.dims[0]
    out = []
    cache = {}
    for b, d in rows:
        if d not in cache:
            cache[d] = [orc.implicit_filter_1d(p, L, channels=[d]) for p in params]
        hs = cache[d]
        y = orc.hyena_operator_rows(v[b, d][None], [x[b, d][None] for x in xs], hs, circular=circular)
        out.append(y[0])
    return np.stack(out)


def rel_err_rows(got_rows, ref_rows, point_axes=1):
    return orc.rel_l2_per_row(got_rows, ref_rows, point_axes=point_axes)


def oracle_threads() -> int:
    """Host threads for the oracle (numpy's FFT releases the interpreter lock): every core this process
    may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def all_row_errors(w, v, xs, params, got, circular=False):
    """Per-row relative L2 error of ``got`` [B, D, *grid] against the oracle on EVERY (b, d) row (3-D: volume)
    of the workload: [B * D] float64.  The filters of every channel are built once; the rows run on a thread
    pool, each through the oracle's own operator."""
    B, D = w.B, w.D
    if w.ndim == 1:
        L = w.dims[0]
        hs = [orc.implicit_filter_1d(p, L) for p in params]                 # [D, L] each

        def one(r):
            b, d = divmod(r, D)
            ref = orc.hyena_operator_rows(v[b, d][None], [x[b, d][None] for x in xs], [h[d][None] for h in hs],
                                          circular=circular)
            return orc.rel_l2_per_row(np.asarray(got[b, d], np.float64)[None], ref)[0]
    else:
        n = w.dims[0]
        if circular:
            hs = [orc.implicit_filter_3d_circular(p, n) for p in params]
        else:
            hs = [orc.implicit_filter_3d(p, n) for p in params]

        def one(r):
            b, d = divmod(r, D)
            ref = orc.hyena_operator_3d(v[b, d][None], [x[b, d][None] for x in xs], [h[d][None] for h in hs],
                                        circular=circular)
            return orc.rel_l2_per_row(np.asarray(got[b, d], np.float64)[None], ref, point_axes=3)[0]
    with ThreadPoolExecutor(oracle_threads()) as ex:
        errs = list(ex.map(one, range(B * D), chunksize=max(1, (B * D) // (8 * oracle_threads()))))
    return np.asarray(errs, dtype=np.float64)


def report_errors(what, e):
    """Print max / median / count of per-row errors (one line, flushed)."""
    say(f"  {what}: max rel err {e.max():.3e} median {np.median(e):.3e} over {e.size} rows "
        f"(worst row {int(np.argmax(e))})")
