"""Helpers shared by the GPU parity tests: seeded workloads onto the device, the HIP operator, and
the oracle on selected rows."""
import sys

import numpy as np

import hyena_inputs as hi
from oracle import hyena_oracle as orc

FP32_TOL = 1e-4      # per-row relative L2, fp32 storage
BF16_TOL = 2e-2      # per-row relative L2, bf16 storage with fp32 arithmetic


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


def run_hip_operator(w, v, xs, params, mode=None):
    """Filter spectra + operator through the C ABI; returns y on the host as float64."""
    import torch
    import attention_free_long_implicit_amd as hy
    dt = torch_dtype(w)
    vd = to_dev(v, dt)
    xd = [to_dev(x, dt) for x in xs]
    spectra = [hy.filter_gen(params_to_dev(p), w.dims, mode=mode) for p in params]
    y = hy.operator(vd, xd, spectra, mode=mode)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


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
