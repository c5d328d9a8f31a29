#!/usr/bin/env python3
"""Benchmark of the Hyena operator hot path on one MI355X.

A step is one call of the order-N operator (every order: load, zero-padded forward transform,
product with the cached filter spectrum, inverse transform, cut to the output window, gate, store)
over one batch of seeded synthetic input already resident in HBM.  The filter spectra depend only on
the filter parameters and the grid, so they are built once (hyena_filter_gen) before the timed region;
that build is reported separately as ``filter_gen_ms``.  Input-dependent (per-sample) filters change with
every batch, so for those workloads the step also builds them: per order, the register summary, the
FiLM-modulated SIREN taps of every (b, d) and their spectra, then the operator reading one filter per
(b, d); the filter network is then the dominant kernel and the roofline object reports it.  Workloads
that start from token-major inputs run the input projection (a matrix-core GEMM that writes v, x_1..x_N
channel-major) before the operator in every step; the roofline object then reports the projection.

The streaming-decode workload times one token of every (b, d) row per step (hyena_decode_step, with the
FFT convolution of the stored prefix at each block start), over a whole sequence by default.

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
    plus the filter read once in its smallest exact form (fp32 taps), shared by the B rows of a channel
    (one filter per row for input-dependent filters)."""
    filters = w.B * w.D if w.filter == "film" else w.D
    return 3 * w.elem_bytes * w.tokens_channels + 4 * filters * w.support


def floor_bytes_per_step(w) -> int:
    """All orders fused on chip: read v and the N gates, write y, plus the N filters (fp32 taps)."""
    filters = w.B * w.D if w.filter == "film" else w.D
    return (w.order + 2) * w.elem_bytes * w.tokens_channels + 4 * w.order * filters * w.support


def uses_matrix_cores(w) -> bool:
    """Causal, bf16 storage, L = 8192, rows in pairs of one channel, order <= 3: the library's matrix-core
    kernel."""
    return (w.mode == "causal" and w.dtype == "bf16" and w.dims[0] == 8192 and w.B % 2 == 0
            and w.filter != "film" and w.order <= 3)


def uses_long_matrix_cores(w) -> bool:
    """Causal, bf16 storage, L = 2^15 .. 2^17, order <= 3: the library's long-row matrix-core kernels (column
    passes on the vector units, 16384-point planes on the matrix cores)."""
    return (w.ndim == 1 and w.mode == "causal" and w.dtype == "bf16" and w.dims[0] in (1 << 15, 1 << 16, 1 << 17)
            and w.filter != "film" and w.order <= 3)


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
    if uses_long_matrix_cores(w):
        return f"mfma_long_L{L}_bf16"
    return f"conv1d_L{L}_{w.dtype}_gate{circ}" if single_launch_per_order(w) else f"fourstep_L{L}_{w.dtype}"


def arithmetic(w) -> str:
    if uses_matrix_cores(w):
        return ("matrix-core DFT steps on fp16 operands (DFT matrices, spectrum copy and transform data rounded to "
                "fp16 after exact power-of-two range scaling; the first product reads the bf16 input exactly), "
                "fp32 accumulation; twiddle and spectral products in packed fp16; u_1 passes between the orders in fp16")
    if uses_long_matrix_cores(w):
        return ("column passes in fp32; 16384-point plane transforms on the matrix cores with fp16 operands and "
                "fp32 accumulation; planes stored between passes as fp16 with power-of-two block scales; split "
                "coefficients fp16, twiddle / split / spectral products in packed fp16; u_i between orders in fp32")
    if w.dtype == "bf16" and not single_launch_per_order(w) and w.ndim == 1:
        return "fp32; transform intermediate stored between passes as fp16 with power-of-two block scales"
    if w.dtype == "bf16":
        return "fp32 (bf16 only for the stored v, x_i and y)"
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


def film_network_flops(w) -> float:
    """Algorithmic flops of one input-dependent filter launch (one order, every sample): per sample and
    tap, layer 1 (n coordinates -> H), layer 2 (H -> H) and the read-out (H -> D), two flops per
    multiply-add; the sines, the FiLM affine maps and the window are not counted."""
    return 2.0 * w.B * w.support * w.hidden * (w.ndim + w.hidden + w.D)


def host_cores() -> int:
    """Cores this process may run on (the GPU machine's own share)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _pool_rows(work, rows, budget_s: float, cores: int):
    """Run work(row) for rows on a pool of `cores` threads (numpy's FFTs release the interpreter lock, so the
    threads run in parallel; BLAS is limited to one thread per call), in rounds of 4*cores rows until
    budget_s of wall time has passed.  Returns (rows done, wall seconds)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    done, wall = 0, 0.0
    with threadpool_limits(1), ThreadPoolExecutor(cores) as ex:
        for k in range(0, len(rows), 4 * cores):
            batch = rows[k:k + 4 * cores]
            t0 = time.perf_counter()
            list(ex.map(work, batch))
            wall += time.perf_counter() - t0
            done += len(batch)
            print(f"cpu baseline: {done} rows, {wall:.1f} s", file=sys.stderr, flush=True)
            if wall >= budget_s:
                break
    return done, wall


def _cpu_result(w, done, wall, cores, what):
    return {"value": done * w.points / wall, "unit": "tokens·channels/s", "cores": cores, "kind": "oracle",
            "cpu_model": host_cpu_model(),
            "sample": f"{done} of {w.B * w.D} (b,d) rows of the same workload, order {w.order}, {what}; float64 numpy "
                      f"FFT convolution on a pool of {cores} threads (one per core of this process's CPU set; numpy's "
                      f"FFT releases the interpreter lock), {wall:.1f} s of wall time"}


def cpu_baseline_film(w, v, xs, fparams, reg, budget_s: float):
    """The oracle on whole (b, d) volumes/rows of the input-dependent workload: per row, both orders'
    filters for that (b, d) (register summary, FiLM-SIREN on every tap, window) and then the operator,
    all inside the timed part, as the GPU step builds its filters per call."""
    from oracle import hyena_oracle as orc
    rows = [tuple(r) for r in hi.sample_rows(w, 4096, seed=99)]
    circ = w.mode == "circular"
    if w.ndim == 1:
        offs = np.arange(w.dims[0])[:, None]
        c = offs / w.dims[0]
        shape = (1, w.dims[0])
    else:
        n = w.dims[0]
        offs = orc.filter_offsets_3d_circular(n) if circ else orc.filter_offsets_3d(n)
        c = offs.astype(np.float64) / n
        m = n if circ else 2 * n - 1
        shape = (1, m, m, m)

    def work(bd):
        b, d = bd
        hs = []
        for p in fparams:
            z = orc.register_summary(reg[b:b + 1], p["q"])[0]
            pd = dict(p, A3=p["A3"][d:d + 1], a3=p["a3"][d:d + 1], sigma=p["sigma"][d:d + 1])
            k = (orc.film_siren(c, z, pd).T * orc.gaussian_window(c, pd["sigma"]))[0]
            if w.ndim == 3 and circ:
                hc = np.zeros((n, n, n))
                ri = offs % n
                hc[ri[:, 0], ri[:, 1], ri[:, 2]] = k
                k = hc
            hs.append(k.reshape(shape))
        if w.ndim == 1:
            orc.hyena_operator_rows(v[b, d][None], [x[b, d][None] for x in xs], hs, circular=circ)
        else:
            orc.hyena_operator_3d(v[b, d][None], [x[b, d][None] for x in xs], hs, circular=circ)

    cores = host_cores()
    done, wall = _pool_rows(work, rows, budget_s, cores)
    return _cpu_result(w, done, wall, cores, "each with its own input-dependent filters built inside the timed part")


def cpu_baseline(w, v, xs, params, budget_s: float, proj_inputs=None):
    """The oracle as it stands on whole (b, d) rows (volumes) of the same workload, on a thread pool over the
    host's cores, until about budget_s seconds of wall time; the filters of the sampled channels are built
    before the timed part (as the GPU's spectra are).  With proj_inputs (x, W_proj, bias) each row's v,
    x_1..x_N come from the oracle's projection of the token-major input, inside the timed part."""
    from oracle import hyena_oracle as orc
    from threadpoolctl import threadpool_limits
    cores = host_cores()
    rows = [tuple(r) for r in hi.sample_rows(w, 4096, seed=99)]
    circ = w.mode == "circular"
    need = sorted({d for _, d in rows})
    t0 = time.perf_counter()
    with threadpool_limits(cores):
        if w.ndim == 1:
            built = [orc.implicit_filter_1d(p, w.dims[0], channels=need) for p in params]
        elif circ:
            built = [orc.implicit_filter_3d_circular(p, w.dims[0], channels=need) for p in params]
        else:
            built = [orc.implicit_filter_3d(p, w.dims[0], channels=need) for p in params]
    print(f"cpu baseline: filters of {len(need)} channels built in {time.perf_counter() - t0:.1f} s",
          file=sys.stderr, flush=True)
    index = {d: k for k, d in enumerate(need)}

    def work(bd):
        b, d = bd
        hs = [h[index[d]][None] for h in built]
        if proj_inputs is not None:
            xt, Wp, bp = proj_inputs
            sel = [j * w.D + d for j in range(w.order + 1)]
            rows_p = orc.input_projection(xt[b:b + 1], Wp[sel], bp[sel], w.order)     # each [1, 1, L]
            orc.hyena_operator_rows(rows_p[0][0], [r[0] for r in rows_p[1:]], hs, circular=circ)
        elif w.ndim == 1:
            orc.hyena_operator_rows(v[b, d][None], [x[b, d][None] for x in xs], hs, circular=circ)
        else:
            orc.hyena_operator_3d(v[b, d][None], [x[b, d][None] for x in xs], hs, circular=circ)

    done, wall = _pool_rows(work, rows, budget_s, cores)
    what = "each row projected from the token-major input" if proj_inputs is not None else "filters prebuilt"
    return _cpu_result(w, done, wall, cores, what)


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


DECODE_METRIC = "Hyena streaming decode tokens·channels/s (one token of every (b, d) row per step), 1 GPU"


def decode_bytes_per_launch(w, n_avg: float) -> float:
    """Algorithmic bytes of one token-step launch: per row read v_t and the N gates, write y_t, append the
    N inputs to the histories, read the N prefix contributions, and read n in-block history values per order;
    per channel read n taps per order (shared by the B rows)."""
    rows, N = w.B * w.D, w.order
    return 4.0 * (rows * ((N + 1) + 1 + N + N) + N * n_avg * (rows + w.D))


def cpu_baseline_decode(w, v, xs, params, budget_s: float):
    """The oracle's token-by-token evaluation on whole rows of the same workload (batches of 8 rows, all L
    tokens each), filters built outside the timed part, until about budget_s seconds of oracle time."""
    from threadpoolctl import threadpool_limits
    from oracle import hyena_oracle as orc
    L = w.dims[0]
    rows = hi.sample_rows(w, 4096, seed=99)
    n_done, t_used = 0, 0.0
    with threadpool_limits(1):
        for k in range(0, len(rows), 8):
            sel = rows[k:k + 8]
            ds = [d for _, d in sel]
            hs = [orc.implicit_filter_1d(p, L, channels=ds) for p in params]
            t0 = time.perf_counter()
            orc.hyena_decode_stream(np.stack([v[b, d] for b, d in sel]),
                                    [np.stack([x[b, d] for b, d in sel]) for x in xs], hs)
            t_used += time.perf_counter() - t0
            n_done += len(sel)
            print(f"cpu baseline (decode): {n_done} rows, {t_used:.1f} s", file=sys.stderr, flush=True)
            if t_used >= budget_s:
                break
    return {"value": n_done * L / t_used, "unit": "tokens·channels/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_done} of {w.B * w.D} (b,d) rows of the same workload decoded token by token over all "
                      f"{L} positions (float64 numpy, direct causal sums, one core), filters prebuilt; "
                      f"{t_used:.1f} s"}


def run_decode(args, w, torch, hy, _lib):
    """Streaming decode: a step is one token of every (b, d) row through hyena_decode_step, the prefix
    convolutions of block starts included; step k decodes position k mod L of a sequence that restarts
    (hyena_decode_reset, inside the step) at position 0."""
    import ctypes
    L, B, D, N = w.dims[0], w.B, w.D, w.order
    block = args.decode_block or w.decode_block
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    pd = [{k: torch.from_numpy(a).to(dev) for k, a in p.items()} for p in params]
    taps = [torch.empty((D, L), dtype=torch.float32, device=dev) for _ in pd]
    spectra = [hy.filter_gen(p, (L,), h_time=h) for p, h in zip(pd, taps)]
    # token-major inputs [L, B, D] resident in HBM; outputs likewise
    vt = torch.from_numpy(np.ascontiguousarray(np.moveaxis(v, -1, 0))).to(dev)
    xt = [torch.from_numpy(np.ascontiguousarray(np.moveaxis(x, -1, 0))).to(dev) for x in xs]
    yt = torch.empty_like(vt)
    nbytes = _lib.decode_state_bytes(N, B, D, L)
    state = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    # argument marshalling done once: per-position pointer tables for the C call
    lib = _lib.lib()
    P = ctypes.c_void_p
    tok = B * D * 4
    ta = (P * N)(*[h.data_ptr() for h in taps])
    sa = (P * N)(*[sp.data_ptr() for sp in spectra])
    xa = [(P * N)(*[x.data_ptr() + t * tok for x in xt]) for t in range(L)]
    vb, yb, sb, hs = vt.data_ptr(), yt.data_ptr(), state.data_ptr(), stream.cuda_stream

    def step(k):
        t = k % L
        if t == 0:
            st = lib.hyena_decode_reset(N, B, D, L, sb, nbytes, hs)
            if st:
                raise _lib.HyenaError(st, "hyena_decode_reset")
        st = lib.hyena_decode_step(N, B, D, L, block, t, _lib.F32, _lib.CAUSAL, vb + t * tok, xa[t], ta, sa, yb + t * tok, sb,
                                   nbytes, hs)
        if st:
            raise _lib.HyenaError(st, "hyena_decode_step")

    k = 0
    for _ in range(args.warmup):
        step(k)
        k += 1
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step(k)
        k += 1
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    event_ms = ev0.elapsed_time(ev1) / args.steps

    # the token kernel alone: the positions of one block after its start (no prefix convolution), launched
    # back to back; and the prefix convolutions of one block start
    kb = (k // L + 1) * L + block             # a block start of the next sequence, past position 0
    while k < kb:
        step(k)
        k += 1
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record(stream)
    step(k)                                   # block start: prefix convolutions + token kernel
    k += 1
    e1.record(stream)
    for _ in range(block - 1):
        step(k)
        k += 1
    e2.record(stream)
    torch.cuda.synchronize()
    token_ms = e1.elapsed_time(e2) / (block - 1)
    boundary_ms = e0.elapsed_time(e1)
    # the prompt path for context: the whole sequence as one prompt (hyena_decode_prefill, P = L)
    yp = torch.empty((B, D, L), dtype=torch.float32, device=dev)
    vd = torch.from_numpy(v).to(dev)
    xd = [torch.from_numpy(x).to(dev) for x in xs]
    for _ in range(2):
        hy.decode_prefill(vd, xd, spectra, state, L, block, y=yp)
    e3, e4 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e3.record(stream)
    for _ in range(5):
        hy.decode_prefill(vd, xd, spectra, state, L, block, y=yp)
    e4.record(stream)
    torch.cuda.synchronize()
    prefill_ms = e3.elapsed_time(e4) / 5
    del yp, vd, xd
    n_avg = block / 2.0                       # in-block positions summed, averaged over the block
    bytes_launch = decode_bytes_per_launch(w, n_avg)
    achieved = bytes_launch / (token_ms / 1e3) / 1e9
    rows = B * D
    out = {
        "metric": DECODE_METRIC,
        "value": rows / (ms_per_step / 1e3),
        "unit": "tokens·channels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded activations, Xavier-uniform filter networks; see hyena_inputs)",
        "config": {"workload": w.name, "order": N, "B": B, "D": D, "grid": [L], "boundary": "causal",
                   "storage": "f32", "arithmetic": "fp32", "decode_block": block, "alpha_range": [w.alpha_lo, w.alpha_hi],
                   "inputs": f"numpy default_rng([{w.index}, stream]): stream 0 activations, stream 1 filter parameters"},
        "us_per_token_step": 1e3 * ms_per_step,
        "event_ms_per_step": event_ms,
        "token_kernel_ms": token_ms,
        "block_start_ms": boundary_ms,
        "prefill_whole_sequence_ms": prefill_ms,
        "state_bytes": nbytes,
        "roofline": {"bound": "hbm", "kernel": f"k_decode_step<{N}> (one token of every row, launched back to back)",
                     "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": None, "launch_ms": token_ms, "alg_bytes_per_launch": bytes_launch,
                     "note": "a few MB per launch: the step is bound by launch and memory latency, not bandwidth"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w, v, xs, params, args.cpu_budget)
    return out


def build_step(w, torch, hy, _lib, dev):
    """Device inputs of workload w and the step closure (one pass of the whole hot path over the batch).
    Returns a dict: step, y, v, xs, params (host), filter_gen_ms, and the extra pieces of the input-dependent
    and projection workloads."""
    film = w.filter == "film"
    proj = w.d_model > 0
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    v, xs = hi.draw_activations(w)
    params = hi.draw_film_params(w) if film else hi.draw_filter_params(w)
    reg = hi.draw_registers(w) if film else None
    vd = torch.from_numpy(v).to(dev).to(dt)
    xd = [torch.from_numpy(x).to(dev).to(dt) for x in xs]
    pd = [{k: torch.from_numpy(a).to(dev) for k, a in p.items()} for p in params]
    y = torch.empty_like(vd)
    mode = {"causal": _lib.CAUSAL, "linear": _lib.LINEAR, "circular": _lib.CIRCULAR}[w.mode]
    ws_n = _lib.workspace_bytes(w.order, w.B, w.D, w.dims, _lib.BF16 if w.dtype == "bf16" else _lib.F32, mode)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    r = {"v": v, "xs": xs, "params": params, "reg": reg, "y": y, "vd": vd, "xd": xd, "pd": pd, "mode": mode,
         "film": film, "proj": proj, "filter_gen_ms": None}
    if proj:
        xtok, Wp, bp = hi.draw_projection(w)
        r["proj_inputs"] = (xtok, Wp, bp)
        xtd = torch.from_numpy(xtok).to(dev).to(dt)
        Wpd = torch.from_numpy(Wp).to(dev).to(dt)
        bpd = torch.from_numpy(bp).to(dev)
        pouts = [vd] + xd                       # the projection writes v, x_1..x_N in place of the drawn ones
        r["projection"] = lambda: hy.projection(xtd, Wpd, w.order, bias=bpd, outs=pouts)
    if film:
        # per-sample filters: rebuilt inside every step into preallocated spectra and workspace
        regd = torch.from_numpy(reg).to(dev)
        op_mode = mode | _lib.PER_SAMPLE
        spectra = [torch.empty(_lib.spectrum_bytes(w.dims, w.B * w.D, op_mode), dtype=torch.uint8, device=dev)
                   for _ in pd]
        fws = torch.empty(_lib.film_filter_workspace_bytes(w.B, w.dims, w.D, mode), dtype=torch.uint8, device=dev)
        r["film_taps_only"] = lambda taps: hy.film_filter_gen(pd[0], regd, w.dims, h_time=taps, mode=mode, ws=fws,
                                                              taps_only=True)

        def step():
            for p, sp in zip(pd, spectra):
                hy.film_filter_gen(p, regd, w.dims, spectrum=sp, mode=mode, ws=fws)
            hy.operator(vd, xd, spectra, y=y, ws=ws, mode=op_mode)
    else:
        # filter spectra (cached per grid): timed separately
        spectra = [hy.filter_gen(p, w.dims, mode=mode) for p in pd]
        torch.cuda.synchronize()
        fg = []
        for _ in range(3):
            t0 = time.perf_counter()
            spectra = [hy.filter_gen(p, w.dims, mode=mode) for p in pd]
            torch.cuda.synchronize()
            fg.append(time.perf_counter() - t0)
        r["filter_gen_ms"] = 1e3 * min(fg)
        projection = r.get("projection")

        def step():
            if projection is not None:
                projection()
            hy.operator(vd, xd, spectra, y=y, ws=ws, mode=mode)
    r["step"] = step
    return r


def time_back_to_back(torch, stream, step, n: int) -> float:
    """ms per step over n steps launched back to back, bracketed by two events on the launch stream."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(n):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / n


def time_evicted(torch, stream, step, n: int, scratch, blocks: int = 5) -> list:
    """ms per step with nothing of the step's working set cached: in each of `blocks` blocks, n/blocks steps
    each launched right after a write of `scratch` (several times the 256 MB memory-side cache), timed as a
    whole, minus the same number of scratch writes alone; both bracketed by two events on the launch stream,
    so no event sits between a write and its step.  A step's cost includes the write-back of its outputs
    that the next eviction forces.  Returns the per-block figures."""
    per = max(1, n // blocks)
    out = []
    for k in range(-1, blocks):                 # block -1: untimed, settles the writes and the clocks
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(per):
            scratch.fill_(float(i))
            step()
        ev[1].record(stream)
        for i in range(per):
            scratch.fill_(float(i))
        ev[2].record(stream)
        torch.cuda.synchronize()
        if k >= 0:
            out.append((ev[0].elapsed_time(ev[1]) - ev[1].elapsed_time(ev[2])) / per)
    return out


def sampled_parity(w, v, xs, params, y_host, rows):
    """Per-row relative L2 error of the GPU output against the oracle on the given (b, d) rows (1-D workloads
    with shared filters), computed on a thread pool: {"rows", "max", "median", "tolerance"}."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    from oracle import hyena_oracle as orc
    circ = w.mode == "circular"
    chans = sorted({int(d) for _, d in rows})
    with threadpool_limits(host_cores()):
        hs = [orc.implicit_filter_1d(p, w.dims[0], channels=chans) for p in params]
    index = {d: k for k, d in enumerate(chans)}

    def one(bd):
        b, d = int(bd[0]), int(bd[1])
        ref = orc.hyena_operator_rows(v[b, d][None], [x[b, d][None] for x in xs], [h[index[d]][None] for h in hs],
                                      circular=circ)
        return orc.rel_l2_per_row(np.asarray(y_host[b, d], np.float64)[None], ref)[0]
    with threadpool_limits(1), ThreadPoolExecutor(host_cores()) as ex:
        e = np.asarray(list(ex.map(one, rows)))
    return {"rows": int(len(rows)), "of_rows": w.B * w.D, "max": float(e.max()), "median": float(np.median(e)),
            "tolerance": 2e-2 if w.dtype == "bf16" else 1e-4,
            "measure": "relative L2 error per (b, d) row against the float64 oracle"}


TIMING_NOTE = ("ms_per_step: the timed steps run each right after a 1 GiB device write that evicts the 256 MB "
               "memory-side cache, so every input comes from HBM; per block of steps, the time of the writes and "
               "steps together minus that of the writes alone (two HIP events on the launch stream per block), "
               "median over 5 blocks; warm: the same step launched back to back (its working set partly cached)")


def measure(w, args, torch, hy, _lib, dev, stream, scratch, warm_steps: int, cold_steps: int, parity_rows=None):
    """The timed part for one workload: W warm-up steps, cold_steps evicted steps (the headline), then
    warm_steps back-to-back steps.  Returns (result dict, build dict)."""
    r = build_step(w, torch, hy, _lib, dev)
    step = r["step"]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    cold = time_evicted(torch, stream, step, cold_steps, scratch)
    cold_ms = float(np.median(cold))
    res_blocks = [float(c) for c in cold]
    warm_ms = time_back_to_back(torch, stream, step, warm_steps) if warm_steps > 0 else None
    T = w.tokens_channels
    alg_step = algorithmic_bytes_per_order(w) * w.order
    res = {"ms_per_step": cold_ms, "value": T / (cold_ms / 1e3),
           "hbm_gbps_alg": alg_step / (cold_ms / 1e3) / 1e9,
           "hbm_frac_alg": alg_step / (cold_ms / 1e3) / 1e9 / PEAK_HBM_GBPS,
           "cold_ms_blocks": res_blocks}
    if warm_ms is not None:
        res["warm"] = {"ms_per_step": warm_ms, "steps": warm_steps, "value": T / (warm_ms / 1e3),
                       "hbm_frac_alg": alg_step / (warm_ms / 1e3) / 1e9 / PEAK_HBM_GBPS}
    if parity_rows is not None and not r["film"] and not r["proj"] and w.ndim == 1:
        y_host = r["y"].float().cpu().numpy()
        res["parity"] = sampled_parity(w, r["v"], r["xs"], r["params"], y_host, parity_rows)
    return res, r


def torch_fft_context(w, r, torch, hy, stream, ours_warm_ms):
    """Context only, not a code path of the library: the same operator written with torch.fft (the platform's
    FFT library) on the same GPU -- rfft of the zero-padded rows, product with the 2L-point filter spectra,
    irfft, cut to L, gate, every order, fp32 -- timed back to back like `warm`.  The filter taps come from
    hyena_filter_gen, their spectra from torch.fft (not timed)."""
    L = w.dims[0]
    n = 2 * L
    spec = []
    for p in r["pd"]:
        taps = torch.empty((w.D, L), dtype=torch.float32, device=r["vd"].device)
        hy.filter_gen(p, w.dims, h_time=taps)
        spec.append(torch.fft.rfft(taps, n=n))
    vd, xd = r["vd"], r["xd"]

    def step():
        u = vd.float()
        for H, x in zip(spec, xd):
            u = torch.fft.irfft(torch.fft.rfft(u, n=n) * H, n=n)[..., :L] * x.float()
        return u.to(vd.dtype)
    for _ in range(3):
        step()
    ms = time_back_to_back(torch, stream, step, 10)
    del spec
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "ours_warm_ms_per_step": ours_warm_ms,
            "ratio": ms / ours_warm_ms if ours_warm_ms else None,
            "note": "context only: torch.fft rfft / product / irfft / gate in fp32 per order on the same GPU, "
                    "back to back (10 steps); not a code path of the library and not a target"}


def roofline_object(w, launch_ms: float, per_step: bool):
    """HBM roofline of the dominant kernel (per_step: the whole step, when a step is several kernels)."""
    key = kernel_key(w)
    if per_step:
        alg = algorithmic_bytes_per_order(w) * w.order
        achieved = alg / (launch_ms / 1e3) / 1e9
        return {"bound": "hbm", "kernel": key + " (whole step)", "achieved": achieved, "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS, "traffic": load_traffic(key),
                "launch_ms": launch_ms, "alg_bytes_per_step": alg}
    if uses_matrix_cores(w):
        alg = algorithmic_bytes_per_order(w) * w.order        # one launch runs every order
        floor = floor_bytes_per_step(w)
        achieved = alg / (launch_ms / 1e3) / 1e9
        return {"bound": "hbm", "kernel": key, "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBPS, "traffic": load_traffic(key), "launch_ms": launch_ms,
                "alg_bytes_per_launch": alg, "floor_bytes_per_launch": floor,
                "floor_frac": floor / (launch_ms / 1e3) / 1e9 / PEAK_HBM_GBPS}
    alg = algorithmic_bytes_per_order(w) * w.order            # one fused launch runs every order
    achieved = alg / (launch_ms / 1e3) / 1e9
    return {"bound": "hbm", "kernel": key, "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS, "traffic": load_traffic(key), "launch_ms": launch_ms,
            "alg_bytes_per_launch": alg}


def config_block(w):
    return {"workload": w.name, "order": w.order, "B": w.B, "D": w.D, "grid": list(w.dims), "boundary": w.mode,
            "storage": w.dtype, "arithmetic": arithmetic(w), "alpha_range": [w.alpha_lo, w.alpha_hi],
            "inputs": f"numpy default_rng([{w.index}, stream]): stream 0 activations, stream 1 filter parameters"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps, each after a cache-evicting write (default 200; decode: one whole "
                         "sequence, L tokens)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps first (default 100; decode: 512 tokens)")
    ap.add_argument("--warm-steps", type=int, default=1000,
                    help="back-to-back steps timed after the evicted ones (reported as warm; 0 skips them).  The "
                         "GPU reaches steady clocks only under sustained load: 0.1 s of back-to-back work measures "
                         "that state")
    ap.add_argument("--workload", type=int, default=1, help="index into hyena_inputs.WORKLOADS")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle wall time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy", action="store_true", help="skip the device copy-bandwidth probe")
    ap.add_argument("--no-torch-fft", action="store_true",
                    help="skip the torch.fft context line (1-D causal workloads with shared filters)")
    ap.add_argument("--no-parity", action="store_true", help="skip the oracle check of the bench's own output")
    ap.add_argument("--no-config3", action="store_true",
                    help="skip the nested line of the 2^20-sample fp32 workload (the second target configuration)")
    ap.add_argument("--evict-mb", type=int, default=1024, help="size of the cache-evicting write")
    ap.add_argument("--decode-block", type=int, default=0, help="decode workloads: tokens per prefix block "
                                                               "(0: the workload's own)")
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
    if args.steps is None:
        args.steps = w.dims[0] if w.decode_block else 200
    if args.warmup is None:
        args.warmup = 512 if w.decode_block else 100
    if w.decode_block:
        out = run_decode(args, w, torch, hy, _lib)
        print(json.dumps(out), flush=True)
        return
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    scratch = torch.empty(args.evict_mb << 18, dtype=torch.float32, device=dev)
    parity_rows = None
    if not args.no_parity and w.ndim == 1 and w.filter != "film" and not w.d_model:
        parity_rows = [tuple(r) for r in hi.sample_rows(w, 4096, seed=5)]      # every row up to 4096
    t_wall = time.perf_counter()
    res, r = measure(w, args, torch, hy, _lib, dev, stream, scratch, args.warm_steps, args.steps, parity_rows)
    film, proj = r["film"], r["proj"]
    out = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "tokens·channels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded activations, Xavier-uniform filter networks; see hyena_inputs)",
        "config": config_block(w),
        "timing": TIMING_NOTE,
        "hbm_gbps_alg": res["hbm_gbps_alg"],
        "hbm_frac_alg": res["hbm_frac_alg"],
        "filter_gen_ms": r["filter_gen_ms"],
    }
    for k in ("warm", "parity", "cold_ms_blocks"):
        if k in res:
            out[k] = res[k]
    if film:
        out["data"] = ("synthetic (seeded activations and register activations, SIREN/FiLM parameters drawn as in "
                       "hyena_inputs.draw_film_params)")
        out["config"].pop("alpha_range")
        out["config"].update({"filters": "input-dependent: one FiLM-SIREN filter per (b, d), rebuilt every step",
                              "registers": w.registers, "hidden": w.hidden,
                              "sigma_range": [w.sigma_lo, w.sigma_hi],
                              "inputs": f"numpy default_rng([{w.index}, stream]): stream 0 activations, stream 1 "
                                        f"filter parameters, stream 2 register activations"})
        # dominant kernel: the filter network, timed alone (taps only: register summary + taps launch)
        taps = torch.empty((w.B, w.D, w.support), dtype=torch.float32, device=dev)
        launch_ms = time_back_to_back(torch, stream, lambda: r["film_taps_only"](taps), 20)
        del taps
        flops = film_network_flops(w)
        tf = flops / (launch_ms / 1e3) / 1e12
        out["roofline"] = {"bound": "mfma", "kernel": f"k_film_tiles ({'3-D' if w.ndim == 3 else '1-D'} taps, "
                                                      f"input-dependent filter network)",
                           "achieved": tf, "peak": 157.3, "unit": "TFLOP/s", "frac": tf / 157.3, "traffic": None,
                           "launch_ms": launch_ms, "alg_flops_per_launch": flops,
                           "note": "peak: dense fp32 matrix-core 157.3 TFLOP/s (layer 2 and the read-out run on "
                                   "fp32 matrix cores; layer 1, the sines and the window on the vector units); "
                                   "the launch time includes the register-summary kernel"}
        out["filter_share_of_step"] = w.order * launch_ms / res["ms_per_step"]
    else:
        # filter network (a GEMM pair per position) for all orders; the time includes the spectrum build
        net_flop = 2.0 * w.order * w.support * w.hidden * (w.features + w.D)
        fg = r["filter_gen_ms"]
        out["filter_gen"] = {"ms": fg, "network_gflop": net_flop / 1e9,
                             "achieved_tflops": net_flop / (fg / 1e3) / 1e12, "peak_tflops": 157.3,
                             "note": "all orders; network flops over the whole filter build (spectra included)"}
    if proj:
        # dominant kernel of the new step part: the projection GEMM, timed alone
        proj_ms = time_back_to_back(torch, stream, r["projection"], 50)
        flops = 2.0 * w.B * w.points * w.d_model * (w.order + 1) * w.D
        peak = 2500.0 if w.dtype == "bf16" else 157.3
        tf = flops / (proj_ms / 1e3) / 1e12
        out["roofline"] = {"bound": "mfma", "kernel": f"k_proj<{'bf16' if w.dtype == 'bf16' else 'fp32'}> "
                                                      f"(input projection, channel-major outputs)",
                           "achieved": tf, "peak": peak, "unit": "TFLOP/s", "frac": tf / peak, "traffic": None,
                           "launch_ms": proj_ms, "alg_flops_per_launch": flops,
                           "note": f"dense {'bf16' if w.dtype == 'bf16' else 'fp32'} matrix-core peak"}
        out["projection_share_of_step"] = proj_ms / res["ms_per_step"]
        out["config"]["d_model"] = w.d_model
        out["config"]["inputs"] += ", stream 3 token-major inputs and W_proj"
    if not (film or proj):
        one_launch = (uses_matrix_cores(w) or single_launch_per_order(w)) and w.order <= 8
        out["roofline"] = roofline_for = roofline_object(w, res["ms_per_step"], per_step=not one_launch)
        roofline_for["timing"] = ("cold step, one launch per step (see timing)" if one_launch else
                                  "cold step (see timing)")
    if (not args.no_torch_fft and w.ndim == 1 and w.mode == "causal" and not (film or proj)
            and res.get("warm") is not None):
        out["torch_fft_context"] = torch_fft_context(w, r, torch, hy, stream, res["warm"]["ms_per_step"])
    host = (r["v"], r["xs"], r["params"], r["reg"], r.get("proj_inputs"))
    del r
    if args.workload == 1 and not args.no_config3:
        # the second target configuration: the 2^20-sample fp32 order-2 workload, in the same run
        w3 = hi.WORKLOADS[3]
        torch.cuda.empty_cache()
        rows3 = [tuple(x) for x in hi.sample_rows(w3, 16, seed=5)] if not args.no_parity else None
        res3, r3 = measure(w3, argparse.Namespace(warmup=3), torch, hy, _lib, dev, stream, scratch, 10, 10, rows3)
        del r3
        torch.cuda.empty_cache()
        res3["steps"] = 10
        res3["config"] = config_block(w3)
        res3["roofline"] = roofline_object(w3, res3["ms_per_step"], per_step=True)
        res3["tokens_channels_per_step"] = w3.tokens_channels
        out["config3"] = res3
    del scratch
    if not args.no_copy:
        out["copy_gbps"] = copy_bandwidth(torch, dev)
    if not args.no_cpu_baseline:
        v, xs, params, reg, proj_inputs = host
        out["cpu_baseline"] = (cpu_baseline_film(w, v, xs, params, reg, args.cpu_budget) if film else
                               cpu_baseline(w, v, xs, params, args.cpu_budget, proj_inputs=proj_inputs))
    out["bench_wall_s"] = time.perf_counter() - t_wall
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
