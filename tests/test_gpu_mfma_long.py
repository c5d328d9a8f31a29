"""The long-row matrix-core kernels (bf16 storage, L = 2^15 .. 2^17, every row packed on its own): against the
oracle, rows of very different magnitudes, chunking and streams, routing, the allocation-free entry point."""
import numpy as np
import pytest

import hyena_inputs as hi
from oracle import hyena_oracle as orc
from gpu_util import (BF16_TOL, all_row_errors, params_to_dev, rel_err_rows, report_errors, say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import attention_free_long_implicit_amd as hy
    hy.lib()
    return torch


def _bf16_inputs(torch, rng, shape):
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("L", [1 << 15, 1 << 16, 1 << 17])
@pytest.mark.parametrize("B", [1, 2, 3])
@pytest.mark.parametrize("gate", [False, True])
def test_long_fftconv(torch_cuda, L, B, gate):
    """hyena_fftconv, one order, with and without a gate: every row against the oracle's causal convolution of
    the bf16-rounded inputs."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    D = 3
    w = hi.WORKLOADS[2].with_(B=B, D=D, dims=(L,), order=1)
    rng = np.random.default_rng(L % 1009 + 7 * B + gate)
    u = _bf16_inputs(torch, rng, (B, D, L))
    g = _bf16_inputs(torch, rng, (B, D, L))
    p = hi.draw_filter_params(w, seed=21 + B)[0]
    say(f"long-row matrix-core fftconv L={L} B={B} gate={gate}")
    spec = hy.filter_gen(params_to_dev(p), (L,))
    y = hy.fftconv(u.cuda(), spec, gate=g.cuda() if gate else None)
    torch.cuda.synchronize()
    h = orc.implicit_filter_1d(p, L)
    un = u.float().numpy().astype(np.float64).reshape(-1, L)
    ref = orc.causal_conv_fft(un, np.tile(h, (B, 1)))
    if gate:
        ref = ref * g.float().numpy().astype(np.float64).reshape(-1, L)
    e = rel_err_rows(y.float().cpu().numpy().reshape(-1, L), ref)
    say(f"  max rel err {e.max():.3e} median {np.median(e):.3e}")
    assert e.max() < BF16_TOL


@pytest.mark.parametrize("L", [1 << 15, 1 << 16, 1 << 17])
@pytest.mark.parametrize("order", [2, 3])
@pytest.mark.parametrize("decay", ["none", "slow"])
def test_long_operator_orders(torch_cuda, L, order, decay):
    """Orders 2 and 3 (u_i kept in fp32 between them inside the column pass) with no decay window (alpha = 0,
    the longest-reaching filters) and with the slowly decaying filters of the 65536-sample workload: every row
    against the oracle."""
    lo, hi_ = (0.0, 0.0) if decay == "none" else (0.1, 2.0)
    w = hi.WORKLOADS[2].with_(B=2, D=6, dims=(L,), order=order, alpha_lo=lo, alpha_hi=hi_)
    v, xs = hi.draw_activations(w, seed=40 + order)
    params = hi.draw_filter_params(w, seed=40 + order)
    say(f"long-row matrix cores: order {order}, L={L}, B=2, D=6, decay {decay}")
    from gpu_util import run_hip_operator
    y = run_hip_operator(w, v, xs, params, host_dtype=np.float32)
    e = all_row_errors(w, v, xs, params, y)
    report_errors(f"order {order} L={L} {decay}", e)
    assert e.max() < BF16_TOL


def test_long_chunks_and_streams(torch_cuda):
    """Ten rows run as one chunk, as chunks of one row cycling over two streams (a workspace sized for two
    rows), and as chunks of four, four and two rows over two streams (a workspace sized for eight): bitwise
    equal, since no row's arithmetic depends on its chunk."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L, B, D, order = 1 << 15, 2, 5, 3
    w = hi.WORKLOADS[2].with_(B=B, D=D, dims=(L,), order=order)
    v, xs = hi.draw_activations(w, seed=51)
    params = hi.draw_filter_params(w, seed=51)
    say("long-row matrix cores: chunks and streams")
    spectra = [hy.filter_gen(params_to_dev(p), (L,)) for p in params]
    vd = to_dev(v, torch.bfloat16)
    xd = [to_dev(x, torch.bfloat16) for x in xs]
    y = hy.operator(vd, xd, spectra)
    outs = []
    for d_room in (1, 4):
        n = hy.workspace_bytes(order, B, d_room, (L,), hy.BF16)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        outs.append(hy.operator(vd, xd, spectra, ws=ws))
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, y)
    e = all_row_errors(w, v, xs, params, y.float().cpu().numpy())
    report_errors("chunks", e)
    assert e.max() < BF16_TOL


def test_long_rows_of_very_different_magnitudes(torch_cuda):
    """Every row is transformed on its own with its own power-of-two block scales: in one channel, rows scaled
    by 2^-50 and 2^40, a single impulse and an all-zero row each stay within the tolerance of the oracle (the
    zero row gives exact zeros), and a NaN in one row leaves every other row bitwise unchanged."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L, B, D = 1 << 16, 5, 2
    w = hi.WORKLOADS[2].with_(B=B, D=D, dims=(L,), order=2)
    v, xs = hi.draw_activations(w, seed=61)
    v[0, 1] *= 2.0 ** -50
    v[1, 1] *= 2.0 ** 40
    v[2, 1] = 0.0
    v[2, 1, L // 3] = 3.0
    v[3, 1] = 0.0
    params = hi.draw_filter_params(w, seed=61)
    say("long-row matrix cores: rows 2^-50 .. 2^40, an impulse and a zero row in one channel")
    spectra = [hy.filter_gen(params_to_dev(p), (L,)) for p in params]
    vd = to_dev(v, torch.bfloat16)
    xd = [to_dev(x, torch.bfloat16) for x in xs]
    y = hy.operator(vd, xd, spectra)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y[3, 1]).item() == 0
    vr = vd.float().cpu().numpy()
    xr = [x.float().cpu().numpy() for x in xd]
    e = all_row_errors(w, vr, xr, params, y.float().cpu().numpy())
    zero = 3 * D + 1
    keep = [i for i in range(B * D) if i != zero]
    report_errors("rows of very different magnitudes", e[keep])
    assert e[keep].max() < BF16_TOL
    vn = vd.clone()
    vn[4, 0, L // 2] = float("nan")
    yn = hy.operator(vn, xd, spectra)
    torch.cuda.synchronize()
    assert torch.isnan(yn[4, 0]).any()
    yf, ynf = y.reshape(B * D, L), yn.reshape(B * D, L)
    others = [i for i in range(B * D) if i != 4 * D + 0]
    assert torch.equal(ynf[others], yf[others])


def test_long_routing(torch_cuda):
    """Which plan a bf16 call at L = 65536 takes: orders up to 3 with 16-byte-aligned activations take the
    long-row matrix-core kernels, so they differ from the same call with a misaligned v (the vector-unit
    multi-pass plan), both within the tolerance of each other; order 4 takes the vector-unit plan whatever
    the alignment (bitwise equal)."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L = 1 << 16
    for order in (3, 4):
        w = hi.WORKLOADS[2].with_(B=2, D=2, dims=(L,), order=order)
        v, xs = hi.draw_activations(w, seed=70 + order)
        params = hi.draw_filter_params(w, seed=70 + order)
        spectra = [hy.filter_gen(params_to_dev(p), w.dims) for p in params]
        vd = to_dev(v, torch.bfloat16)
        xd = [to_dev(x, torch.bfloat16) for x in xs]
        ya = hy.operator(vd, xd, spectra)
        buf = torch.empty(v.size + 1, dtype=torch.bfloat16, device="cuda")
        vm = buf[1:].view(v.shape)
        vm.copy_(vd)
        assert vm.data_ptr() % 16 != 0
        ym = hy.operator(vm, xd, spectra)
        torch.cuda.synchronize()
        say(f"routing order {order}")
        if order == 4:
            assert torch.equal(ya, ym)
        else:
            assert not torch.equal(ya, ym)
            e = rel_err_rows(ym.float().cpu().numpy().reshape(-1, L), ya.float().cpu().numpy().reshape(-1, L))
            assert e.max() < BF16_TOL


def test_long_noalloc_matches_operator(torch_cuda):
    """hyena_operator_noalloc (the library's own scratch, chunks cycling over two streams) against
    hyena_operator with a caller's workspace, twice in a row with a smaller batch the second time: bitwise."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L, order = 1 << 16, 3
    for B, D in ((2, 160), (2, 3)):
        w = hi.WORKLOADS[2].with_(B=B, D=D, dims=(L,), order=order)
        v, xs = hi.draw_activations(w, seed=90 + D)
        params = hi.draw_filter_params(w, seed=90 + D)
        say(f"long-row noalloc B={B} D={D}")
        spectra = [hy.filter_gen(params_to_dev(p), (L,)) for p in params]
        vd = to_dev(v, torch.bfloat16)
        xd = [to_dev(x, torch.bfloat16) for x in xs]
        y = hy.operator(vd, xd, spectra)
        y2 = torch.empty_like(y)
        hy.operator_noalloc(vd, xd, spectra, y2)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)


def test_long_inplace_and_determinism(torch_cuda):
    """The operator with y = v, and fftconv with y = u and with y = gate, on the long-row matrix-core kernels
    (several chunks on two streams): bitwise equal to the out-of-place calls, which repeat bitwise."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L, B, D, order = 1 << 16, 2, 5, 2
    w = hi.WORKLOADS[2].with_(B=B, D=D, dims=(L,), order=order)
    v, xs = hi.draw_activations(w, seed=97)
    params = hi.draw_filter_params(w, seed=97)
    say("long-row matrix cores: in place and determinism")
    spectra = [hy.filter_gen(params_to_dev(p), (L,)) for p in params]
    vd = to_dev(v, torch.bfloat16)
    xd = [to_dev(x, torch.bfloat16) for x in xs]
    ws = torch.empty(hy.workspace_bytes(order, B, 2, (L,), hy.BF16), dtype=torch.uint8, device="cuda")
    y1 = hy.operator(vd, xd, spectra, ws=ws)
    y2 = hy.operator(vd, xd, spectra, ws=ws)
    vi = vd.clone()
    hy.operator(vi, xd, spectra, y=vi, ws=ws)
    c1 = hy.fftconv(vd, spectra[0], gate=xd[0])
    ui = vd.clone()
    hy.fftconv(ui, spectra[0], gate=xd[0], y=ui)
    gi = xd[0].clone()
    hy.fftconv(vd, spectra[0], gate=gi, y=gi)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y1, vi)
    assert torch.equal(c1, ui)
    assert torch.equal(c1, gi)


@pytest.mark.parametrize("L", [1 << 15, 1 << 17])
def test_long_single_row(torch_cuda, L):
    """B = D = 1: one row, one channel (the filter build stages one channel's L + 1 natural-order bins, which
    the workspace query sizes for); order 2 against the oracle."""
    w = hi.WORKLOADS[2].with_(B=1, D=1, dims=(L,), order=2)
    v, xs = hi.draw_activations(w, seed=3)
    params = hi.draw_filter_params(w, seed=3)
    say(f"long-row matrix cores: one row, L={L}")
    from gpu_util import run_hip_operator
    y = run_hip_operator(w, v, xs, params, host_dtype=np.float32)
    e = all_row_errors(w, v, xs, params, y)
    report_errors(f"one row L={L}", e)
    assert e.max() < BF16_TOL
