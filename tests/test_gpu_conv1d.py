"""GPU parity of the 1-D path (filter generation, spectrum, convolution, operator) against the
CPU oracle, through the C ABI."""
import math

import numpy as np
import pytest
import scipy.signal

import hyena_inputs as hi
from oracle import hyena_oracle as orc
from gpu_util import (BF16_TOL, FP32_TOL, all_row_errors, oracle_rows_1d, params_to_dev, rel_err_rows,
                      report_errors, run_hip_operator, say, to_dev)

pytestmark = pytest.mark.gpu

SINGLE_PASS_L = [1024, 2048, 4096, 8192, 16384]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import attention_free_long_implicit_amd as hy
    hy.lib()
    return torch


def _small(w, **kw):
    return w.with_(**kw)


@pytest.mark.parametrize("L", SINGLE_PASS_L)
def test_filter_taps_and_spectrum_match_oracle(torch_cuda, L):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = _small(hi.WORKLOADS[0], D=24, dims=(L,))
    p = hi.draw_filter_params(w, seed=100 + L)[0]
    say(f"filter_gen L={L} D=24")
    h = torch.empty((24, L), dtype=torch.float32, device="cuda")
    spec = hy.filter_gen(params_to_dev(p), (L,), h_time=h)
    H = hy.spectrum_export(spec, (L,), 24)
    torch.cuda.synchronize()
    ref = orc.implicit_filter_1d(p, L)
    e = rel_err_rows(h.cpu().numpy(), ref)
    assert e.max() < 1e-5, e.max()
    Href = np.fft.rfft(ref, 2 * L)
    Hg = H.cpu().numpy().astype(np.complex128)
    num = np.linalg.norm(Hg - Href, axis=1)
    den = np.linalg.norm(Href, axis=1)
    assert (num / den).max() < 1e-5, (num / den).max()


@pytest.mark.parametrize("L", [1024, 8192, 1 << 16])
def test_filter_taps_with_biases(torch_cuda, L):
    """Non-zero hidden-layer and output biases (b1, b2): the 1-D taps against the oracle, and the spectrum
    against numpy's FFT of the oracle's taps."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    D = 24
    w = _small(hi.WORKLOADS[0], D=D, dims=(L,))
    p = hi.draw_filter_params(w, seed=300 + L % 97)[0]
    rng = np.random.default_rng(L)
    p["b1"] = rng.uniform(-1, 1, 64).astype(np.float32)
    p["b2"] = rng.uniform(-1, 1, D).astype(np.float32)
    say(f"filter_gen with biases L={L} D={D}")
    h = torch.empty((D, L), dtype=torch.float32, device="cuda")
    spec = hy.filter_gen(params_to_dev(p), (L,), h_time=h)
    H = hy.spectrum_export(spec, (L,), D)
    torch.cuda.synchronize()
    ref = orc.implicit_filter_1d(p, L)
    e = rel_err_rows(h.cpu().numpy(), ref)
    say(f"  taps max rel err {e.max():.3e}")
    assert e.max() < 1e-5, e.max()
    Href = np.fft.rfft(ref, 2 * L)
    num = np.linalg.norm(H.cpu().numpy().astype(np.complex128) - Href, axis=1)
    assert (num / np.linalg.norm(Href, axis=1)).max() < 1e-5


@pytest.mark.parametrize("L", SINGLE_PASS_L)
@pytest.mark.parametrize("gate", [False, True])
def test_fftconv_fp32_matches_oracle(torch_cuda, L, gate):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    B, D = 3, 7     # 21 rows: not a multiple of the 8-way block remap
    w = _small(hi.WORKLOADS[0], B=B, D=D, dims=(L,))
    rng = np.random.default_rng(L)
    u = rng.standard_normal((B, D, L)).astype(np.float32)
    g = rng.standard_normal((B, D, L)).astype(np.float32)
    p = hi.draw_filter_params(w, seed=L)[0]
    say(f"fftconv fp32 L={L} gate={gate}")
    spec = hy.filter_gen(params_to_dev(p), (L,))
    y = hy.fftconv(to_dev(u, torch.float32), spec, gate=to_dev(g, torch.float32) if gate else None)
    torch.cuda.synchronize()
    h = orc.implicit_filter_1d(p, L)
    ref = orc.causal_conv_fft(u.astype(np.float64), h[None])
    if gate:
        ref = ref * g
    e = rel_err_rows(y.cpu().numpy(), ref)
    assert e.max() < 2e-5, e.max()


def test_exponential_filter_closed_form(torch_cuda):
    """W2 = 0, b2 = 1 makes h[t] = exp(-alpha t/L): the convolution is y[t] = a y[t-1] + u[t]."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L, D = 8192, 4
    alpha = np.array([0.01, 0.3, 1.0, 3.0], np.float32)
    p = dict(W1=np.zeros((64, 64), np.float32), b1=np.zeros(64, np.float32), W2=np.zeros((D, 64), np.float32),
             b2=np.ones(D, np.float32), alpha=alpha)
    u = np.random.default_rng(1).standard_normal((1, D, L)).astype(np.float32)
    say("closed form exp filter")
    spec = hy.filter_gen(params_to_dev(p), (L,))
    y = hy.fftconv(to_dev(u, torch.float32), spec).cpu().numpy()[0]
    for d in range(D):
        a = math.exp(-float(alpha[d]) / L)
        ref = scipy.signal.lfilter([1.0], [1.0, -a], u[0, d].astype(np.float64))
        assert np.linalg.norm(y[d] - ref) / np.linalg.norm(ref) < 2e-6


def test_delta_filter_gives_product_of_gates(torch_cuda):
    """A window so steep that h = b2 * delta: y = b2_1 b2_2 v x_1 x_2."""
    torch = torch_cuda
    L, D, B = 2048, 8, 2
    w = _small(hi.WORKLOADS[0], B=B, D=D, dims=(L,))
    v, xs = hi.draw_activations(w, seed=5)
    params = []
    for i, scale in enumerate((0.5, -2.0)):
        params.append(dict(W1=np.zeros((64, 64), np.float32), b1=np.zeros(64, np.float32),
                           W2=np.zeros((D, 64), np.float32), b2=np.full(D, scale, np.float32),
                           alpha=np.full(D, 200.0 * L, np.float32)))
    say("delta filter")
    y = run_hip_operator(w, v, xs, params)
    ref = -1.0 * v * xs[0] * xs[1]
    assert np.max(np.abs(y - ref)) < 1e-5 * np.max(np.abs(ref))


def test_operator_f32_B1_D16_L1024_all_rows(torch_cuda):
    w = hi.WORKLOADS[0]
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    say("operator workload 0 (order 2, L=1024, fp32), all rows")
    y = run_hip_operator(w, v, xs, params)
    rows = [(b, d) for b in range(w.B) for d in range(w.D)]
    ref = oracle_rows_1d(w, v, xs, params, rows)
    got = np.stack([y[b, d] for b, d in rows])
    e = rel_err_rows(got, ref)
    say(f"  max rel err {e.max():.3e} median {np.median(e):.3e}")
    assert e.max() < FP32_TOL


@pytest.mark.timeout(600)
def test_operator_bf16_B4_D768_L8192_all_rows(torch_cuda):
    """Workload 1 at full size (the matrix-core path, as the bench runs it): every one of the 3072 (b, d)
    rows against the oracle."""
    w = hi.WORKLOADS[1]
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    say("operator workload 1 (order 2, B=4 D=768 L=8192, bf16), all rows")
    y = run_hip_operator(w, v, xs, params, host_dtype=np.float32)
    assert np.all(np.isfinite(y))
    e = all_row_errors(w, v, xs, params, y)
    report_errors("workload 1", e)
    assert e.max() < BF16_TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_inplace_and_bitwise_determinism(torch_cuda, dtype):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = _small(hi.WORKLOADS[1], B=2, D=16, dims=(4096,), dtype=dtype)
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    say(f"in-place / determinism {dtype}")
    spectra = [hy.filter_gen(params_to_dev(p), w.dims) for p in params]
    vd = to_dev(v, dt)
    xd = [to_dev(x, dt) for x in xs]
    y1 = hy.operator(vd, xd, spectra)
    y2 = hy.operator(vd, xd, spectra)
    v_inplace = vd.clone()
    hy.operator(v_inplace, xd, spectra, y=v_inplace)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y1, v_inplace)


def test_rows_are_independent_and_causal(torch_cuda):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L = 4096
    w = _small(hi.WORKLOADS[0], B=2, D=8, dims=(L,))
    v, xs = hi.draw_activations(w, seed=9)
    params = hi.draw_filter_params(w, seed=9)
    say("row independence / causality")
    spectra = [hy.filter_gen(params_to_dev(p), w.dims) for p in params]
    xd = [to_dev(x, torch.float32) for x in xs]
    base = hy.operator(to_dev(v, torch.float32), xd, spectra).cpu().numpy()
    vn = v.copy()
    vn[1, 3, 100] = np.nan
    yn = hy.operator(to_dev(vn, torch.float32), xd, spectra).cpu().numpy()
    bad = ~np.isfinite(yn)
    assert bad[1, 3].any()
    bad[1, 3] = False
    assert not bad.any()
    np.testing.assert_array_equal(np.delete(yn.reshape(16, L), 11, axis=0), np.delete(base.reshape(16, L), 11, axis=0))
    t0 = 1500
    vp = v.copy()
    vp[0, 2, t0] += 50.0
    yp = hy.operator(to_dev(vp, torch.float32), xd, spectra).cpu().numpy()
    scale = np.max(np.abs(base[0, 2]))
    assert np.max(np.abs(yp[0, 2, :t0] - base[0, 2, :t0])) < 1e-5 * scale
    assert np.max(np.abs(yp[0, 2, t0:] - base[0, 2, t0:])) > 1e-2 * scale


@pytest.mark.parametrize("B", [2, 4])
def test_matrix_core_path_bf16_L8192(torch_cuda, B):
    """bf16 storage, L = 8192, even B: the rows of a channel are transformed in pairs on the matrix
    cores.  All rows against the oracle, plus in-place and bitwise determinism."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[1].with_(B=B, D=6, dims=(8192,))
    v, xs = hi.draw_activations(w, seed=21)
    params = hi.draw_filter_params(w, seed=21)
    say(f"matrix-core path B={B}")
    spectra = [hy.filter_gen(params_to_dev(p), w.dims) for p in params]
    vd = to_dev(v, torch.bfloat16)
    xd = [to_dev(x, torch.bfloat16) for x in xs]
    y1 = hy.operator(vd, xd, spectra)
    y2 = hy.operator(vd, xd, spectra)
    vi = vd.clone()
    hy.operator(vi, xd, spectra, y=vi)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, vi)
    rows = [(b, d) for b in range(B) for d in range(6)]
    ref = oracle_rows_1d(w, v, xs, params, rows)
    got = np.stack([y1.float().cpu().numpy()[b, d] for b, d in rows])
    e = rel_err_rows(got, ref)
    say(f"  max rel err {e.max():.3e} median {np.median(e):.3e}")
    assert e.max() < BF16_TOL
    # the same data through the fp32-arithmetic path (odd B takes it): one extra row of zeros
    vz = np.concatenate([v, np.zeros_like(v[:1])])
    xz = [np.concatenate([x, np.zeros_like(x[:1])]) for x in xs]
    y3 = hy.operator(to_dev(vz, torch.bfloat16), [to_dev(x, torch.bfloat16) for x in xz], spectra)
    torch.cuda.synchronize()
    got3 = np.stack([y3.float().cpu().numpy()[b, d] for b, d in rows])
    e2 = rel_err_rows(got3, ref)
    say(f"  odd-B (fp32 engine) max rel err {e2.max():.3e}")
    assert e2.max() < BF16_TOL


def test_matrix_core_path_misaligned_falls_back(torch_cuda):
    """Activations that are not 16-byte aligned take the fp32-arithmetic engine; results agree with
    the aligned (matrix-core) call to the bf16 tolerance."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[1].with_(B=2, D=3, dims=(8192,))
    v, xs = hi.draw_activations(w, seed=5)
    params = hi.draw_filter_params(w, seed=5)
    spectra = [hy.filter_gen(params_to_dev(p), w.dims) for p in params]
    vd = to_dev(v, torch.bfloat16)
    xd = [to_dev(x, torch.bfloat16) for x in xs]
    ya = hy.operator(vd, xd, spectra)
    n = v.size
    buf = torch.empty(n + 1, dtype=torch.bfloat16, device="cuda")
    vm = buf[1:].view(v.shape)
    vm.copy_(vd)
    assert vm.data_ptr() % 16 != 0
    ym = hy.operator(vm, xd, spectra)
    torch.cuda.synchronize()
    e = rel_err_rows(ym.float().cpu().numpy().reshape(-1, 8192), ya.float().cpu().numpy().reshape(-1, 8192))
    say(f"misaligned vs aligned max rel diff {e.max():.3e}")
    assert e.max() < BF16_TOL


def test_matrix_core_order2_fused_against_oracle(torch_cuda):
    """Order 2 at L = 8192, bf16, B = 2: both orders run in one matrix-core launch with u_1 kept on chip
    (fp16 operands, scaled by the row pair's maximum); against the oracle on every row, and within the
    bf16 tolerance of two one-order calls (which store u_1 in bf16)."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[1].with_(B=2, D=6)
    v, xs = hi.draw_activations(w, seed=31)
    params = hi.draw_filter_params(w, seed=31)
    say("fused orders on the matrix cores: order 2, B=2, D=6, L=8192, bf16")
    spectra = [hy.filter_gen(params_to_dev(p), w.dims) for p in params]
    vd = to_dev(v, torch.bfloat16)
    xd = [to_dev(x, torch.bfloat16) for x in xs]
    y = hy.operator(vd, xd, spectra)
    cur = vd
    for x, sp in zip(xd, spectra):
        cur = hy.fftconv(cur, sp, gate=x)
    torch.cuda.synchronize()
    e = all_row_errors(w, v, xs, params, y.float().cpu().numpy())
    report_errors("order 2 matrix cores", e)
    assert e.max() < BF16_TOL
    e2 = all_row_errors(w, v, xs, params, cur.float().cpu().numpy())
    report_errors("two one-order calls", e2)
    assert e2.max() < BF16_TOL


@pytest.mark.parametrize("B", [2, 4])
@pytest.mark.parametrize("gate", [False, True])
def test_matrix_core_fftconv(torch_cuda, B, gate):
    """hyena_fftconv on the matrix cores (bf16, L = 8192), with and without a gate, in both workgroup forms
    (B = 2: one row pair per workgroup; B = 4: two): every row against the oracle's gated causal
    convolution of the bf16-rounded inputs."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L, D = 8192, 10
    w = hi.WORKLOADS[1].with_(B=B, D=D, order=1)
    rng = np.random.default_rng(90 + B + 2 * gate)
    u = torch.from_numpy(rng.standard_normal((B, D, L)).astype(np.float32)).to(torch.bfloat16)
    g = torch.from_numpy(rng.standard_normal((B, D, L)).astype(np.float32)).to(torch.bfloat16)
    p = hi.draw_filter_params(w, seed=13)[0]
    say(f"matrix-core fftconv B={B} gate={gate}")
    spec = hy.filter_gen(params_to_dev(p), (L,))
    y = hy.fftconv(u.cuda(), spec, gate=g.cuda() if gate else None)
    torch.cuda.synchronize()
    h = orc.implicit_filter_1d(p, L)
    un = u.float().numpy().astype(np.float64).reshape(-1, L)
    ref = orc.causal_conv_fft(un, np.tile(h, (B, 1)))
    if gate:
        ref = ref * g.float().numpy().astype(np.float64).reshape(-1, L)
    e = rel_err_rows(y.float().cpu().numpy().reshape(-1, L), ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < BF16_TOL


@pytest.mark.parametrize("B", [2, 4])
def test_matrix_core_rows_of_very_different_magnitudes(torch_cuda, B):
    """The matrix-core kernel transforms two rows of a channel together, each with its own power-of-two scale:
    rows 2^-50 and 2^40 in one pair, a zero row paired with a normal one (exact zeros), and a normal row paired
    with a single impulse each stay within the tolerance of the oracle."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L, D = 8192, 4
    w = hi.WORKLOADS[1].with_(B=B, D=D, order=2)
    v, xs = hi.draw_activations(w, seed=44 + B)
    v[0, 0] *= 2.0 ** -50
    v[1, 0] *= 2.0 ** 40
    v[0, 1] = 0.0
    v[1, 2] = 0.0
    v[1, 2, L // 3] = 3.0
    params = hi.draw_filter_params(w, seed=44 + B)
    say(f"matrix cores, rows of very different magnitudes in a pair, B={B}")
    spectra = [hy.filter_gen(params_to_dev(p), w.dims) for p in params]
    vd = to_dev(v, torch.bfloat16)
    xd = [to_dev(x, torch.bfloat16) for x in xs]
    y = hy.operator(vd, xd, spectra)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y[0, 1]).item() == 0
    vr = vd.float().cpu().numpy()
    xr = [x.float().cpu().numpy() for x in xd]
    e = all_row_errors(w, vr, xr, params, y.float().cpu().numpy())
    keep = [i for i in range(B * D) if i != 1]
    report_errors("rows of very different magnitudes", e[keep])
    assert e[keep].max() < BF16_TOL


@pytest.mark.parametrize("order,B", [(1, 4), (3, 4), (2, 8), (3, 6)])
def test_matrix_core_workgroup_forms(torch_cuda, order, B):
    """The matrix-core kernel takes two row pairs of a channel per workgroup when B / 2 is even (B = 4, 8) and
    one otherwise (B = 6): every row against the oracle, and each row pair bitwise equal to the same pair run
    alone (B = 2, one pair per workgroup), which checks the pair / channel mapping and the per-pair scale
    reductions of the two-pair form."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[1].with_(B=B, D=12, order=order)
    v, xs = hi.draw_activations(w, seed=80 + 10 * order + B)
    params = hi.draw_filter_params(w, seed=80 + 10 * order + B)
    say(f"matrix-core workgroup forms: order {order} B={B} D=12 L=8192 bf16")
    spectra = [hy.filter_gen(params_to_dev(p), w.dims) for p in params]
    vd = to_dev(v, torch.bfloat16)
    xd = [to_dev(x, torch.bfloat16) for x in xs]
    y = hy.operator(vd, xd, spectra)
    torch.cuda.synchronize()
    e = all_row_errors(w, v, xs, params, y.float().cpu().numpy())
    report_errors(f"order {order} B={B}", e)
    assert e.max() < BF16_TOL
    for p in range(B // 2):
        sl = slice(2 * p, 2 * p + 2)
        yp = hy.operator(vd[sl], [x[sl] for x in xd], spectra)
        torch.cuda.synchronize()
        assert torch.equal(yp, y[sl]), f"row pair {p}"


@pytest.mark.parametrize("order", [3, 4, 5, 8])
@pytest.mark.parametrize("decay", ["none", "slow"])
def test_high_orders_bf16_L8192_against_oracle(torch_cuda, order, decay):
    """bf16 storage, L = 8192, even B, orders above 2: order 3 on the matrix cores (fp16 operands), 4, 5 and 8
    on the fp32 engine (every order in one launch with u_i kept in fp32, so only the bf16 stores
    round).  No decay window (alpha = 0) and the slowly decaying filters of workload 2 (alpha in [0.1, 2]):
    every row against the oracle."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    lo, hi_ = (0.0, 0.0) if decay == "none" else (0.1, 2.0)
    w = hi.WORKLOADS[1].with_(B=2, D=48, order=order, alpha_lo=lo, alpha_hi=hi_)
    v, xs = hi.draw_activations(w, seed=60 + order)
    params = hi.draw_filter_params(w, seed=60 + order)
    say(f"order {order} bf16 L=8192 B=2 D=48, decay {decay}")
    y = run_hip_operator(w, v, xs, params, host_dtype=np.float32)
    e = all_row_errors(w, v, xs, params, y)
    report_errors(f"order {order} {decay}", e)
    assert e.max() < BF16_TOL


def test_order_routing_bf16_L8192(torch_cuda):
    """Which engine an order-N call takes: order 4 runs the fp32 engine whatever the alignment (the call with
    a misaligned v, which can never take the matrix cores, is bitwise equal); orders 2 and 3 take the matrix
    cores when every pointer is 16-byte aligned (then they differ from the misaligned call, which takes the
    fp32 engine), both within the bf16 tolerance of each other."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    for order in (2, 3, 4):
        w = hi.WORKLOADS[1].with_(B=2, D=4, order=order)
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
        if order == 4:
            assert torch.equal(ya, ym)
        else:
            assert not torch.equal(ya, ym)
            e = rel_err_rows(ym.float().cpu().numpy().reshape(-1, 8192), ya.float().cpu().numpy().reshape(-1, 8192))
            assert e.max() < BF16_TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nine_orders_two_launches(torch_cuda, dtype):
    """Nine orders: eight in one launch of the fused fp32 engine, then one more (u_8 passes through y
    between the launches); against the oracle.  For fp32 storage also bitwise equal to nine one-order
    calls.  Nine convolutions in a row compound the fp32 rounding of each (the worst of these rows measures
    about 1e-4, 40 times its median), so the fp32 bound here is 1e-3 rather than the workloads' 1e-4."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[0].with_(B=1, D=3, order=9, dims=(4096,), dtype=dtype)
    rng = np.random.default_rng(7)
    v = rng.standard_normal((1, 3, 4096)).astype(np.float32)
    xs = [rng.uniform(0.5, 1.5, (1, 3, 4096)).astype(np.float32) for _ in range(9)]
    if dtype == "bf16":
        v = hi.bf16_bits_to_f32(hi.bf16_bits_rne(v))
        xs = [hi.bf16_bits_to_f32(hi.bf16_bits_rne(x)) for x in xs]
    params = hi.draw_filter_params(w.with_(order=1), seed=7) * 9
    say(f"nine orders {dtype}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    sp = hy.filter_gen(params_to_dev(params[0]), w.dims)
    vd = to_dev(v, dt)
    xd = [to_dev(x, dt) for x in xs]
    y = hy.operator(vd, xd, [sp] * 9)
    cur = vd
    for x in xd:
        cur = hy.fftconv(cur, sp, gate=x)
    torch.cuda.synchronize()
    if dtype == "f32":
        assert torch.equal(y, cur)
    e = all_row_errors(w, v, xs, params, y.float().cpu().numpy())
    report_errors(f"nine orders {dtype}", e)
    assert e.max() < (1e-3 if dtype == "f32" else BF16_TOL)


@pytest.mark.parametrize("L,B,dtype", [(1024, 1, "f32"), (8192, 1, "bf16"), (8192, 2, "bf16"), (16384, 3, "f32")])
def test_zero_input_gives_exact_zero(torch_cuda, L, B, dtype):
    """v = 0 gives y = 0 exactly on every single-pass path (fp32 engine, bf16 engine, matrix cores)."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    D = 4
    w = hi.WORKLOADS[0].with_(B=B, D=D, dims=(L,))
    p = hi.draw_filter_params(w, seed=11)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    spectra = [hy.filter_gen(params_to_dev(q), (L,)) for q in p]
    v = torch.zeros((B, D, L), dtype=tdt, device="cuda")
    xs = [torch.randn((B, D, L), device="cuda").to(tdt) for _ in p]
    y = hy.operator(v, xs, spectra)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


@pytest.mark.parametrize("L,B,dtype", [(4096, 1, "f32"), (8192, 2, "bf16")])
def test_no_decay_window(torch_cuda, L, B, dtype):
    """alpha = 0: the window is 1 over the whole length (the longest-reaching filter the method
    allows); against the oracle."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    D = 4
    w = hi.WORKLOADS[1].with_(B=B, D=D, dims=(L,), dtype=dtype)
    v, xs = hi.draw_activations(w, seed=13)
    params = hi.draw_filter_params(w, seed=13)
    for q in params:
        q["alpha"][:] = 0.0
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    spectra = [hy.filter_gen(params_to_dev(q), (L,)) for q in params]
    y = hy.operator(to_dev(v, tdt), [to_dev(x, tdt) for x in xs], spectra)
    torch.cuda.synchronize()
    rows = [(b, d) for b in range(B) for d in range(D)]
    ref = oracle_rows_1d(w, v, xs, params, rows)
    got = np.stack([y.float().cpu().numpy()[b, d] for b, d in rows])
    e = rel_err_rows(got, ref)
    say(f"no decay L={L} {dtype}: max rel err {e.max():.3e}")
    assert e.max() < (1e-3 if dtype == "f32" else BF16_TOL)


def test_operator_from_parameters_with_spectrum_cache(torch_cuda):
    """hyena() builds each order's spectrum once per grid size and reuses it: equal to operator() with spectra
    from filter_gen, two builds over two calls, a third after an in-place parameter update."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[0].with_(B=2, D=8, dims=(4096,))
    v, xs = hi.draw_activations(w, seed=91)
    params = [params_to_dev(p) for p in hi.draw_filter_params(w, seed=91)]
    cache = hy.SpectrumCache()
    vd = to_dev(v, torch.float32)
    xd = [to_dev(x, torch.float32) for x in xs]
    y1 = hy.hyena(vd, xd, params, cache=cache)
    y2 = hy.hyena(vd, xd, params, cache=cache)
    ref = hy.operator(vd, xd, [hy.filter_gen(p, w.dims) for p in params])
    torch.cuda.synchronize()
    assert cache.builds == 2
    assert torch.equal(y1, ref) and torch.equal(y2, ref)
    params[0]["alpha"].mul_(0.5)
    y3 = hy.hyena(vd, xd, params, cache=cache)
    torch.cuda.synchronize()
    assert cache.builds == 3 and not torch.equal(y3, ref)
