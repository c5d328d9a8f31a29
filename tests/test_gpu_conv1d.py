"""GPU parity of the 1-D path (filter generation, spectrum, convolution, operator) against the
CPU oracle, through the C ABI."""
import math

import numpy as np
import pytest
import scipy.signal

import hyena_inputs as hi
from oracle import hyena_oracle as orc
from gpu_util import (BF16_TOL, FP32_TOL, oracle_rows_1d, params_to_dev, rel_err_rows, run_hip_operator, say,
                      to_dev)

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


def test_operator_bf16_B4_D768_L8192_sampled_rows(torch_cuda):
    w = hi.WORKLOADS[1]
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    say("operator workload 1 (order 2, B=4 D=768 L=8192, bf16), sampled rows")
    y = run_hip_operator(w, v, xs, params)
    rows = [tuple(r) for r in hi.sample_rows(w, 24)]
    ref = oracle_rows_1d(w, v, xs, params, rows)
    got = np.stack([y[b, d] for b, d in rows])
    e = rel_err_rows(got, ref)
    say(f"  max rel err {e.max():.3e} median {np.median(e):.3e}")
    assert e.max() < BF16_TOL
    assert np.all(np.isfinite(y))


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


def test_matrix_core_orders_fused_order3(torch_cuda):
    """Order 3 at L = 8192, bf16, B = 2: the orders run back to back in one launch with u_1, u_2 kept
    on chip.  All rows against the oracle; bitwise equal to the same orders as separate one-order
    calls (each storing u_i in bf16)."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[2].with_(B=2, D=6, dims=(8192,))
    assert w.order == 3
    v, xs = hi.draw_activations(w, seed=31)
    params = hi.draw_filter_params(w, seed=31)
    say("fused orders: order 3, B=2, D=6, L=8192, bf16")
    spectra = [hy.filter_gen(params_to_dev(p), w.dims) for p in params]
    vd = to_dev(v, torch.bfloat16)
    xd = [to_dev(x, torch.bfloat16) for x in xs]
    y = hy.operator(vd, xd, spectra)
    cur = vd
    for x, sp in zip(xd, spectra):
        cur = hy.fftconv(cur, sp, gate=x)
    torch.cuda.synchronize()
    assert torch.equal(y, cur)
    rows = [(b, d) for b in range(2) for d in range(6)]
    ref = oracle_rows_1d(w, v, xs, params, rows)
    got = np.stack([y.float().cpu().numpy()[b, d] for b, d in rows])
    e = rel_err_rows(got, ref)
    say(f"  max rel err {e.max():.3e} median {np.median(e):.3e}")
    assert e.max() < BF16_TOL


def test_matrix_core_orders_beyond_one_launch(torch_cuda):
    """Nine orders: eight fused in one launch, then one more; equal to nine one-order calls."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[1].with_(B=2, D=3, dims=(8192,))
    rng = np.random.default_rng(7)
    v = rng.standard_normal((2, 3, 8192)).astype(np.float32)
    xs = [rng.uniform(0.5, 1.5, (2, 3, 8192)).astype(np.float32) for _ in range(9)]
    params = hi.draw_filter_params(w, seed=7)[0]
    sp = hy.filter_gen(params_to_dev(params), w.dims)
    vd = to_dev(v, torch.bfloat16)
    xd = [to_dev(x, torch.bfloat16) for x in xs]
    y = hy.operator(vd, xd, [sp] * 9)
    cur = vd
    for x in xd:
        cur = hy.fftconv(cur, sp, gate=x)
    torch.cuda.synchronize()
    assert torch.equal(y, cur)
    assert torch.isfinite(y.float()).all()


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
    assert e.max() < (FP32_TOL if dtype == "f32" else BF16_TOL)
