"""GPU parity of the periodic (circular) 1-D mode against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import hyena_inputs as hi
from oracle import hyena_oracle as orc
from gpu_util import (BF16_TOL, FP32_TOL, all_row_errors, oracle_rows_1d, params_to_dev, rel_err_rows,
                      report_errors, run_hip_operator, say, to_dev)

pytestmark = pytest.mark.gpu

CIRCULAR_L = [2048, 4096, 8192, 16384, 32768]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import attention_free_long_implicit_amd as hy
    hy.lib()
    return torch


def _w(L, B=3, D=7, dtype="f32", order=2):
    return hi.WORKLOADS[0].with_(B=B, D=D, dims=(L,), dtype=dtype, order=order, mode="circular")


@pytest.mark.parametrize("L", CIRCULAR_L)
def test_circular_filter_taps_and_spectrum(torch_cuda, L):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    D = 12
    w = _w(L, D=D)
    p = hi.draw_filter_params(w, seed=300 + L)[0]
    say(f"circular filter_gen L={L} D={D}")
    h = torch.empty((D, L), dtype=torch.float32, device="cuda")
    spec = hy.filter_gen(params_to_dev(p), (L,), h_time=h, mode=hy.CIRCULAR)
    assert spec.numel() == D * (L // 2) * 8
    H = hy.spectrum_export(spec, (L,), D, mode=hy.CIRCULAR)
    torch.cuda.synchronize()
    ref = orc.implicit_filter_1d(p, L)                       # one period: the causal taps t = 0..L-1
    assert rel_err_rows(h.cpu().numpy(), ref).max() < 1e-5
    Href = np.fft.rfft(ref)                                  # L-point transform, no padding
    Hg = H.cpu().numpy().astype(np.complex128)
    assert Hg.shape == Href.shape
    e = np.linalg.norm(Hg - Href, axis=1) / np.linalg.norm(Href, axis=1)
    assert e.max() < 1e-5, e.max()


@pytest.mark.parametrize("L", CIRCULAR_L)
@pytest.mark.parametrize("gate", [False, True])
def test_circular_fftconv_fp32(torch_cuda, L, gate):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = _w(L)
    rng = np.random.default_rng(L + 7)
    u = rng.standard_normal(w.shape).astype(np.float32)
    g = rng.standard_normal(w.shape).astype(np.float32)
    p = hi.draw_filter_params(w, seed=L)[0]
    say(f"circular fftconv fp32 L={L} gate={gate}")
    spec = hy.filter_gen(params_to_dev(p), (L,), mode=hy.CIRCULAR)
    y = hy.fftconv(to_dev(u, torch.float32), spec, to_dev(g, torch.float32) if gate else None, mode=hy.CIRCULAR)
    torch.cuda.synchronize()
    h = orc.implicit_filter_1d(p, L)                         # [D, L]
    ref = orc.circular_conv_fft(u.astype(np.float64), h[None])
    if gate:
        ref = ref * g
    e = rel_err_rows(y.cpu().numpy(), ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < FP32_TOL, e.max()


def test_circular_wraps_around(torch_cuda):
    # an impulse at the last sample: the periodic result is the filter advanced by one step,
    # c[t] = h[(t + 1) mod L]; a causal convolution would be zero before the last sample
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L, D = 4096, 5
    w = _w(L, B=1, D=D)
    p = hi.draw_filter_params(w, seed=77)[0]
    h = torch.empty((D, L), dtype=torch.float32, device="cuda")
    spec = hy.filter_gen(params_to_dev(p), (L,), h_time=h, mode=hy.CIRCULAR)
    u = np.zeros(w.shape, np.float32)
    u[:, :, L - 1] = 1.0
    say("circular impulse at the last sample")
    y = hy.fftconv(to_dev(u, torch.float32), spec, None, mode=hy.CIRCULAR)
    torch.cuda.synchronize()
    want = np.roll(h.cpu().numpy().astype(np.float64), -1, axis=1)[None]
    e = rel_err_rows(y.cpu().numpy(), want)
    assert e.max() < FP32_TOL, e.max()


@pytest.mark.parametrize("L", CIRCULAR_L)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_circular_operator_order2(torch_cuda, L, dtype):
    w = _w(L, B=2, D=5, dtype=dtype)
    v, xs = hi.draw_activations(w, seed=L)
    params = hi.draw_filter_params(w, seed=L + 1)
    import attention_free_long_implicit_amd as hy
    say(f"circular operator order 2 L={L} {dtype}")
    y = run_hip_operator(w, v, xs, params, mode=hy.CIRCULAR)
    rows = [(b, d) for b in range(w.B) for d in range(w.D)]
    ref = oracle_rows_1d(w, v, xs, params, rows, circular=True)
    got = np.stack([y[b, d] for b, d in rows])
    e = rel_err_rows(got, ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < (BF16_TOL if dtype == "bf16" else FP32_TOL), e.max()


# ---------------------------------------------------------------- periodic 3-D (64^3)
N3 = 64


def _w3(B=1, D=3, dtype="f32", order=2):
    return hi.WORKLOADS[4].with_(B=B, D=D, dtype=dtype, order=order, mode="circular")


def test_circular3d_filter_taps_and_spectrum(torch_cuda):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    D = 2
    w = _w3(D=D)
    p = hi.draw_filter_params(w, seed=51)[0]
    say("periodic 3-D filter taps + spectrum, D=2")
    h = torch.empty((D, N3, N3, N3), dtype=torch.float32, device="cuda")   # offsets from -32 (index - 32)
    spec = hy.filter_gen(params_to_dev(p), (N3, N3, N3), h_time=h, mode=hy.CIRCULAR)
    assert spec.numel() == D * N3 * N3 * 33 * 8
    H = hy.spectrum_export(spec, (N3, N3, N3), D, mode=hy.CIRCULAR)
    torch.cuda.synchronize()
    ref = orc.implicit_filter_3d_circular(p, N3)                             # index r mod 64
    centred = np.roll(ref, N3 // 2, axis=(1, 2, 3))                          # index r + 32
    e = rel_err_rows(h.cpu().numpy(), centred, point_axes=3)
    assert e.max() < 1e-5, e.max()
    Href = np.fft.rfftn(ref, axes=(-3, -2, -1))
    Hg = H.cpu().numpy().astype(np.complex128)
    assert Hg.shape == Href.shape
    e = np.sqrt(np.sum(np.abs(Hg - Href) ** 2, axis=(1, 2, 3)) / np.sum(np.abs(Href) ** 2, axis=(1, 2, 3)))
    assert e.max() < 2e-5, e.max()


@pytest.mark.parametrize("gate", [False, True])
def test_circular3d_fftconv_fp32(torch_cuda, gate):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    B, D = 1, 3
    w = _w3(B=B, D=D)
    rng = np.random.default_rng(52)
    u = rng.standard_normal(w.shape).astype(np.float32)
    g = rng.standard_normal(w.shape).astype(np.float32)
    p = hi.draw_filter_params(w, seed=52)[0]
    say(f"periodic 3-D fftconv fp32 gate={gate}")
    spec = hy.filter_gen(params_to_dev(p), (N3, N3, N3), mode=hy.CIRCULAR)
    ws = torch.empty(2 * N3 * N3 * 33 * 8, dtype=torch.uint8, device="cuda")   # two volumes per chunk: 2 chunks
    y = hy.operator(to_dev(u, torch.float32), [to_dev(g, torch.float32)], [spec], ws=ws, mode=hy.CIRCULAR) \
        if gate else hy.fftconv(to_dev(u, torch.float32), spec, mode=hy.CIRCULAR)
    torch.cuda.synchronize()
    h = orc.implicit_filter_3d_circular(p, N3)
    ref = orc.circular_conv3d_fft(u[0].astype(np.float64), h)
    if gate:
        ref = ref * g[0]
    e = rel_err_rows(y.cpu().numpy()[0], ref, point_axes=3)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < 2e-5, e.max()


def test_circular3d_wraps_around(torch_cuda):
    # impulse at the last voxel: c[p] = h[(p + 1) mod 64] on every axis
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    D = 2
    w = _w3(D=D)
    p = hi.draw_filter_params(w, seed=53)[0]
    spec = hy.filter_gen(params_to_dev(p), (N3, N3, N3), mode=hy.CIRCULAR)
    u = np.zeros(w.shape, np.float32)
    u[:, :, -1, -1, -1] = 1.0
    say("periodic 3-D impulse at the last voxel")
    y = hy.fftconv(to_dev(u, torch.float32), spec, mode=hy.CIRCULAR)
    torch.cuda.synchronize()
    want = np.roll(orc.implicit_filter_3d_circular(p, N3), -1, axis=(1, 2, 3))
    e = rel_err_rows(y.cpu().numpy()[0], want, point_axes=3)
    assert e.max() < 2e-5, e.max()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_circular3d_operator_order2(torch_cuda, dtype):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = _w3(B=2, D=3, dtype=dtype)
    v, xs = hi.draw_activations(w, seed=54)
    params = hi.draw_filter_params(w, seed=55)
    say(f"periodic 3-D operator order 2 {dtype}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    spectra = [hy.filter_gen(params_to_dev(p), w.dims, mode=hy.CIRCULAR) for p in params]
    y = hy.operator(to_dev(v, dt), [to_dev(x, dt) for x in xs], spectra, mode=hy.CIRCULAR)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().reshape((-1,) + w.dims)
    hs = [orc.implicit_filter_3d_circular(p, N3) for p in params]
    vv = v.reshape((-1,) + w.dims)
    ref = orc.hyena_operator_3d(vv, [x.reshape((-1,) + w.dims) for x in xs],
                                [np.tile(h, (w.B, 1, 1, 1)) for h in hs], circular=True)
    e = rel_err_rows(y, ref, point_axes=3)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < (BF16_TOL if dtype == "bf16" else FP32_TOL), e.max()


@pytest.mark.timeout(600)
def test_operator_periodic_f32_B4_D768_L8192_all_rows(torch_cuda):
    """The periodic 1-D workload at full size (B=4, D=768, L=8192, fp32), as the bench runs it: every row
    against the oracle."""
    w = hi.WORKLOADS[5]
    import attention_free_long_implicit_amd as hy
    say("operator workload 5 (periodic 1-D, full size)")
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    y = run_hip_operator(w, v, xs, params, mode=hy.CIRCULAR, host_dtype=np.float32)
    assert np.all(np.isfinite(y))
    e = all_row_errors(w, v, xs, params, y, circular=True)
    report_errors("workload 5", e)
    assert e.max() < FP32_TOL, e.max()


@pytest.mark.timeout(600)
def test_operator3d_periodic_f32_D128_64cubed_all_channels(torch_cuda):
    """The periodic 3-D workload at full size (B=1, D=128, 64^3, fp32): every volume against the oracle."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[6]
    say("operator workload 6 (periodic 3-D, full size)")
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    spectra = [hy.filter_gen(params_to_dev(p), w.dims, mode=hy.CIRCULAR) for p in params]
    y = hy.operator(to_dev(v, torch.float32), [to_dev(x, torch.float32) for x in xs], spectra, mode=hy.CIRCULAR)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.all(np.isfinite(y))
    e = all_row_errors(w, v, xs, params, y, circular=True)
    report_errors("workload 6", e)
    assert e.max() < FP32_TOL, e.max()


# ---------------------------------------------------------------- long periodic rows (multi-pass)
LONG_L = [1 << 16, 1 << 17, 1 << 21]


@pytest.mark.parametrize("L", [1 << 16, 1 << 21])
def test_circular_long_filter_spectrum(torch_cuda, L):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    D = 3
    w = _w(L, D=D)
    p = hi.draw_filter_params(w, seed=400 + L % 97)[0]
    say(f"periodic multi-pass filter_gen L={L}")
    spec = hy.filter_gen(params_to_dev(p), (L,), mode=hy.CIRCULAR)
    H = hy.spectrum_export(spec, (L,), D, mode=hy.CIRCULAR)
    torch.cuda.synchronize()
    Href = np.fft.rfft(orc.implicit_filter_1d(p, L))
    Hg = H.cpu().numpy().astype(np.complex128)
    e = np.linalg.norm(Hg - Href, axis=1) / np.linalg.norm(Href, axis=1)
    assert e.max() < 1e-5, e.max()


@pytest.mark.parametrize("L", LONG_L)
def test_circular_long_operator_fp32_chunked(torch_cuda, L):
    # B*D = 3 rows through a workspace of two rows: chunks of 2 and 1
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = _w(L, B=1, D=3)
    v, xs = hi.draw_activations(w, seed=L % 1009)
    params = hi.draw_filter_params(w, seed=L % 1013)
    say(f"periodic multi-pass operator fp32 L={L}")
    spectra = [hy.filter_gen(params_to_dev(p), (L,), mode=hy.CIRCULAR) for p in params]
    ws = torch.empty(2 * (L // 2) * 8, dtype=torch.uint8, device="cuda")
    y = hy.operator(to_dev(v, torch.float32), [to_dev(x, torch.float32) for x in xs], spectra, ws=ws,
                    mode=hy.CIRCULAR)
    torch.cuda.synchronize()
    rows = [(0, d) for d in range(w.D)]
    ref = oracle_rows_1d(w, v, xs, params, rows, circular=True)
    e = rel_err_rows(y.cpu().numpy()[0], ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < FP32_TOL, e.max()


@pytest.mark.parametrize("L", [1 << 16, 1 << 17])
def test_circular_long_operator_bf16(torch_cuda, L):
    w = _w(L, B=2, D=2, dtype="bf16")
    v, xs = hi.draw_activations(w, seed=L % 1019)
    params = hi.draw_filter_params(w, seed=L % 1021)
    import attention_free_long_implicit_amd as hy
    say(f"periodic multi-pass operator bf16 L={L}")
    y = run_hip_operator(w, v, xs, params, mode=hy.CIRCULAR)
    rows = [(b, d) for b in range(w.B) for d in range(w.D)]
    ref = oracle_rows_1d(w, v, xs, params, rows, circular=True)
    got = np.stack([y[b, d] for b, d in rows])
    e = rel_err_rows(got, ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < BF16_TOL, e.max()


def test_circular_long_wraps_around(torch_cuda):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L, D = 1 << 16, 2
    w = _w(L, B=1, D=D)
    p = hi.draw_filter_params(w, seed=78)[0]
    h = torch.empty((D, L), dtype=torch.float32, device="cuda")
    spec = hy.filter_gen(params_to_dev(p), (L,), h_time=h, mode=hy.CIRCULAR)
    u = np.zeros(w.shape, np.float32)
    u[:, :, L - 1] = 1.0
    say("periodic multi-pass impulse at the last sample")
    y = hy.fftconv(to_dev(u, torch.float32), spec, None, mode=hy.CIRCULAR)
    torch.cuda.synchronize()
    want = np.roll(h.cpu().numpy().astype(np.float64), -1, axis=1)[None]
    e = rel_err_rows(y.cpu().numpy(), want)
    assert e.max() < FP32_TOL, e.max()
