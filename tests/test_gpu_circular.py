"""GPU parity of the periodic (circular) 1-D mode against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import hyena_inputs as hi
from oracle import hyena_oracle as orc
from gpu_util import (BF16_TOL, FP32_TOL, oracle_rows_1d, params_to_dev, rel_err_rows, run_hip_operator, say,
                      to_dev)

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
