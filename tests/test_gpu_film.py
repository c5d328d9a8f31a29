"""GPU parity of the input-dependent (per-sample) filters: register summary, FiLM-modulated SIREN taps,
their spectra, and the operator reading one filter per (b, d), against the oracle."""
import numpy as np
import pytest

import hyena_inputs as hi
from oracle import hyena_oracle as orc
from gpu_util import BF16_TOL, FP32_TOL, rel_err_rows, say, to_dev

pytestmark = pytest.mark.gpu
N = 64


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import attention_free_long_implicit_amd as hy
    hy.lib()
    return torch


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _film(w, seed):
    return hi.draw_film_params(w, seed=seed), hi.draw_registers(w, seed=seed)


def _mode(w):
    import attention_free_long_implicit_amd as hy
    return {"causal": hy.CAUSAL, "linear": hy.LINEAR, "circular": hy.CIRCULAR}[w.mode]


def _hip_operator(w, v, xs, params, reg):
    import torch
    import attention_free_long_implicit_amd as hy
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    mode = _mode(w)
    spectra = [hy.film_filter_gen({k: _dev(a) for k, a in p.items()}, _dev(reg), w.dims, mode=mode) for p in params]
    y = hy.operator(to_dev(v, dt), [to_dev(x, dt) for x in xs], spectra, mode=mode | hy.PER_SAMPLE)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _oracle_filters(w, params, reg):
    if w.ndim == 1:
        return [orc.input_dependent_filter_1d(p, reg, w.dims[0]) for p in params]
    return [orc.input_dependent_filter_3d(p, reg, N, circular=w.mode == "circular") for p in params]


@pytest.mark.parametrize("L", [1024, 4096])
def test_film_taps_1d_match_oracle(torch_cuda, L):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[7].with_(B=3, D=24, dims=(L,), mode="causal", registers=5)
    (p,), reg = hi.draw_film_params(w.with_(order=1), seed=11), hi.draw_registers(w, seed=11)
    say(f"FiLM taps 1-D L={L} B=3 D=24")
    h = torch.empty((3, 24, L), dtype=torch.float32, device="cuda")
    hy.film_filter_gen({k: _dev(a) for k, a in p.items()}, _dev(reg), (L,), h_time=h)
    torch.cuda.synchronize()
    ref = orc.input_dependent_filter_1d(p, reg, L)
    e = rel_err_rows(h.cpu().numpy(), ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < 2e-5, e.max()
    # the samples' filters differ (the registers differ), so a shared-filter bug would show
    assert np.max(np.abs(ref[0] - ref[1])) > 1e-2


@pytest.mark.parametrize("circular", [False, True])
def test_film_taps_3d_sampled_offsets(torch_cuda, circular):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    B, D = 2, 6
    w = hi.WORKLOADS[7].with_(B=B, D=D, order=1, mode="circular" if circular else "linear")
    (p,), reg = hi.draw_film_params(w, seed=12), hi.draw_registers(w, seed=12)
    m = N if circular else 2 * N - 1
    say(f"FiLM taps 3-D circular={circular} B={B} D={D}")
    h = torch.empty((B, D, m, m, m), dtype=torch.float32, device="cuda")
    hy.film_filter_gen({k: _dev(a) for k, a in p.items()}, _dev(reg), (N, N, N), h_time=h, mode=_mode(w))
    torch.cuda.synchronize()
    got = h.cpu().numpy().reshape(B, D, -1)
    offs = orc.filter_offsets_3d_circular(N) if circular else orc.filter_offsets_3d(N)
    sel = np.unique(np.concatenate([np.arange(0, len(offs), 101), [0, len(offs) - 1, len(offs) // 2]]))
    c = offs[sel].astype(np.float64) / N
    idx = sel                     # h_time holds tap index = offset + (n-1) (zero-padded) or + n/2 (periodic)
    z = orc.register_summary(reg, p["q"])
    win = orc.gaussian_window(c, p["sigma"])
    worst = 0.0
    for b in range(B):
        ref = orc.film_siren(c, z[b], p).T * win                          # [D, S]
        e = rel_err_rows(got[b][:, idx], ref)
        worst = max(worst, e.max())
    say(f"  max rel err {worst:.3e} over {len(sel)} offsets")
    assert worst < 2e-5, worst


def test_film_spectrum_matches_fft_of_taps(torch_cuda):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L, B, D = 2048, 2, 8
    w = hi.WORKLOADS[7].with_(B=B, D=D, dims=(L,), mode="causal", order=1, registers=3)
    (p,), reg = hi.draw_film_params(w, seed=13), hi.draw_registers(w, seed=13)
    say("FiLM spectrum export, L=2048")
    h = torch.empty((B, D, L), dtype=torch.float32, device="cuda")
    spec = hy.film_filter_gen({k: _dev(a) for k, a in p.items()}, _dev(reg), (L,), h_time=h)
    H = hy.spectrum_export(spec, (L,), B * D, mode=hy.CAUSAL | hy.PER_SAMPLE)
    torch.cuda.synchronize()
    ref = np.fft.rfft(h.cpu().numpy().astype(np.float64).reshape(B * D, L), 2 * L)
    Hg = H.cpu().numpy().astype(np.complex128)
    e = np.sqrt(np.sum(np.abs(Hg - ref) ** 2, axis=1) / np.sum(np.abs(ref) ** 2, axis=1))
    assert e.max() < 2e-6, e.max()


@pytest.mark.parametrize("mode,L,dtype,B,D", [
    ("causal", 1024, "f32", 3, 8),          # one workgroup per row
    ("causal", 8192, "bf16", 2, 6),         # bf16, even B: still the fp32 engine (filters differ per row)
    ("causal", 32768, "f32", 2, 3),         # multi-pass
    ("causal", 65536, "bf16", 2, 3),        # multi-pass bf16: fp16 intermediate, fp32 spectra of B*D filters
    ("circular", 4096, "f32", 2, 5),
    ("circular", 65536, "f32", 3, 2),       # periodic multi-pass
])
def test_per_sample_operator_1d(torch_cuda, mode, L, dtype, B, D):
    w = hi.WORKLOADS[7].with_(B=B, D=D, dims=(L,), mode=mode, dtype=dtype, registers=4)
    params, reg = _film(w, seed=L + B)
    v, xs = hi.draw_activations(w, seed=L + B)
    say(f"per-sample operator 1-D {mode} L={L} {dtype} B={B} D={D}")
    y = _hip_operator(w, v, xs, params, reg)
    ref = orc.hyena_operator_rows(v, xs, _oracle_filters(w, params, reg), circular=mode == "circular")
    e = rel_err_rows(y, ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < (BF16_TOL if dtype == "bf16" else FP32_TOL), e.max()


@pytest.mark.parametrize("mode", ["linear", "circular"])
def test_per_sample_operator_3d(torch_cuda, mode):
    B, D = 2, 2
    w = hi.WORKLOADS[7].with_(B=B, D=D, mode=mode)
    params, reg = _film(w, seed=21)
    v, xs = hi.draw_activations(w, seed=21)
    say(f"per-sample operator 3-D {mode} B={B} D={D}")
    y = _hip_operator(w, v, xs, params, reg)
    hs = [h.reshape((B * D,) + h.shape[2:]) for h in _oracle_filters(w, params, reg)]
    ref = orc.hyena_operator_3d(v.reshape(B * D, N, N, N), [x.reshape(B * D, N, N, N) for x in xs], hs,
                                circular=mode == "circular")
    e = rel_err_rows(y.reshape(B * D, N, N, N), ref, point_axes=3)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < FP32_TOL, e.max()


def test_per_sample_full_workload_sampled_volumes(torch_cuda):
    """The 3-D input-dependent workload at full size (B = 2, D = 128, 64^3, order 2): a few (b, d)
    volumes against the oracle."""
    w = hi.WORKLOADS[7]
    params, reg = _film(w, seed=None)
    v, xs = hi.draw_activations(w)
    say(f"per-sample operator full size {w.name}")
    y = _hip_operator(w, v, xs, params, reg)
    r = orc.filter_offsets_3d(N)
    c = r.astype(np.float64) / N
    m = 2 * N - 1
    worst = 0.0
    for b, d in [(0, 0), (1, 127), (1, 45)]:
        hs = []
        for p in params:
            z = orc.register_summary(reg, p["q"])[b]
            pd = dict(p, A3=p["A3"][d:d + 1], a3=p["a3"][d:d + 1], sigma=p["sigma"][d:d + 1])
            hs.append((orc.film_siren(c, z, pd).T * orc.gaussian_window(c, pd["sigma"])).reshape(1, m, m, m))
        ref = orc.hyena_operator_3d(v[b, d][None], [x[b, d][None] for x in xs], hs)
        e = rel_err_rows(y[b, d][None], ref, point_axes=3)[0]
        say(f"  (b={b}, d={d}) rel err {e:.3e}")
        worst = max(worst, e)
    assert worst < FP32_TOL, worst


@pytest.mark.parametrize("mode,dims", [("causal", (8192,)), ("causal", (65536,)), ("linear", (64, 64, 64))])
def test_per_sample_with_equal_registers_matches_shared_filters_bitwise(torch_cuda, mode, dims):
    """Every sample given the same registers: the per-(b, d) path must reproduce, bit for bit, the shared
    path fed with one sample's spectra (same kernels, filter index b*D + d against d)."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    B, D = 2, 4
    w = hi.WORKLOADS[7].with_(B=B, D=D, dims=dims, mode=mode)
    params, reg = _film(w, seed=31)
    reg[1] = reg[0]
    v, xs = hi.draw_activations(w, seed=31)
    md = _mode(w)
    say(f"per-sample vs shared, {mode} {dims}")
    pdev = [{k: _dev(a) for k, a in p.items()} for p in params]
    sp_ps = [hy.film_filter_gen(p, _dev(reg), dims, mode=md) for p in pdev]
    sp_one = [hy.film_filter_gen(p, _dev(reg[:1]), dims, mode=md) for p in pdev]
    vd, xd = to_dev(v, torch.float32), [to_dev(x, torch.float32) for x in xs]
    y_ps = hy.operator(vd, xd, sp_ps, mode=md | hy.PER_SAMPLE)
    y_sh = hy.operator(vd, xd, sp_one, mode=md)
    torch.cuda.synchronize()
    assert torch.equal(y_ps, y_sh)


@pytest.mark.parametrize("mode,L,dtype,B,D,gate", [
    ("causal", 4096, "bf16", 3, 4, True),       # odd B with bf16 storage
    ("causal", 1 << 20, "f32", 2, 2, True),     # the longest causal rows, multi-pass
    ("circular", 8192, "f32", 2, 3, False),     # no gate
])
def test_per_sample_fftconv(torch_cuda, mode, L, dtype, B, D, gate):
    """hyena_fftconv with one filter per (b, d): y = gate * (h_{b,d} conv u) row by row."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[7].with_(B=B, D=D, dims=(L,), mode=mode, dtype=dtype, order=1, registers=3)
    params, reg = _film(w, seed=L + D)
    v, xs = hi.draw_activations(w, seed=L + D)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    md = _mode(w)
    say(f"per-sample fftconv {mode} L={L} {dtype} B={B} D={D} gate={gate}")
    sp = hy.film_filter_gen({k: _dev(a) for k, a in params[0].items()}, _dev(reg), (L,), mode=md)
    y = hy.fftconv(to_dev(v, dt), sp, gate=to_dev(xs[0], dt) if gate else None, mode=md | hy.PER_SAMPLE)
    torch.cuda.synchronize()
    h = _oracle_filters(w, params, reg)[0]
    conv = orc.circular_conv_fft if mode == "circular" else orc.causal_conv_fft
    ref = conv(v.astype(np.float64), h)
    if gate:
        ref = ref * xs[0]
    e = rel_err_rows(y.float().cpu().numpy().astype(np.float64), ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < (BF16_TOL if dtype == "bf16" else FP32_TOL), e.max()
