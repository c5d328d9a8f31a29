"""GPU parity of the multi-pass (four-step) 1-D path, 2^15 <= L <= 2^20, against the CPU oracle."""
import numpy as np
import pytest

import hyena_inputs as hi
from oracle import hyena_oracle as orc
from gpu_util import (BF16_TOL, FP32_TOL, all_row_errors, oracle_rows_1d, params_to_dev, rel_err_rows,
                      report_errors, run_hip_operator, say, to_dev)

pytestmark = pytest.mark.gpu

MULTI_L = [1 << 15, 1 << 16, 1 << 17, 1 << 18, 1 << 19, 1 << 20]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import attention_free_long_implicit_amd as hy
    hy.lib()
    return torch


@pytest.mark.parametrize("L", [1 << 15, 1 << 16, 1 << 20])
def test_fourstep_spectrum_matches_numpy(torch_cuda, L):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    D = 3
    w = hi.WORKLOADS[0].with_(D=D, dims=(L,))
    p = hi.draw_filter_params(w, seed=L % 997)[0]
    say(f"four-step spectrum L={L}")
    h = torch.empty((D, L), dtype=torch.float32, device="cuda")
    spec = hy.filter_gen(params_to_dev(p), (L,), h_time=h)
    H = hy.spectrum_export(spec, (L,), D)
    torch.cuda.synchronize()
    ref = orc.implicit_filter_1d(p, L)
    assert rel_err_rows(h.cpu().numpy(), ref).max() < 1e-5
    Href = np.fft.rfft(ref, 2 * L)
    Hg = H.cpu().numpy().astype(np.complex128)
    e = np.linalg.norm(Hg - Href, axis=1) / np.linalg.norm(Href, axis=1)
    assert e.max() < 2e-5, e.max()


@pytest.mark.parametrize("L", MULTI_L)
def test_fourstep_fftconv_fp32_chunked(torch_cuda, L):
    """fp32 convolution with a workspace of 3 rows, so B*D = 5 rows take two chunks (one ragged)."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    from attention_free_long_implicit_amd import _lib
    B, D = 1, 5
    w = hi.WORKLOADS[0].with_(B=B, D=D, dims=(L,))
    rng = np.random.default_rng(L % 1009)
    u = rng.standard_normal((B, D, L)).astype(np.float32)
    g = rng.standard_normal((B, D, L)).astype(np.float32)
    p = hi.draw_filter_params(w, seed=3)[0]
    say(f"four-step fftconv fp32 L={L}")
    spec = hy.filter_gen(params_to_dev(p), (L,))
    ws = torch.empty(3 * L * 8, dtype=torch.uint8, device="cuda")
    y = hy.operator(to_dev(u, torch.float32), [to_dev(g, torch.float32)], [spec], ws=ws)
    torch.cuda.synchronize()
    h = orc.implicit_filter_1d(p, L)
    ref = orc.causal_conv_fft(u.astype(np.float64), h[None]) * g
    e = rel_err_rows(y.cpu().numpy(), ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < 5e-5, e.max()


def test_fourstep_no_gate_and_chunk_invariance(torch_cuda):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L, B, D = 1 << 16, 2, 3
    w = hi.WORKLOADS[2].with_(B=B, D=D, dims=(L,))
    v, xs = hi.draw_activations(w, seed=4)
    params = hi.draw_filter_params(w, seed=4)
    say("four-step chunk invariance (bf16, order 3)")
    spectra = [hy.filter_gen(params_to_dev(p), (L,)) for p in params]
    vd = to_dev(v, torch.bfloat16)
    xd = [to_dev(x, torch.bfloat16) for x in xs]
    y_big = hy.operator(vd, xd, spectra)
    # a workspace sized for one channel's rows: one chunk per channel
    one = hy.workspace_bytes(3, B, 1, (L,), hy.BF16)
    y_one = hy.operator(vd, xd, spectra, ws=torch.empty(one, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(y_big, y_one)
    # no-gate fftconv of one channel == order-1 oracle convolution
    p1 = {k: (a[:1] if k in ("W2", "b2", "alpha") else a) for k, a in params[0].items()}
    spec1 = hy.filter_gen(params_to_dev(p1), (L,))
    u = np.ascontiguousarray(v[:1, :1]).astype(np.float32)
    c = hy.fftconv(to_dev(u, torch.float32), spec1)
    torch.cuda.synchronize()
    h0 = orc.implicit_filter_1d(params[0], L, channels=[0])
    ref = orc.causal_conv_fft(u[0].astype(np.float64), h0)
    assert rel_err_rows(c.cpu().numpy()[0], ref).max() < 5e-5


@pytest.mark.timeout(600)
def test_operator_bf16_order3_B2_D1024_L65536_all_rows(torch_cuda):
    """Workload 2 at full size: every one of the 2048 (b, d) rows against the oracle."""
    w = hi.WORKLOADS[2]
    say("operator workload 2 (order 3, B=2 D=1024 L=65536, bf16): drawing inputs")
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    say("  running HIP operator")
    y = run_hip_operator(w, v, xs, params, host_dtype=np.float32)
    assert np.all(np.isfinite(y))
    say("  oracle on every row")
    e = all_row_errors(w, v, xs, params, y)
    report_errors("workload 2", e)
    assert e.max() < BF16_TOL


@pytest.mark.timeout(600)
def test_operator_f32_B1_D256_L1M_dna_all_rows(torch_cuda):
    """Workload 3 at full size: every one of the 256 rows of 2^20 samples against the oracle."""
    w = hi.WORKLOADS[3]
    say("operator workload 3 (HyenaDNA order 2, B=1 D=256 L=1M, fp32): drawing inputs")
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    say("  running HIP operator")
    y = run_hip_operator(w, v, xs, params, host_dtype=np.float32)
    assert np.all(np.isfinite(y))
    say("  oracle on every row")
    e = all_row_errors(w, v, xs, params, y)
    report_errors("workload 3", e)
    assert e.max() < FP32_TOL


@pytest.mark.parametrize("L", [1 << 15, 1 << 16, 1 << 17, 1 << 20])
def test_fourstep_fftconv_bf16_chunked(torch_cuda, L):
    """bf16 storage (the intermediate is block-scaled fp16), five rows in chunks of two, two and one on two
    streams (a workspace sized for four rows), every multi-pass plan family (the long-row matrix-core kernels up
    to 2^17 samples, the vector-unit plan above); against the oracle on the bf16-rounded inputs."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    B, D = 1, 5
    w = hi.WORKLOADS[2].with_(B=B, D=D, dims=(L,))
    rng = np.random.default_rng(L % 1013)
    u = torch.from_numpy(rng.standard_normal((B, D, L)).astype(np.float32)).to(torch.bfloat16)
    g = torch.from_numpy(rng.standard_normal((B, D, L)).astype(np.float32)).to(torch.bfloat16)
    p = hi.draw_filter_params(w, seed=5)[0]
    say(f"four-step fftconv bf16 L={L}")
    spec = hy.filter_gen(params_to_dev(p), (L,))
    ws = torch.empty(hy.workspace_bytes(1, 1, 4, (L,), hy.BF16), dtype=torch.uint8, device="cuda")
    y = hy.operator(u.cuda(), [g.cuda()], [spec], ws=ws)
    torch.cuda.synchronize()
    h = orc.implicit_filter_1d(p, L)
    un, gn = u.float().numpy().astype(np.float64), g.float().numpy().astype(np.float64)
    ref = orc.causal_conv_fft(un, h[None]) * gn
    e = rel_err_rows(y.float().cpu().numpy(), ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < BF16_TOL, e.max()


@pytest.mark.parametrize("dtype,B", [("f32", 1), ("bf16", 1), ("bf16", 2)])
def test_fourstep_zero_input_gives_exact_zero(torch_cuda, dtype, B):
    """v = 0 gives y = 0 exactly on the multi-pass plans (per row, and the long-row matrix cores for B = 2)."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L, D = 1 << 15, 3
    w = hi.WORKLOADS[0].with_(B=B, D=D, dims=(L,))
    p = hi.draw_filter_params(w, seed=9)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    spectra = [hy.filter_gen(params_to_dev(q), (L,)) for q in p]
    v = torch.zeros((B, D, L), dtype=tdt, device="cuda")
    xs = [torch.randn((B, D, L), device="cuda").to(tdt) for _ in p]
    y = hy.operator(v, xs, spectra)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L", [1 << 16, 1 << 20])
def test_fourstep_block_scales_per_row(torch_cuda, L, dtype):
    """Rows whose magnitudes differ by 2^100 (a single impulse among them, the widest spread within a row) each
    stay within the storage type's tolerance of the oracle, and a NaN row turns NaN and leaves the others
    bitwise unchanged.  With bf16 storage the intermediate is fp16 with one power-of-two scale per block, and
    every block belongs to one (b, d) row; with fp32 storage it is fp32."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    B, D = 1, 6
    w = hi.WORKLOADS[2].with_(B=B, D=D, dims=(L,), order=2)
    rng = np.random.default_rng(L % 997)
    v = rng.standard_normal((B, D, L)).astype(np.float32)
    v[0, 0] *= 2.0 ** -60
    v[0, 1] *= 2.0 ** -20
    v[0, 3] *= 2.0 ** 40
    v[0, 4] = 0.0
    v[0, 4, L // 3] = 3.0
    xs = [rng.standard_normal((B, D, L)).astype(np.float32) for _ in range(2)]
    params = hi.draw_filter_params(w, seed=11)
    say(f"four-step {dtype} block scales, rows 2^-60 .. 2^40 and an impulse, L={L}")
    spectra = [hy.filter_gen(params_to_dev(q), (L,)) for q in params]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    vd = torch.from_numpy(v).to(tdt).cuda()
    xd = [torch.from_numpy(x).to(tdt).cuda() for x in xs]
    y = hy.operator(vd, xd, spectra)
    torch.cuda.synchronize()
    vr = vd.float().cpu().numpy()
    xr = [x.float().cpu().numpy() for x in xd]
    e = all_row_errors(w, vr, xr, params, y.float().cpu().numpy())
    report_errors("block scales", e)
    assert e.max() < (BF16_TOL if dtype == "bf16" else FP32_TOL)
    vn = vd.clone()
    vn[0, 2, L // 2] = float("nan")
    yn = hy.operator(vn, xd, spectra)
    torch.cuda.synchronize()
    assert torch.isnan(yn[0, 2]).any()
    keep = [0, 1, 3, 4, 5]
    assert torch.equal(yn[0, keep], y[0, keep])
