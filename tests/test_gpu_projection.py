"""GPU parity of the input projection split(W_proj x) -> channel-major v, x_1..x_N, and of the layer
from token-major inputs (projection, then the operator), against the oracle."""
import numpy as np
import pytest

import hyena_inputs as hi
from oracle import hyena_oracle as orc
from gpu_util import BF16_TOL, FP32_TOL, rel_err_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import attention_free_long_implicit_amd as hy
    hy.lib()
    return torch


def _round(a, dtype):
    return hi.bf16_bits_to_f32(hi.bf16_bits_rne(a)) if dtype == "bf16" else a.astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,L,Dm,D,order", [
    (2, 300, 64, 80, 2),       # ragged tokens (300 = 2 tiles + 44) and channels (240 = 128 + 112)
    (1, 128, 32, 128, 1),      # exactly one tile each way, one k-tile
    (3, 1000, 96, 40, 3),      # four outputs, channel tiles cutting across chunks, a k tail
    (2, 264, 200, 300, 2),     # k tail of 8 (bf16) / 8 (fp32) past whole k tiles; 900 channels
    (1, 100, 40, 16, 1),       # L not a multiple of 8: element stores
])
def test_projection_matches_oracle(torch_cuda, dtype, B, L, Dm, D, order):
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    rng = np.random.default_rng(B * 1000 + L + Dm)
    M = (order + 1) * D
    x = _round(rng.standard_normal((B, L, Dm)).astype(np.float32), dtype)
    W = _round((rng.standard_normal((M, Dm)) / np.sqrt(Dm)).astype(np.float32), dtype)
    bias = rng.standard_normal(M).astype(np.float32) * 0.1
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    say(f"projection {dtype} B={B} L={L} d_model={Dm} D={D} order={order}")
    outs = hy.projection(to_dev(x, dt), to_dev(W, dt), order, bias=to_dev(bias, torch.float32))
    torch.cuda.synchronize()
    ref = orc.input_projection(x, W, bias, order)
    worst = 0.0
    for o, r in zip(outs, ref):
        assert tuple(o.shape) == (B, D, L)
        worst = max(worst, rel_err_rows(o.float().cpu().numpy(), r).max())
    say(f"  max rel err {worst:.3e}")
    assert worst < (BF16_TOL if dtype == "bf16" else FP32_TOL) / 4, worst


def test_projection_block_identity_is_bit_exact(torch_cuda):
    """W = [I; 2I; 3I]: every output is one exact product, so the stores must equal the oracle's values
    rounded once to bf16 -- a check of the output layout (chunk order, channel-major rows, token columns)."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    B, L, D = 2, 520, 160
    rng = np.random.default_rng(7)
    x = _round(rng.standard_normal((B, L, D)).astype(np.float32), "bf16")
    W = np.concatenate([np.eye(D), 2 * np.eye(D), 3 * np.eye(D)]).astype(np.float32)
    say("projection block identity, bf16")
    outs = hy.projection(to_dev(x, torch.bfloat16), to_dev(W, torch.bfloat16), 2)
    torch.cuda.synchronize()
    for o, r in zip(outs, orc.input_projection(x, W, None, 2)):
        got = o.view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, hi.bf16_bits_rne(r.astype(np.float32)))


def test_projection_full_size_sampled_channels(torch_cuda):
    """Workload 8's projection at full size (B = 4, L = 8192, d_model = 768, 3 x 768 channels, bf16)."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[8]
    x, W, bias = hi.draw_projection(w)
    say(f"projection full size {w.name}")
    outs = hy.projection(to_dev(x, torch.bfloat16), to_dev(W, torch.bfloat16), w.order, bias=to_dev(bias, torch.float32))
    torch.cuda.synchronize()
    worst = 0.0
    for j, o in enumerate(outs):
        for d in (0, 1, 255, 500, w.D - 1):
            c = j * w.D + d
            ref = x.astype(np.float64) @ W[c].astype(np.float64) + bias[c]          # [B, L]
            got = o[:, d, :].float().cpu().numpy()
            worst = max(worst, rel_err_rows(got, ref).max())
    say(f"  max rel err {worst:.3e}")
    assert worst < BF16_TOL / 4, worst


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_from_token_major_inputs(torch_cuda, dtype):
    """Projection then the order-2 operator, against the oracle's projection and operator."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[8].with_(B=2, D=24, dims=(2048,), d_model=64, dtype=dtype)
    x, W, bias = hi.draw_projection(w, seed=5)
    params = hi.draw_filter_params(w, seed=5)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    say(f"layer from token-major inputs {dtype}")
    v, *gates = hy.projection(to_dev(x, dt), to_dev(W, dt), w.order)
    spectra = [hy.filter_gen({k: to_dev(a, torch.float32) for k, a in p.items()}, w.dims) for p in params]
    y = hy.operator(v, gates, spectra)
    torch.cuda.synchronize()
    rv, *rx = orc.input_projection(x, W, None, w.order)
    hs = [orc.implicit_filter_1d(p, w.dims[0]) for p in params]
    ref = orc.hyena_operator_rows(rv, rx, hs)
    e = rel_err_rows(y.float().cpu().numpy(), ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < (BF16_TOL if dtype == "bf16" else FP32_TOL), e.max()


def test_projection_nine_outputs(torch_cuda):
    """order 8: nine output chunks (the largest the entry point takes)."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    B, L, Dm, D, order = 1, 384, 64, 24, 8
    rng = np.random.default_rng(9)
    x = _round(rng.standard_normal((B, L, Dm)).astype(np.float32), "bf16")
    W = _round((rng.standard_normal(((order + 1) * D, Dm)) / 8).astype(np.float32), "bf16")
    say("projection, nine outputs")
    outs = hy.projection(to_dev(x, torch.bfloat16), to_dev(W, torch.bfloat16), order)
    torch.cuda.synchronize()
    assert len(outs) == 9
    worst = max(rel_err_rows(o.float().cpu().numpy(), r).max() for o, r in zip(outs, orc.input_projection(x, W, None, order)))
    assert worst < BF16_TOL / 4, worst
