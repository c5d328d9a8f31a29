"""GPU parity of streaming decode: every token of a sequence through hyena_decode_step (prefix blocks
convolved by FFT against the cached spectra, the rest of each block summed directly), against the
oracle's token-by-token evaluation (or, for long rows, the whole-sequence form it is pinned to)."""
import numpy as np
import pytest

import hyena_inputs as hi
from oracle import hyena_oracle as orc
from gpu_util import BF16_TOL, FP32_TOL, params_to_dev, rel_err_rows, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import attention_free_long_implicit_amd as hy
    hy.lib()
    return torch


def _filters(torch, w, params):
    import attention_free_long_implicit_amd as hy
    L = w.dims[0]
    taps = [torch.empty((w.D, L), dtype=torch.float32, device="cuda") for _ in params]
    spectra = [hy.filter_gen(params_to_dev(p), (L,), h_time=h) for p, h in zip(params, taps)]
    return taps, spectra


def _decode(torch, w, v, xs, taps, spectra, block, state=None):
    """All L tokens of [B, D, L] inputs through the decode entry points; y as float64 [B, D, L]."""
    import attention_free_long_implicit_amd as hy
    B, D, L, order = w.B, w.D, w.dims[0], len(xs)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    vt = to_dev(np.moveaxis(v, -1, 0), dt)                            # token-major [L, B, D]
    xt = [to_dev(np.moveaxis(x, -1, 0), dt) for x in xs]
    yt = torch.empty_like(vt)
    if state is None:
        state = torch.empty(hy.decode_state_bytes(order, B, D, L), dtype=torch.uint8, device="cuda")
    hy.decode_reset(state, order, B, D, L)
    for t in range(L):
        hy.decode_step(t, vt[t], [x[t] for x in xt], taps, spectra, state, L, block, y_t=yt[t])
    torch.cuda.synchronize()
    return np.moveaxis(yt.float().cpu().numpy().astype(np.float64), 0, -1)


def _rows(a):
    return a.reshape(-1, a.shape[-1])


@pytest.mark.parametrize("order,B,D,L,block", [
    (2, 2, 8, 1024, 64),       # 16 blocks: 15 prefix convolutions
    (2, 2, 8, 1024, 1024),     # one block: direct sums only
    (3, 1, 4, 2048, 128),      # order 3
    (1, 3, 5, 1024, 1),        # a prefix convolution before every token, no in-block sum
    (2, 1, 6, 1024, 512),      # D not a multiple of the 4 rows of a workgroup
])
def test_decode_matches_oracle(torch_cuda, order, B, D, L, block):
    torch = torch_cuda
    w = hi.WORKLOADS[9].with_(order=order, B=B, D=D, dims=(L,))
    v, xs = hi.draw_activations(w, seed=L + block)
    params = hi.draw_filter_params(w, seed=L + block)
    say(f"decode order={order} B={B} D={D} L={L} block={block}")
    taps, spectra = _filters(torch, w, params)
    y = _decode(torch, w, v, xs, taps, spectra, block)
    hs = [np.tile(orc.implicit_filter_1d(p, L), (B, 1)) for p in params]
    ref = orc.hyena_decode_stream(_rows(v), [_rows(x) for x in xs], hs)
    e = rel_err_rows(_rows(y), ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < FP32_TOL, e.max()


def test_decode_multipass_prefix(torch_cuda):
    """L = 32768: the prefix convolutions take the multi-pass plan and the state's workspace."""
    torch = torch_cuda
    w = hi.WORKLOADS[9].with_(B=1, D=2, dims=(32768,))
    v, xs = hi.draw_activations(w, seed=3)
    params = hi.draw_filter_params(w, seed=3)
    say("decode L=32768 block=4096")
    taps, spectra = _filters(torch, w, params)
    y = _decode(torch, w, v, xs, taps, spectra, 4096)
    hs = [orc.implicit_filter_1d(p, 32768) for p in params]
    ref = orc.hyena_operator_rows(_rows(v), [_rows(x) for x in xs], hs)      # pinned to the streaming form
    e = rel_err_rows(_rows(y), ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < FP32_TOL, e.max()


def test_decode_full_size(torch_cuda):
    """The decode workload at full size (B = 4, D = 768, L = 8192, blocks of 256): sampled rows against
    the oracle's token-by-token evaluation; every row against the whole-sequence HIP operator."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[9]
    L = w.dims[0]
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    say(f"decode full size {w.name}")
    taps, spectra = _filters(torch, w, params)
    y = _decode(torch, w, v, xs, taps, spectra, w.decode_block)
    rows = [(0, 0), (1, 5), (2, 383), (3, 767)]
    sel = [b * w.D + d for b, d in rows]
    hs = [orc.implicit_filter_1d(p, L, channels=[d for _, d in rows]) for p in params]
    ref = orc.hyena_decode_stream(_rows(v)[sel], [_rows(x)[sel] for x in xs], hs)
    e = rel_err_rows(_rows(y)[sel], ref)
    say(f"  sampled rows: max rel err {e.max():.3e}")
    assert e.max() < FP32_TOL, e.max()
    whole = hy.operator(to_dev(v, torch.float32), [to_dev(x, torch.float32) for x in xs], spectra)
    torch.cuda.synchronize()
    e2 = rel_err_rows(_rows(y), _rows(whole.cpu().numpy().astype(np.float64)))
    say(f"  every row vs the whole-sequence operator: max rel diff {e2.max():.3e}")
    assert e2.max() < FP32_TOL, e2.max()


def test_decode_state_reuse_after_reset(torch_cuda):
    """A state that decoded one sequence, once reset, gives bit-identical results for the next."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[9].with_(B=2, D=4, dims=(1024,))
    taps, spectra = _filters(torch, w, hi.draw_filter_params(w, seed=11))
    state = torch.empty(hy.decode_state_bytes(2, 2, 4, 1024), dtype=torch.uint8, device="cuda")
    v1, xs1 = hi.draw_activations(w, seed=12)
    v2, xs2 = hi.draw_activations(w, seed=13)
    _decode(torch, w, v1, xs1, taps, spectra, 128, state=state)
    again = _decode(torch, w, v2, xs2, taps, spectra, 128, state=state)
    fresh = _decode(torch, w, v2, xs2, taps, spectra, 128)
    np.testing.assert_array_equal(again, fresh)


@pytest.mark.parametrize("order,B,D,L,block", [(2, 2, 8, 1024, 64), (3, 1, 4, 2048, 128)])
def test_decode_bf16_tokens_match_oracle(torch_cuda, order, B, D, L, block):
    """bf16 tokens (inputs rounded to bf16 once, as both sides see them; the GPU's intermediates u_i stay
    fp32, only y_t is rounded)."""
    torch = torch_cuda
    w = hi.WORKLOADS[9].with_(order=order, B=B, D=D, dims=(L,), dtype="bf16")
    v, xs = hi.draw_activations(w, seed=L + block + 1)
    params = hi.draw_filter_params(w, seed=L + block + 1)
    say(f"decode bf16 order={order} B={B} D={D} L={L} block={block}")
    taps, spectra = _filters(torch, w, params)
    y = _decode(torch, w, v, xs, taps, spectra, block)
    hs = [np.tile(orc.implicit_filter_1d(p, L), (B, 1)) for p in params]
    ref = orc.hyena_decode_stream(_rows(v), [_rows(x) for x in xs], hs)
    e = rel_err_rows(_rows(y), ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < BF16_TOL, e.max()


def test_decode_bf16_layer_of_workload_1(torch_cuda):
    """The layer of workload 1 (B = 4, D = 768, L = 8192, bf16) decoded token by token: sampled rows against
    the oracle, every row against the whole-sequence bf16 operator (matrix-core path)."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[1].with_(decode_block=256)
    L = w.dims[0]
    v, xs = hi.draw_activations(w)
    params = hi.draw_filter_params(w)
    say(f"decode bf16 {w.name}")
    taps, spectra = _filters(torch, w, params)
    y = _decode(torch, w, v, xs, taps, spectra, w.decode_block)
    rows = [(0, 0), (1, 77), (3, 767)]
    sel = [b * w.D + d for b, d in rows]
    hs = [orc.implicit_filter_1d(p, L, channels=[d for _, d in rows]) for p in params]
    ref = orc.hyena_decode_stream(_rows(v)[sel], [_rows(x)[sel] for x in xs], hs)
    e = rel_err_rows(_rows(y)[sel], ref)
    say(f"  sampled rows: max rel err {e.max():.3e}")
    assert e.max() < BF16_TOL, e.max()
    whole = hy.operator(to_dev(v, torch.bfloat16), [to_dev(x, torch.bfloat16) for x in xs], spectra)
    torch.cuda.synchronize()
    e2 = rel_err_rows(_rows(y), _rows(whole.float().cpu().numpy().astype(np.float64)))
    say(f"  every row vs the whole-sequence operator: max rel diff {e2.max():.3e}")
    # each path is held to BF16_TOL against the oracle (the operator's matrix-core transforms round their
    # operands to bf16 and carry most of it), so their difference is bounded by the sum of the two
    assert e2.max() < 2 * BF16_TOL, e2.max()


@pytest.mark.parametrize("order,B,D,L,block,P,dtype", [
    (2, 2, 8, 1024, 64, 512, "f32"),        # half the sequence as a prompt, the rest token by token
    (3, 1, 4, 2048, 128, 384, "f32"),
    (2, 2, 8, 1024, 64, 256, "bf16"),
    (2, 1, 3, 1024, 256, 1024, "f32"),      # the whole sequence as a prompt
])
def test_decode_after_prefill_matches_oracle(torch_cuda, order, B, D, L, block, P, dtype):
    """hyena_decode_prefill on the first P tokens, then hyena_decode_step for t = P..L-1: the joined outputs
    against the oracle's token-by-token evaluation of the whole sequence."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    w = hi.WORKLOADS[9].with_(order=order, B=B, D=D, dims=(L,), dtype=dtype)
    v, xs = hi.draw_activations(w, seed=P + block)
    params = hi.draw_filter_params(w, seed=P + block)
    say(f"decode after prefill order={order} B={B} D={D} L={L} block={block} P={P} {dtype}")
    taps, spectra = _filters(torch, w, params)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    state = torch.empty(hy.decode_state_bytes(order, B, D, L), dtype=torch.uint8, device="cuda")
    state.fill_(255)                                   # prefill needs no reset: every history row is written
    y_pre = hy.decode_prefill(to_dev(v[..., :P], dt), [to_dev(x[..., :P], dt) for x in xs], spectra, state, L, block)
    vt = to_dev(np.moveaxis(v, -1, 0), dt)
    xt = [to_dev(np.moveaxis(x, -1, 0), dt) for x in xs]
    yt = torch.empty_like(vt)
    for t in range(P, L):
        hy.decode_step(t, vt[t], [x[t] for x in xt], taps, spectra, state, L, block, y_t=yt[t])
    torch.cuda.synchronize()
    y = np.concatenate([y_pre.float().cpu().numpy(), np.moveaxis(yt.float().cpu().numpy(), 0, -1)[..., P:]], axis=-1)
    hs = [np.tile(orc.implicit_filter_1d(p, L), (B, 1)) for p in params]
    ref = orc.hyena_decode_stream(_rows(v), [_rows(x) for x in xs], hs)
    e = rel_err_rows(_rows(y.astype(np.float64)), ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < (BF16_TOL if dtype == "bf16" else FP32_TOL), e.max()


def test_decode_after_prefill_multipass(torch_cuda):
    """L = 32768: the prompt's convolutions and the later prefix convolutions on the multi-pass plan."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    L, P, block = 32768, 28672, 4096
    w = hi.WORKLOADS[9].with_(B=1, D=2, dims=(L,))
    v, xs = hi.draw_activations(w, seed=21)
    params = hi.draw_filter_params(w, seed=21)
    say("decode after prefill L=32768 P=28672 block=4096")
    taps, spectra = _filters(torch, w, params)
    state = torch.empty(hy.decode_state_bytes(2, 1, 2, L), dtype=torch.uint8, device="cuda")
    y_pre = hy.decode_prefill(to_dev(v[..., :P], torch.float32), [to_dev(x[..., :P], torch.float32) for x in xs],
                              spectra, state, L, block)
    vt = to_dev(np.moveaxis(v, -1, 0), torch.float32)
    xt = [to_dev(np.moveaxis(x, -1, 0), torch.float32) for x in xs]
    yt = torch.empty_like(vt)
    for t in range(P, L):
        hy.decode_step(t, vt[t], [x[t] for x in xt], taps, spectra, state, L, block, y_t=yt[t])
    torch.cuda.synchronize()
    y = np.concatenate([y_pre.cpu().numpy(), np.moveaxis(yt.cpu().numpy(), 0, -1)[..., P:]], axis=-1)
    hs = [orc.implicit_filter_1d(p, L) for p in params]
    ref = orc.hyena_operator_rows(_rows(v), [_rows(x) for x in xs], hs)      # pinned to the streaming form
    e = rel_err_rows(_rows(y.astype(np.float64)), ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < FP32_TOL, e.max()


def test_decode_per_sample_filters(torch_cuda):
    """Input-dependent (per (b, d)) filters: FiLM-SIREN taps [B, D, L] and spectra of B*D filters, decoded with
    HYENA_PER_SAMPLE (a prompt through the prefill, then token steps), against the oracle."""
    torch = torch_cuda
    import attention_free_long_implicit_amd as hy
    B, D, L, block, P = 2, 6, 1024, 64, 320
    w = hi.WORKLOADS[7].with_(B=B, D=D, dims=(L,), mode="causal", registers=4)
    params, reg = hi.draw_film_params(w, seed=31), hi.draw_registers(w, seed=31)
    v, xs = hi.draw_activations(w, seed=31)
    say(f"decode per-sample filters B={B} D={D} L={L} block={block} P={P}")
    mode = hy.CAUSAL | hy.PER_SAMPLE
    taps = [torch.empty((B, D, L), dtype=torch.float32, device="cuda") for _ in params]
    spectra = [hy.film_filter_gen(params_to_dev(p), to_dev(reg, torch.float32), (L,), h_time=h)
               for p, h in zip(params, taps)]
    state = torch.empty(hy.decode_state_bytes(2, B, D, L), dtype=torch.uint8, device="cuda")
    y_pre = hy.decode_prefill(to_dev(v[..., :P], torch.float32), [to_dev(x[..., :P], torch.float32) for x in xs],
                              spectra, state, L, block, mode=mode)
    vt = to_dev(np.moveaxis(v, -1, 0), torch.float32)
    xt = [to_dev(np.moveaxis(x, -1, 0), torch.float32) for x in xs]
    yt = torch.empty_like(vt)
    for t in range(P, L):
        hy.decode_step(t, vt[t], [x[t] for x in xt], taps, spectra, state, L, block, y_t=yt[t], mode=mode)
    torch.cuda.synchronize()
    y = np.concatenate([y_pre.cpu().numpy(), np.moveaxis(yt.cpu().numpy(), 0, -1)[..., P:]], axis=-1)
    hs = [_rows(orc.input_dependent_filter_1d(p, reg, L)) for p in params]
    ref = orc.hyena_decode_stream(_rows(v), [_rows(x) for x in xs], hs)
    e = rel_err_rows(_rows(y.astype(np.float64)), ref)
    say(f"  max rel err {e.max():.3e}")
    assert e.max() < FP32_TOL, e.max()
