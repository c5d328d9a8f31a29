"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import subprocess

import pytest

import attention_free_long_implicit_amd as hy
from attention_free_long_implicit_amd import _lib as L


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from attention_free_long_implicit_amd import build
        build.build()
    return hy.lib()


def test_exports_every_declared_symbol(lib):
    names = hy.declared_symbols()
    assert len(names) >= 8
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    assert lib.hyena_status_str(0) == b"ok"
    for s in (-1, -2, -3, -4, -5):
        assert lib.hyena_status_str(s) != b"unknown status"
    assert lib.hyena_version() >= 100


def _size(fn, *args):
    n = ctypes.c_size_t()
    return fn(*args, ctypes.byref(n)), n.value


def test_size_queries(lib):
    st, n = _size(lib.hyena_spectrum_bytes, L.dims_of([8192]), L.CAUSAL, 768)
    # L = 8192 adds the matrix-core copy: 9 slabs x 16 registers x 64 lanes of fp16 pairs per channel, then a
    # 256-byte tail holding the copy's scale
    assert st == 0 and n == 768 * 8192 * 8 + 768 * (9 * 16 * 64 * 4 + 256)
    st, n = _size(lib.hyena_spectrum_bytes, L.dims_of([4096]), L.CAUSAL, 768)
    assert st == 0 and n == 768 * 4096 * 8
    st, n = _size(lib.hyena_filter_workspace_bytes, L.dims_of([1024]), L.CAUSAL, 16)
    assert st == 0 and n == 16 * 1024 * 4
    st, n = _size(lib.hyena_workspace_bytes, 2, 4, 768, L.dims_of([8192]), L.BF16, L.CAUSAL)
    assert st == 0 and n == 0
    # multi-pass lengths need a workspace of whole rows: L complex fp32 values, or with bf16 storage L fp16
    # pairs and 1024 words of block exponents
    st, n = _size(lib.hyena_workspace_bytes, 3, 2, 1024, L.dims_of([65536]), L.BF16, L.CAUSAL)
    assert st == 0 and n > 0 and n % (65536 * 4 + 4096) == 0
    st, n = _size(lib.hyena_workspace_bytes, 1, 1, 3, L.dims_of([65536]), L.BF16, L.CAUSAL)
    assert st == 0 and n == 3 * (65536 * 4 + 4096)
    st, n = _size(lib.hyena_workspace_bytes, 2, 1, 3, L.dims_of([1 << 20]), L.F32, L.CAUSAL)
    assert st == 0 and n == 3 * (1 << 20) * 8          # never more rows than there are
    # 3-D: spectrum 128 x 128 x 65 bins per channel; intermediate 65 x 64 x 64 per volume (after the
    # z transform only)
    st, n = _size(lib.hyena_spectrum_bytes, L.dims_of([64, 64, 64]), L.LINEAR, 128)
    assert st == 0 and n == 128 * 128 * 128 * 65 * 8
    st, n = _size(lib.hyena_workspace_bytes, 2, 1, 2, L.dims_of([64, 64, 64]), L.F32, L.LINEAR)
    assert st == 0 and n == 2 * 65 * 64 * 64 * 8
    # 128 volumes (272 MB of intermediate): two chunks of about 96 MB (47 volumes each) in the workspace
    st, n = _size(lib.hyena_workspace_bytes, 2, 1, 128, L.dims_of([64, 64, 64]), L.F32, L.LINEAR)
    assert st == 0 and n == 2 * 47 * 65 * 64 * 64 * 8
    # periodic 1-D: L/2 packed bins per channel, no workspace, taps only for the filter
    for Lc in (2048, 8192, 32768):
        st, n = _size(lib.hyena_spectrum_bytes, L.dims_of([Lc]), L.CIRCULAR, 16)
        assert st == 0 and n == 16 * (Lc // 2) * 8
        st, n = _size(lib.hyena_workspace_bytes, 2, 4, 16, L.dims_of([Lc]), L.F32, L.CIRCULAR)
        assert st == 0 and n == 0
        st, n = _size(lib.hyena_filter_workspace_bytes, L.dims_of([Lc]), L.CIRCULAR, 16)
        assert st == 0 and n == 16 * Lc * 4
    # long periodic rows: multi-pass on L/2 packed points, rows of L/2 complex fp32 values
    st, n = _size(lib.hyena_workspace_bytes, 2, 1, 3, L.dims_of([1 << 21]), L.F32, L.CIRCULAR)
    assert st == 0 and n == 3 * (1 << 20) * 8
    st, n = _size(lib.hyena_spectrum_bytes, L.dims_of([1 << 16]), L.CIRCULAR, 2)
    assert st == 0 and n == 2 * (1 << 15) * 8               # fp32 spectrum (every plan keeps fp32 intermediates)
    st, n = _size(lib.hyena_spectrum_bytes, L.dims_of([65536]), L.CAUSAL, 3)
    # fp32 spectrum, then the long-row matrix-core split coefficients: two fp16 complex values per packed
    # bin (L of them) and a 256-byte tail per channel
    for Lc in (1 << 15, 1 << 16, 1 << 17):
        st, n = _size(lib.hyena_spectrum_bytes, L.dims_of([Lc]), L.CAUSAL, 3)
        assert st == 0 and n == 3 * Lc * 8 + 3 * (Lc * 8 + 256)
    st, n = _size(lib.hyena_spectrum_bytes, L.dims_of([1 << 18]), L.CAUSAL, 3)
    assert st == 0 and n == 3 * (1 << 18) * 8
    # one channel: the filter workspace holds the taps and the L + 1 natural-order bins staged for the
    # long-row copy (8 bytes more than the multi-pass intermediate of one channel)
    for Lc in (1 << 15, 1 << 17):
        st, n = _size(lib.hyena_filter_workspace_bytes, L.dims_of([Lc]), L.CAUSAL, 1)
        assert st == 0 and n >= Lc * 4 + 256 + (Lc + 1) * 8
    # periodic 3-D: 64 x 64 x 33 bins per channel, intermediate 64 x-slabs of 64 x 33 per volume
    st, n = _size(lib.hyena_spectrum_bytes, L.dims_of([64, 64, 64]), L.CIRCULAR, 128)
    assert st == 0 and n == 128 * 64 * 64 * 33 * 8
    st, n = _size(lib.hyena_workspace_bytes, 2, 1, 2, L.dims_of([64, 64, 64]), L.F32, L.CIRCULAR)
    assert st == 0 and n == 2 * 64 * 64 * 33 * 8
    st, n = _size(lib.hyena_filter_workspace_bytes, L.dims_of([64, 64, 64]), L.CIRCULAR, 3)
    assert st == 0 and n == 3 * 64 ** 3 * 4 + 256 + 3 * 64 * 64 * 33 * 8


@pytest.mark.parametrize("shape,mode,status", [
    ([8191], L.CAUSAL, L.EUNSUPPORTED),      # not a power of two
    ([512], L.CAUSAL, L.EUNSUPPORTED),       # below the supported range
    ([1 << 21], L.CAUSAL, L.EUNSUPPORTED),   # above it
    ([0], L.CAUSAL, L.EINVAL),
    ([1024], L.LINEAR, L.EINVAL),            # linear mode needs a 3-D grid
    ([64, 64, 64], L.CAUSAL, L.EINVAL),      # causal mode needs 1-D
    ([32, 32, 32], L.LINEAR, L.EUNSUPPORTED),  # only the 64^3 grid is planned
    ([1024], L.CIRCULAR, L.EUNSUPPORTED),    # periodic rows: 2^11 .. 2^15
    ([1 << 22], L.CIRCULAR, L.EUNSUPPORTED),
    ([6144], L.CIRCULAR, L.EUNSUPPORTED),
    ([0], L.CIRCULAR, L.EINVAL),
    ([32, 32, 32], L.CIRCULAR, L.EUNSUPPORTED),   # periodic 3-D: the 64^3 grid only
    ([64, 64], L.CIRCULAR, L.EINVAL),
])
def test_bad_shapes(lib, shape, mode, status):
    st, _ = _size(lib.hyena_spectrum_bytes, L.dims_of(shape), mode, 4)
    assert st == status


def test_invalid_arguments_return_before_launch(lib):
    d = L.dims_of([8192])
    # null pointers
    assert lib.hyena_fftconv(4, 768, d, L.BF16, L.CAUSAL, None, 0x2000, None, 0x3000, None, 0, None) == L.EINVAL
    assert lib.hyena_fftconv(0, 768, d, L.BF16, L.CAUSAL, 0x1000, 0x2000, None, 0x3000, None, 0, None) == L.EINVAL
    assert lib.hyena_fftconv(4, 768, d, 7, L.CAUSAL, 0x1000, 0x2000, None, 0x3000, None, 0, None) == L.EINVAL
    # partial overlap of y with u / gate
    base = 1 << 32
    assert lib.hyena_fftconv(4, 768, d, L.BF16, L.CAUSAL, base, 0x2000, None, base + 64, None, 0, None) == L.EALIAS
    assert lib.hyena_fftconv(4, 768, d, L.BF16, L.CAUSAL, 0x10, 0x2000, base, base + 64, None, 0, None) == L.EALIAS
    # operator: order < 1, null gate, y overlapping a gate
    xs = (ctypes.c_void_p * 2)(base, base + (1 << 30))
    sp = (ctypes.c_void_p * 2)(0x100, 0x200)
    assert lib.hyena_operator(0, 4, 768, d, L.BF16, L.CAUSAL, 0x10, xs, sp, 1 << 40, None, 0, None) == L.EINVAL
    xs_null = (ctypes.c_void_p * 2)(base, None)
    assert lib.hyena_operator(2, 4, 768, d, L.BF16, L.CAUSAL, 0x10, xs_null, sp, 1 << 40, None, 0, None) == L.EINVAL
    assert lib.hyena_operator(2, 4, 768, d, L.BF16, L.CAUSAL, 1 << 40, xs, sp, base + 128, None, 0, None) == L.EALIAS
    # multi-pass length without a workspace
    d64 = L.dims_of([65536])
    assert lib.hyena_operator(2, 4, 768, d64, L.BF16, L.CAUSAL, 1 << 40, xs, sp, 1 << 41, None, 0, None) \
        == L.EWORKSPACE
    assert lib.hyena_fftconv(1, 4, d64, L.F32, L.CAUSAL, 1 << 40, 0x10, None, 1 << 41, 1 << 42, 100, None) \
        == L.EWORKSPACE
    # filter parameters of an unsupported width
    p = L.FilterParams(32, 64, 16, 1, 2, 3, 4, 5)
    assert lib.hyena_filter_gen(ctypes.byref(p), L.dims_of([1024]), L.CAUSAL, 0x1000, 0x2000, None, 0, None) \
        == L.EUNSUPPORTED
    p = L.FilterParams(64, 64, 16, 1, 2, 3, 4, 5)
    assert lib.hyena_filter_gen(ctypes.byref(p), L.dims_of([1024]), L.CAUSAL, None, 0x2000, None, 0, None) \
        == L.EWORKSPACE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(ImportError):
        L.lib()


def test_per_sample_sizes(lib):
    # one filter per (b, d): the spectrum of B*D filters, without the matrix-core copy at L = 8192
    st, n = _size(lib.hyena_spectrum_bytes, L.dims_of([8192]), L.CAUSAL | L.PER_SAMPLE, 4 * 768)
    assert st == 0 and n == 4 * 768 * 8192 * 8
    st, n = _size(lib.hyena_spectrum_bytes, L.dims_of([64, 64, 64]), L.LINEAR | L.PER_SAMPLE, 2 * 128)
    assert st == 0 and n == 2 * 128 * 128 * 128 * 65 * 8
    st, n = _size(lib.hyena_spectrum_bytes, L.dims_of([65536]), L.CAUSAL | L.PER_SAMPLE, 6)
    assert st == 0 and n == 6 * 65536 * 8
    # workspace: FiLM vectors (B x 4 x 64 floats) and the transposed 64 x 64 and D x 64 weights (256-byte
    # rounded), taps of B*D filters, transform chunk
    scratch = lambda B, D: -(-(B * 4 * 64 + 64 * (64 + D)) * 4 // 256) * 256
    st, n = _size(lib.hyena_film_filter_workspace_bytes, 2, L.dims_of([1024]), L.CAUSAL, 16)
    assert st == 0 and n == scratch(2, 16) + 2 * 16 * 1024 * 4
    st, n = _size(lib.hyena_film_filter_workspace_bytes, 2, L.dims_of([64, 64, 64]), L.LINEAR, 3)
    assert st == 0 and n == scratch(2, 3) + 6 * 127 ** 3 * 4 + 256 + 6 * 128 * 128 * 65 * 8
    st, n = _size(lib.hyena_film_filter_workspace_bytes, 0, L.dims_of([1024]), L.CAUSAL, 16)
    assert st == L.EINVAL
    # the flag leaves the conv workspace unchanged
    for mode in (L.CAUSAL, L.CAUSAL | L.PER_SAMPLE):
        st, n = _size(lib.hyena_workspace_bytes, 2, 1, 3, L.dims_of([1 << 20]), L.F32, mode)
        assert st == 0 and n == 3 * (1 << 20) * 8


def test_film_filter_gen_rejects_before_launch(lib):
    ptrs = [0x1000 + 64 * i for i in range(17)]
    d = L.dims_of([1024])
    ws = 1 << 40
    p = L.FilmParams(16, 64, 8, *ptrs)
    # null registers, workspace or parameter
    assert lib.hyena_film_filter_gen(ctypes.byref(p), 2, 4, None, d, L.CAUSAL, None, 0x2000, ws, 1 << 30, None) \
        == L.EINVAL
    assert lib.hyena_film_filter_gen(ctypes.byref(p), 2, 4, 0x3000, d, L.CAUSAL, None, 0x2000, None, 0, None) \
        == L.EINVAL
    q = L.FilmParams(16, 64, 8, *(ptrs[:5] + [None] + ptrs[6:]))
    assert lib.hyena_film_filter_gen(ctypes.byref(q), 2, 4, 0x3000, d, L.CAUSAL, None, 0x2000, ws, 1 << 30, None) \
        == L.EINVAL
    # unsupported widths and counts
    for bad in (L.FilmParams(16, 32, 8, *ptrs), L.FilmParams(5000, 64, 8, *ptrs)):
        assert lib.hyena_film_filter_gen(ctypes.byref(bad), 2, 4, 0x3000, d, L.CAUSAL, None, 0x2000, ws, 1 << 30,
                                         None) == L.EUNSUPPORTED
    assert lib.hyena_film_filter_gen(ctypes.byref(p), 2, 2000, 0x3000, d, L.CAUSAL, None, 0x2000, ws, 1 << 30,
                                     None) == L.EUNSUPPORTED
    assert lib.hyena_film_filter_gen(ctypes.byref(p), 2, 4, 0x3000, L.dims_of([1000]), L.CAUSAL, None, 0x2000, ws,
                                     1 << 30, None) == L.EUNSUPPORTED
    # workspace too small for the taps of B*D filters
    assert lib.hyena_film_filter_gen(ctypes.byref(p), 2, 4, 0x3000, d, L.CAUSAL, None, 0x2000, ws, 4096, None) \
        == L.EWORKSPACE


def test_projection_rejects_before_launch(lib):
    outs = (ctypes.c_void_p * 3)(1 << 40, 1 << 41, 1 << 42)
    x, W = 1 << 43, 1 << 44
    assert lib.hyena_projection(0, 2, 256, 64, 32, L.BF16, x, W, None, outs, None) == L.EINVAL
    assert lib.hyena_projection(2, 2, 256, 64, 32, 5, x, W, None, outs, None) == L.EINVAL
    assert lib.hyena_projection(2, 2, 256, 100, 32, L.BF16, x, W, None, outs, None) == L.EUNSUPPORTED   # d_model % 8
    assert lib.hyena_projection(9, 2, 256, 64, 32, L.BF16, x, W, None,
                                (ctypes.c_void_p * 10)(*[(i + 1) << 36 for i in range(10)]), None) == L.EUNSUPPORTED
    nul = (ctypes.c_void_p * 3)(1 << 40, None, 1 << 42)
    assert lib.hyena_projection(2, 2, 256, 64, 32, L.BF16, x, W, None, nul, None) == L.EINVAL
    # outputs overlapping each other or the input
    ov = (ctypes.c_void_p * 3)(1 << 40, (1 << 40) + 64, 1 << 42)
    assert lib.hyena_projection(2, 2, 256, 64, 32, L.BF16, x, W, None, ov, None) == L.EALIAS
    ox = (ctypes.c_void_p * 3)(1 << 40, x + 128, 1 << 42)
    assert lib.hyena_projection(2, 2, 256, 64, 32, L.BF16, x, W, None, ox, None) == L.EALIAS


def test_noalloc_rejects_before_launch(lib):
    xs = (ctypes.c_void_p * 2)(1 << 43, 1 << 44)
    sp = (ctypes.c_void_p * 2)(1 << 45, 1 << 46)
    d1 = L.dims_of([1 << 17])
    assert lib.hyena_operator_noalloc(0, 2, 8, d1, L.F32, L.CAUSAL, 1 << 41, xs, sp, 1 << 42, None) == L.EINVAL
    assert lib.hyena_operator_noalloc(2, 2, 8, d1, 7, L.CAUSAL, 1 << 41, xs, sp, 1 << 42, None) == L.EINVAL
    assert lib.hyena_operator_noalloc(2, 2, 8, L.dims_of([3000]), L.F32, L.CAUSAL, 1 << 41, xs, sp, 1 << 42,
                                      None) == L.EUNSUPPORTED
    assert lib.hyena_operator_noalloc(2, 2, 8, d1, L.F32, L.CAUSAL, 1 << 41, xs, sp, (1 << 41) + 64,
                                      None) == L.EALIAS


def test_decode_sizes_and_rejects_before_launch(lib):
    n = ctypes.c_size_t()
    # histories and prefix contributions, fp32, two planes per order; no workspace below 32768 points
    assert lib.hyena_decode_state_bytes(2, 4, 768, 8192, ctypes.byref(n)) == L.OK
    assert n.value == 2 * 2 * 4 * 768 * 8192 * 4
    assert lib.hyena_decode_state_bytes(2, 1, 256, 1 << 20, ctypes.byref(n)) == L.OK
    assert n.value > 2 * 2 * 256 * (1 << 20) * 4            # plus the multi-pass workspace
    assert lib.hyena_decode_state_bytes(0, 1, 8, 8192, ctypes.byref(n)) == L.EINVAL
    assert lib.hyena_decode_state_bytes(9, 1, 8, 8192, ctypes.byref(n)) == L.EUNSUPPORTED
    assert lib.hyena_decode_state_bytes(2, 1, 8, 3000, ctypes.byref(n)) == L.EUNSUPPORTED
    assert lib.hyena_decode_state_bytes(2, 1, 8, 512, ctypes.byref(n)) == L.EUNSUPPORTED
    assert lib.hyena_decode_state_bytes(2, 1, 8, 8192, None) == L.EINVAL
    B, D, Lq, order = 2, 8, 1024, 2
    assert lib.hyena_decode_state_bytes(order, B, D, Lq, ctypes.byref(n)) == L.OK
    need = n.value
    state = 1 << 40
    v, y = 1 << 41, 1 << 42
    xs = (ctypes.c_void_p * 2)(1 << 43, 1 << 44)
    taps = (ctypes.c_void_p * 2)(1 << 45, 1 << 46)
    sp = (ctypes.c_void_p * 2)(1 << 47, 3 << 46)

    def step(t=5, block=64, st=state, nbytes=need, yy=y, vv=v, x=xs, dtype=L.F32, mode=L.CAUSAL):
        return lib.hyena_decode_step(order, B, D, Lq, block, t, dtype, mode, vv, x, taps, sp, yy, st, nbytes, None)
    assert step(t=-1) == L.EINVAL and step(t=Lq) == L.EINVAL and step(dtype=7) == L.EINVAL
    assert step(mode=L.CIRCULAR) == L.EUNSUPPORTED and step(mode=L.LINEAR | L.PER_SAMPLE) == L.EUNSUPPORTED
    assert step(block=48) == L.EUNSUPPORTED and step(block=2 * Lq) == L.EUNSUPPORTED
    assert step(nbytes=need - 1) == L.EWORKSPACE
    assert step(st=state + 16) == L.EWORKSPACE                 # not 256-byte aligned
    assert step(st=None) == L.EINVAL and step(yy=None) == L.EINVAL
    assert step(x=(ctypes.c_void_p * 2)(1 << 43, None)) == L.EINVAL
    assert step(yy=state + 4096) == L.EALIAS                    # output inside the state
    assert step(yy=v + 4) == L.EALIAS                           # output overlapping an input
    assert step(yy=v + 2 * B * D - 2, dtype=L.BF16) == L.EALIAS  # bf16 tokens: 2 bytes per row
    assert step(vv=state + 256) == L.EALIAS                     # input inside the state
    assert lib.hyena_decode_step(order, B, D, Lq, 64, 5, L.F32, L.CAUSAL, v, xs, (ctypes.c_void_p * 2)(state + 512, 1 << 46),
                                 sp, y, state, need, None) == L.EALIAS          # taps inside the state
    assert lib.hyena_decode_step(order, B, D, Lq, 64, 5, L.F32, L.CAUSAL, v, xs, taps, (ctypes.c_void_p * 2)(1 << 47, y - 64),
                                 y, state, need, None) == L.EALIAS              # output inside a spectrum
    def prefill(P=128, block=64, st=state, yy=y, dtype=L.F32):
        return lib.hyena_decode_prefill(order, B, D, Lq, block, P, dtype, L.CAUSAL, v, xs, sp, yy, st, need, None)
    assert prefill(P=100) == L.EINVAL and prefill(P=0) == L.EINVAL and prefill(P=2 * Lq) == L.EINVAL
    assert prefill(block=3) == L.EUNSUPPORTED and prefill(dtype=9) == L.EINVAL
    assert prefill(st=state + 8) == L.EWORKSPACE
    assert prefill(yy=state + 1024) == L.EALIAS and prefill(yy=v + 8) == L.EALIAS
    sp_in_state = (ctypes.c_void_p * 2)(1 << 47, state + 2048)
    assert lib.hyena_decode_prefill(order, B, D, Lq, 64, 128, L.F32, L.CAUSAL, v, xs, sp_in_state, y, state, need,
                                    None) == L.EALIAS             # a spectrum inside the state
    y_in_sp = (ctypes.c_void_p * 2)(1 << 47, y - 64)
    assert lib.hyena_decode_prefill(order, B, D, Lq, 64, 128, L.F32, L.CAUSAL, v, xs, y_in_sp, y, state, need,
                                    None) == L.EALIAS             # the output inside a spectrum
    assert lib.hyena_decode_reset(order, B, D, Lq, state, need - 1, None) == L.EWORKSPACE
    assert lib.hyena_decode_reset(order, B, D, Lq, None, need, None) == L.EINVAL


def test_binding_rejects_wrong_dtypes_before_calling():
    import torch
    p = {k: torch.zeros(4, dtype=torch.float64) for k in ("W1", "b1", "W2", "b2", "alpha")}
    p["W1"] = torch.zeros(64, 64, dtype=torch.float64)
    p["W2"] = torch.zeros(8, 64, dtype=torch.float64)
    with pytest.raises(TypeError):
        hy.filter_gen(p, (1024,))
    x = torch.zeros(1, 128, 32, dtype=torch.bfloat16)
    W = torch.zeros(64, 32, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        hy.projection(x, W, 1, bias=torch.zeros(64, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        hy.projection(x, torch.zeros(64, 32, dtype=torch.float32), 1)
