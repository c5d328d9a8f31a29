"""ctypes binding of libhyena.so (include/hyena.h).  Argument marshalling only: every step of the
operator runs in the library's HIP kernels; PyTorch supplies device memory and the current stream.

The library must have been built (``python -m attention_free_long_implicit_amd.build``); loading
fails loudly otherwise -- there is no fallback path."""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhyena.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "hyena.h")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, EALIAS = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
CAUSAL, LINEAR, CIRCULAR = 0, 1, 2
PER_SAMPLE = 8          # mode flag: one filter per (b, d) (input-dependent filters)


class HyenaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_str(status)})")


class Dims(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32), ("n", ctypes.c_int64 * 3)]


class FilterParams(ctypes.Structure):
    _fields_ = [("F", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("W1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("W2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("alpha", ctypes.c_void_p)]


class FilmParams(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32)] + [
        (k, ctypes.c_void_p) for k in ("q", "A1", "a1", "omega0", "A2", "a2", "A3", "a3", "G1", "g1", "P1", "p1",
                                       "G2", "g2", "P2", "p2", "sigma")]


_lib = None
_c = ctypes
_SIG = {
    "hyena_version": (_c.c_int, []),
    "hyena_init": (_c.c_int, []),
    "hyena_status_str": (_c.c_char_p, [_c.c_int]),
    "hyena_spectrum_bytes": (_c.c_int, [Dims, _c.c_int, _c.c_int64, _c.POINTER(_c.c_size_t)]),
    "hyena_filter_workspace_bytes": (_c.c_int, [Dims, _c.c_int, _c.c_int64, _c.POINTER(_c.c_size_t)]),
    "hyena_workspace_bytes": (_c.c_int, [_c.c_int, _c.c_int64, _c.c_int64, Dims, _c.c_int, _c.c_int,
                                         _c.POINTER(_c.c_size_t)]),
    "hyena_filter_gen": (_c.c_int, [_c.POINTER(FilterParams), Dims, _c.c_int, _c.c_void_p, _c.c_void_p,
                                    _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "hyena_fftconv": (_c.c_int, [_c.c_int64, _c.c_int64, Dims, _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p,
                                 _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "hyena_operator": (_c.c_int, [_c.c_int, _c.c_int64, _c.c_int64, Dims, _c.c_int, _c.c_int, _c.c_void_p,
                                  _c.POINTER(_c.c_void_p), _c.POINTER(_c.c_void_p), _c.c_void_p, _c.c_void_p,
                                  _c.c_size_t, _c.c_void_p]),
    "hyena_operator_noalloc": (_c.c_int, [_c.c_int, _c.c_int64, _c.c_int64, Dims, _c.c_int, _c.c_int, _c.c_void_p,
                                          _c.POINTER(_c.c_void_p), _c.POINTER(_c.c_void_p), _c.c_void_p, _c.c_void_p]),
    "hyena_spectrum_export": (_c.c_int, [Dims, _c.c_int, _c.c_int64, _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "hyena_projection": (_c.c_int, [_c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int, _c.c_void_p,
                                    _c.c_void_p, _c.c_void_p, _c.POINTER(_c.c_void_p), _c.c_void_p]),
    "hyena_film_filter_workspace_bytes": (_c.c_int, [_c.c_int64, Dims, _c.c_int, _c.c_int64,
                                                     _c.POINTER(_c.c_size_t)]),
    "hyena_film_filter_gen": (_c.c_int, [_c.POINTER(FilmParams), _c.c_int64, _c.c_int32, _c.c_void_p, Dims,
                                         _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_size_t,
                                         _c.c_void_p]),
    "hyena_decode_state_bytes": (_c.c_int, [_c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.POINTER(_c.c_size_t)]),
    "hyena_decode_reset": (_c.c_int, [_c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p, _c.c_size_t,
                                      _c.c_void_p]),
    "hyena_decode_prefill": (_c.c_int, [_c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64,
                                        _c.c_int, _c.c_int, _c.c_void_p, _c.POINTER(_c.c_void_p), _c.POINTER(_c.c_void_p),
                                        _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "hyena_decode_step": (_c.c_int, [_c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int,
                                     _c.c_int, _c.c_void_p, _c.POINTER(_c.c_void_p), _c.POINTER(_c.c_void_p),
                                     _c.POINTER(_c.c_void_p), _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
}


def lib():
    """Load libhyena.so once and attach the C signatures.  Raises if the library is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m attention_free_long_implicit_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def declared_symbols() -> list:
    """Names of the functions include/hyena.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(hyena_\w+)\s*\(", text, flags=re.M)))


def status_str(status: int) -> str:
    try:
        return lib().hyena_status_str(int(status)).decode()
    except Exception:  # pragma: no cover - used while formatting another error
        return "?"


def _check(status: int, what: str):
    if status != OK:
        raise HyenaError(status, what)


def dims_of(shape: Sequence[int]) -> Dims:
    pts = list(shape)
    d = Dims()
    d.ndim = len(pts)
    for i in range(3):
        d.n[i] = pts[i] if i < len(pts) else 0
    return d


def mode_for(ndim: int) -> int:
    return CAUSAL if ndim == 1 else LINEAR


# ----------------------------------------------------------------------------- torch-facing wrappers
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors must be contiguous CUDA (HIP) tensors")
    return t.data_ptr()


def spectrum_bytes(point_shape: Sequence[int], D: int, mode: Optional[int] = None) -> int:
    n = ctypes.c_size_t()
    mode = mode_for(len(point_shape)) if mode is None else mode
    _check(lib().hyena_spectrum_bytes(dims_of(point_shape), mode, D, ctypes.byref(n)), "hyena_spectrum_bytes")
    return n.value


def filter_workspace_bytes(point_shape: Sequence[int], D: int, mode: Optional[int] = None) -> int:
    n = ctypes.c_size_t()
    mode = mode_for(len(point_shape)) if mode is None else mode
    _check(lib().hyena_filter_workspace_bytes(dims_of(point_shape), mode, D, ctypes.byref(n)),
           "hyena_filter_workspace_bytes")
    return n.value


def workspace_bytes(order: int, B: int, D: int, point_shape: Sequence[int], dtype_code: int,
                    mode: Optional[int] = None) -> int:
    n = ctypes.c_size_t()
    mode = mode_for(len(point_shape)) if mode is None else mode
    _check(lib().hyena_workspace_bytes(order, B, D, dims_of(point_shape), dtype_code, mode, ctypes.byref(n)),
           "hyena_workspace_bytes")
    return n.value


def _workspace(nbytes: int, device):
    if nbytes == 0:
        return None
    torch = _torch()
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def filter_gen(params: dict, point_shape: Sequence[int], h_time=None, spectrum=None, mode: Optional[int] = None):
    """One order's implicit filter.  params: dict of CUDA float32 tensors W1 [H,F], b1 [H], W2 [D,H],
    b2 [D], alpha [D].  Returns the spectrum (opaque uint8 tensor); fills h_time when given."""
    torch = _torch()
    W1, W2 = params["W1"], params["W2"]
    H, F = W1.shape
    D = W2.shape[0]
    _require_f32("filter parameters and h_time", h_time, *[params[k] for k in ("W1", "b1", "W2", "b2", "alpha")])
    dev = W1.device
    mode = mode_for(len(point_shape)) if mode is None else mode
    if spectrum is None:
        spectrum = torch.empty(spectrum_bytes(point_shape, D, mode), dtype=torch.uint8, device=dev)
    ws = _workspace(filter_workspace_bytes(point_shape, D, mode), dev)
    p = FilterParams(F, H, D, _ptr(W1), _ptr(params["b1"]), _ptr(W2), _ptr(params["b2"]), _ptr(params["alpha"]))
    _check(lib().hyena_filter_gen(ctypes.byref(p), dims_of(point_shape), mode, _ptr(h_time), _ptr(spectrum),
                                  _ptr(ws), 0 if ws is None else ws.numel(), _stream(W1)),
           "hyena_filter_gen")
    # ws may be released now: the caching allocator hands it out again only to work ordered after
    # this call on the same stream.
    return spectrum


class SpectrumCache:
    """Filter spectra cached per (parameters, grid, mode): the implicit filter is a function of the position, so
    one set of parameters gives one spectrum per grid size, which the operator reuses on every call at that size
    (the Hyena study note's filter adapts to any sequence length; it need not be rebuilt per call).

    The key holds, for every parameter tensor, its device, storage address, shape and version counter (torch
    bumps the counter on every in-place change), so updating a parameter in place, or passing other tensors,
    builds a new spectrum.  At most `max_entries` spectra are kept (least recently used dropped first).
    `builder(params, point_shape, mode)` makes a spectrum (filter_gen by default)."""

    def __init__(self, max_entries: int = 64, builder=None):
        from collections import OrderedDict
        self.max_entries = max_entries
        self.builder = builder if builder is not None else (lambda p, shape, mode: filter_gen(p, shape, mode=mode))
        self._d = OrderedDict()
        self.builds = 0

    @staticmethod
    def key(params: dict, point_shape: Sequence[int], mode: int):
        parts = tuple((k, str(t.device), t.data_ptr(), tuple(t.shape), t._version) for k, t in sorted(params.items()))
        return parts, tuple(int(n) for n in point_shape), int(mode)

    def get(self, params: dict, point_shape: Sequence[int], mode: Optional[int] = None):
        mode = mode_for(len(point_shape)) if mode is None else mode
        k = self.key(params, point_shape, mode)
        sp = self._d.get(k)
        if sp is None:
            sp = self.builder(params, tuple(point_shape), mode)
            self.builds += 1
            self._d[k] = sp
            while len(self._d) > self.max_entries:
                self._d.popitem(last=False)
        else:
            self._d.move_to_end(k)
        return sp

    def clear(self):
        self._d.clear()


_default_cache = None


def default_spectrum_cache() -> SpectrumCache:
    global _default_cache
    if _default_cache is None:
        _default_cache = SpectrumCache()
    return _default_cache


def hyena(v, xs: Sequence, filter_params: Sequence[dict], y=None, mode: Optional[int] = None,
          cache: Optional[SpectrumCache] = None):
    """The order-N operator from filter parameters (one dict per order, as filter_gen takes): spectra come from
    the cache (built on the first call at a grid size, reused afterwards), then operator()."""
    cache = default_spectrum_cache() if cache is None else cache
    pts = tuple(v.shape[2:])
    spectra = [cache.get(p, pts, mode) for p in filter_params]
    return operator(v, xs, spectra, y=y, mode=mode)


def film_filter_workspace_bytes(B: int, point_shape: Sequence[int], D: int, mode: Optional[int] = None) -> int:
    n = ctypes.c_size_t()
    mode = mode_for(len(point_shape)) if mode is None else mode
    _check(lib().hyena_film_filter_workspace_bytes(B, dims_of(point_shape), mode, D, ctypes.byref(n)),
           "hyena_film_filter_workspace_bytes")
    return n.value


FILM_KEYS = ("q", "A1", "a1", "omega0", "A2", "a2", "A3", "a3", "G1", "g1", "P1", "p1", "G2", "g2", "P2", "p2",
             "sigma")


def _require_f32(what: str, *tensors):
    torch = _torch()
    for t in tensors:
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{what} must be float32, got {t.dtype}")


def film_filter_gen(params: dict, registers, point_shape: Sequence[int], h_time=None, spectrum=None,
                    mode: Optional[int] = None, ws=None, taps_only: bool = False):
    """Input-dependent filters of one order for every sample.  params: dict of CUDA float32 tensors
    (FILM_KEYS; A3 [D, H], G1 [H, E], ...); registers: [B, R, E] CUDA float32.  Returns the spectra of
    the B*D filters (opaque uint8 tensor, for mode | PER_SAMPLE); fills h_time [B, D, taps] when given.
    taps_only (with h_time): no spectrum is built and None is returned."""
    torch = _torch()
    B, R, E = registers.shape
    H = params["A2"].shape[0]
    D = params["A3"].shape[0]
    _require_f32("registers, FiLM-SIREN parameters and h_time", registers, h_time, *[params[k] for k in FILM_KEYS])
    if params["A1"].shape[1] != len(point_shape) or params["q"].shape[0] != E:
        raise ValueError("A1 needs one column per grid axis and q one entry per register feature")
    dev = registers.device
    mode = mode_for(len(point_shape)) if mode is None else mode
    if taps_only:
        if h_time is None:
            raise ValueError("taps_only needs h_time")
        spectrum = None
    elif spectrum is None:
        spectrum = torch.empty(spectrum_bytes(point_shape, B * D, mode | PER_SAMPLE), dtype=torch.uint8, device=dev)
    if ws is None:
        ws = _workspace(film_filter_workspace_bytes(B, point_shape, D, mode), dev)
    p = FilmParams(E, H, D, *[_ptr(params[k]) for k in FILM_KEYS])
    _check(lib().hyena_film_filter_gen(ctypes.byref(p), B, R, _ptr(registers), dims_of(point_shape), mode,
                                       _ptr(h_time), _ptr(spectrum), _ptr(ws), ws.numel(), _stream(registers)),
           "hyena_film_filter_gen")
    return spectrum


def projection(x, W, order: int, bias=None, outs: Optional[Sequence] = None):
    """[v, x_1, ..., x_N] (channel-major [B, D, L] each) = split(x W^T + bias); x: [B, L, d_model] token-major,
    W: [(order+1) D, d_model], both CUDA tensors of one dtype (float32 or bfloat16); bias: float32 or None."""
    torch = _torch()
    B, L, K = x.shape
    M = W.shape[0]
    if W.shape[1] != K or M % (order + 1) or W.dtype != x.dtype:
        raise ValueError("W must be [(order+1)*D, d_model] of x's dtype")
    _require_f32("bias", bias)
    if bias is not None and bias.numel() != M:
        raise ValueError("bias must hold one value per projected channel")
    D = M // (order + 1)
    if outs is None:
        outs = [torch.empty((B, D, L), dtype=x.dtype, device=x.device) for _ in range(order + 1)]
    oa = (ctypes.c_void_p * (order + 1))(*[_ptr(o) for o in outs])
    _check(lib().hyena_projection(order, B, L, K, D, _dtype_code(x), _ptr(x), _ptr(W), _ptr(bias), oa, _stream(x)),
           "hyena_projection")
    return list(outs)


def fftconv(u, spectrum, gate=None, y=None, mode: Optional[int] = None):
    """y = gate * (h conv u) (or h conv u when gate is None); u: [B, D, *points]."""
    torch = _torch()
    B, D = u.shape[:2]
    pts = tuple(u.shape[2:])
    mode = mode_for(len(pts)) if mode is None else mode
    if y is None:
        y = torch.empty_like(u)
    dt = _dtype_code(u)
    ws = _workspace(workspace_bytes(1, B, D, pts, dt, mode), u.device)
    _check(lib().hyena_fftconv(B, D, dims_of(pts), dt, mode, _ptr(u), _ptr(spectrum), _ptr(gate), _ptr(y),
                               _ptr(ws), 0 if ws is None else ws.numel(), _stream(u)), "hyena_fftconv")
    return y


def operator(v, xs: Sequence, spectra: Sequence, y=None, ws=None, mode: Optional[int] = None):
    """y = x_N * (h_N conv (... x_1 * (h_1 conv v))); v, xs[i]: [B, D, *points]; spectra from filter_gen."""
    torch = _torch()
    B, D = v.shape[:2]
    pts = tuple(v.shape[2:])
    order = len(xs)
    if len(spectra) != order:
        raise ValueError("need one spectrum per gate")
    mode = mode_for(len(pts)) if mode is None else mode
    if y is None:
        y = torch.empty_like(v)
    dt = _dtype_code(v)
    for x in xs:
        if x.dtype != v.dtype or x.shape != v.shape:
            raise ValueError("gates must match v in shape and dtype")
    if ws is None:
        ws = _workspace(workspace_bytes(order, B, D, pts, dt, mode), v.device)
    xa = (ctypes.c_void_p * order)(*[_ptr(x) for x in xs])
    sa = (ctypes.c_void_p * order)(*[_ptr(s) for s in spectra])
    _check(lib().hyena_operator(order, B, D, dims_of(pts), dt, mode, _ptr(v), xa, sa, _ptr(y), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(v)), "hyena_operator")
    return y


def operator_noalloc(v, xs: Sequence, spectra: Sequence, y, mode: Optional[int] = None):
    """The operator through hyena_operator_noalloc: no workspace, and nothing allocated here either, so y
    (the output, shaped and typed like v) is required.  Calls on one device share the library's scratch:
    order them on one stream."""
    B, D = v.shape[:2]
    pts = tuple(v.shape[2:])
    order = len(xs)
    if len(spectra) != order:
        raise ValueError("need one spectrum per gate")
    if y is None or y.shape != v.shape or y.dtype != v.dtype:
        raise ValueError("y must be given, shaped and typed like v")
    for x in xs:
        if x.dtype != v.dtype or x.shape != v.shape:
            raise ValueError("gates must match v in shape and dtype")
    mode = mode_for(len(pts)) if mode is None else mode
    xa = (ctypes.c_void_p * order)(*[_ptr(x) for x in xs])
    sa = (ctypes.c_void_p * order)(*[_ptr(s) for s in spectra])
    _check(lib().hyena_operator_noalloc(order, B, D, dims_of(pts), _dtype_code(v), mode, _ptr(v), xa, sa, _ptr(y),
                                        _stream(v)), "hyena_operator_noalloc")
    return y


def spectrum_export(spectrum, point_shape: Sequence[int], D: int, mode: Optional[int] = None):
    """Engine-ordered spectrum -> complex64 tensor of natural-order bins (testing aid)."""
    torch = _torch()
    mode = mode_for(len(point_shape)) if mode is None else mode
    circ = (mode & ~PER_SAMPLE) == CIRCULAR
    if len(point_shape) == 1:
        shape = (D, (point_shape[0] // 2 if circ else point_shape[0]) + 1)
    else:
        nx, ny, nz = point_shape
        shape = (D, nx, ny, nz // 2 + 1) if circ else (D, 2 * nx, 2 * ny, nz + 1)
    H = torch.zeros(shape, dtype=torch.complex64, device=spectrum.device)
    _check(lib().hyena_spectrum_export(dims_of(point_shape), mode, D, _ptr(spectrum), H.data_ptr(),
                                       _stream(spectrum)), "hyena_spectrum_export")
    return H


def decode_state_bytes(order: int, B: int, D: int, L: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().hyena_decode_state_bytes(order, B, D, L, ctypes.byref(n)), "hyena_decode_state_bytes")
    return n.value


def decode_reset(state, order: int, B: int, D: int, L: int):
    """Clear a decode state (uint8 CUDA tensor of decode_state_bytes bytes) before a new sequence."""
    _check(lib().hyena_decode_reset(order, B, D, L, _ptr(state), state.numel(), _stream(state)), "hyena_decode_reset")


def decode_step(t: int, v_t, x_t: Sequence, taps: Sequence, spectra: Sequence, state, L: int, block: int, y_t=None,
                mode: int = CAUSAL):
    """Token t of every (b, d) row: y_t [B, D] from v_t, x_t[i] [B, D] (float32 or bfloat16, one dtype);
    taps[i]: float32 [D, L] (filter_gen's h_time), spectra[i] from filter_gen; state from
    decode_state_bytes / decode_reset.  mode CAUSAL | PER_SAMPLE: taps [B, D, L] and spectra from
    film_filter_gen."""
    torch = _torch()
    B, D = v_t.shape
    order = len(x_t)
    if len(taps) != order or len(spectra) != order:
        raise ValueError("need one tap row set and one spectrum per gate")
    _require_f32("decode taps", *taps)
    dt = _dtype_code(v_t)
    if y_t is None:
        y_t = torch.empty_like(v_t)
    if any(x.dtype != v_t.dtype for x in x_t) or y_t.dtype != v_t.dtype:
        raise ValueError("v_t, x_t and y_t must share one dtype")
    xa = (ctypes.c_void_p * order)(*[_ptr(x) for x in x_t])
    ta = (ctypes.c_void_p * order)(*[_ptr(h) for h in taps])
    sa = (ctypes.c_void_p * order)(*[_ptr(sp) for sp in spectra])
    _check(lib().hyena_decode_step(order, B, D, L, block, t, dt, mode, _ptr(v_t), xa, ta, sa, _ptr(y_t), _ptr(state),
                                   state.numel(), _stream(v_t)), "hyena_decode_step")
    return y_t


def decode_prefill(v, xs: Sequence, spectra: Sequence, state, L: int, block: int, y=None, mode: int = CAUSAL):
    """The first P tokens at once (v, xs[i]: [B, D, P], P a multiple of block); returns y [B, D, P].  The next
    call is decode_step at t = P."""
    torch = _torch()
    B, D, P = v.shape
    order = len(xs)
    if len(spectra) != order:
        raise ValueError("need one spectrum per gate")
    dt = _dtype_code(v)
    if y is None:
        y = torch.empty_like(v)
    if any(x.dtype != v.dtype or x.shape != v.shape for x in xs) or y.dtype != v.dtype:
        raise ValueError("v, xs and y must share one shape and dtype")
    xa = (ctypes.c_void_p * order)(*[_ptr(x) for x in xs])
    sa = (ctypes.c_void_p * order)(*[_ptr(sp) for sp in spectra])
    _check(lib().hyena_decode_prefill(order, B, D, L, block, P, dt, mode, _ptr(v), xa, sa, _ptr(y), _ptr(state),
                                      state.numel(), _stream(v)), "hyena_decode_prefill")
    return y
