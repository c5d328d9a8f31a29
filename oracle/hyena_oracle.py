"""CPU oracle for the Hyena operator -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path (the HIP library and its
binding) never calls it and shares no code with it.

Everything here is plain NumPy in float64, written for a reader to check against
the pages by eye.  The pages are cited by title:

  [Hyena note]   "Hyena: 암묵적 장거리 컨볼루션으로 어텐션을 완전 대체한 서브-이차 모델"
                 (obsidian-dorae222.pages.dev/20.AI/22.SSM/hyena)
  [EulerStack]   "4. Hyena 상세" (eulerwa.com, EulerStack tutorial, mixers/04_hyena)
  [HyenaND]      "Native Multi-Dimensional Subquadratic Operators via Input Dependent
                 Long Convolutions" (gist.science summary, Korean and Italian copies)
  [SPECTRE news] "FFT의 반격: Self-Attention의 효율적 대안" (news.hada.io digest)

What is computed (y = x_N * (h_N conv (... x_1 * (h_1 conv v)))):

  * positional features phi(t) of the normalised position t/L            [Hyena note, step 2]
  * filter network g = W2 SiLU(W1 phi + b1) + b2, one per order           [Hyena note, listing
    ``ImplicitFilter``; EulerStack YAML ``filter_hidden``]
  * exponential decay window h = g * exp(-alpha t/L)                      [Hyena note, step 2, w(t)]
  * causal linear convolution over the whole sequence                      [EulerStack, "how it works" 2]
  * multiplicative gating, innermost gate x_1 with filter h_1              [Hyena note, step 3 equation;
                                                                           listing ``hyena_operator``]
  * 3-D: non-causal "same" linear convolution by zero-padding every axis
    to twice its size                                                      [HyenaND, method: native N-D
                                                                           convolution; boundary handling]
  * circular (periodic) convolution, no padding, 1-D and 3-D              [HyenaND, boundary handling:
                                                                           circular convolutions for
                                                                           periodic physical systems]
  * the input projection v, x_1..x_N = split(W_proj x), v first           [Hyena note, step 1 equation;
                                                                           listing x.chunk]
  * streaming decode: the same causal operator evaluated token by token,
    every order advancing one position at a time                          [Hyena note, step 3 equation;
                                                                           SPECTRE news, generation
                                                                           support]
  * input-dependent (per-sample) filters: z(x) = softmax-weighted mean of
    the register activations; K = w(c) * f(c; z) with a FiLM-modulated
    SIREN f and a Gaussian window w                                        [HyenaND, method: registers,
                                                                           FiLM conditioning, kernel
                                                                           synthesis, parameterisation]

Readings where the pages are silent (each also listed in the design notes):
  order N = number of filters = number of gates (listing chunks len(filters)+1);
  phi(t) = [sin(2 pi f t/L) for f=1..F/2] + [cos(2 pi f t/L) for f=1..F/2];
  time normalised as t/L for both features and window; one alpha per (order, channel);
  3-D features: per axis 16 frequencies x {sin, cos} of r/n for signed offsets r in [-(n-1), n-1];
  3-D window exp(-alpha |r/n|_2);
  circular mode: indices taken modulo the grid, no padding; 1-D keeps the causal taps t = 0..L-1
  (one period), 3-D evaluates the filter on the centred offsets r in [-n/2, n/2)^3, placed at r mod n.
  input-dependent filters: the register activations arrive as an input [B, R, E]; softmax weights
  from a learned score vector q (a[b, r] = softmax_r(q . reg[b, r])); two FiLM-modulated sine layers
  (gamma = G z + g scales the pre-activation omega0 * (A1 c + a1) or A2 h1 + a2, beta = P z + p is
  added) and a linear read-out; omega0 one scale per first-layer unit; window exp(-|c|^2 / (2 sigma_d^2));
  coordinates c = t/L (1-D) or r/n per axis (3-D), as for the exponential filter.

Pins (each function is checked against something other than itself in
tests/test_oracle.py): direct sum vs FFT form, numpy.convolve special case,
first-order-recurrence and geometric-sum closed forms, delta and unit-delay
filters, linearity, causality, 3-D brute force, separable 3-D products,
hand-computed worked examples under tests/golden/; circular mode: direct sum vs
FFT, cyclic shifts by delta filters, numpy.convolve when nothing wraps, the
geometric-filter eigenvalue closed form, 3-D brute force and separable products,
and the circular 3-D filter against the linear one at shared offsets; input-dependent filters: the
plain mean and the two-register logistic closed form of the softmax summary, permutation invariance,
closed-form SIREN outputs with and without FiLM terms, the Gaussian window against the normal density
and its separability, kernels that follow the registers sample by sample, axis order of the 3-D taps,
and per-(b, d) filters in the operator against row-by-row direct sums; the projection: a pure-Python
triple loop on tiny shapes and block-identity weights that return the input transposed and scaled;
streaming decode: the whole-sequence operator (FFT form), unit-delay filters that shift each order by one
token, delta filters (a pointwise product), and prefix stability (outputs before t do not move when
later inputs change).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "positional_features_1d", "positional_features_3d", "silu", "filter_network",
    "implicit_filter_1d", "implicit_filter_3d", "causal_conv_direct", "causal_conv_fft",
    "linear_conv3d_direct", "linear_conv3d_fft", "hyena_operator_rows", "hyena_operator_3d",
    "rel_l2_per_row", "filter_offsets_3d_circular", "implicit_filter_3d_circular", "circular_conv_direct",
    "circular_conv_fft", "circular_conv3d_direct", "circular_conv3d_fft", "register_summary", "film_siren",
    "gaussian_window", "input_dependent_filter_1d", "input_dependent_filter_3d", "input_projection",
    "hyena_decode_stream",
]


# --------------------------------------------------------------------------------------------
# implicit filter  [Hyena note, step 2: h(t) = FFN(pos_enc(t)) * w(t), w(t) = exp(-alpha t)]
# --------------------------------------------------------------------------------------------

def positional_features_1d(L: int, F: int = 64, t: Optional[np.ndarray] = None) -> np.ndarray:
    """phi(t) for t = 0..L-1 (or the given t): [L, F] float64.

    Sinusoidal features of the normalised position t/L ([EulerStack] "how it works" 1: a small
    MLP over sinusoidal features of the position).  Block order: F/2 sines, then F/2 cosines,
    frequencies 1..F/2 cycles per sequence.
    """
    if t is None:
        t = np.arange(L, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    f = np.arange(1, F // 2 + 1, dtype=np.float64)
    ang = 2.0 * math.pi * np.outer(t, f) / L
    return np.concatenate([np.sin(ang), np.cos(ang)], axis=1)


def positional_features_3d(offsets: np.ndarray, n: int, F: int = 96) -> np.ndarray:
    """phi(r) for signed integer offsets r [P, 3]: [P, F] float64.

    Per axis (x, y, z in that order): F/6 sines then F/6 cosines of 2 pi f r_a / n, f = 1..F/6.
    """
    r = np.asarray(offsets, dtype=np.float64) / n
    per = F // 6
    f = np.arange(1, per + 1, dtype=np.float64)
    cols = []
    for a in range(3):
        ang = 2.0 * math.pi * np.outer(r[:, a], f)
        cols.append(np.sin(ang))
        cols.append(np.cos(ang))
    return np.concatenate(cols, axis=1)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z)  ([Hyena note] listing ``nn.SiLU``)."""
    return z / (1.0 + np.exp(-z))


def filter_network(phi: np.ndarray, p: dict, channels: Optional[Sequence[int]] = None) -> np.ndarray:
    """g = W2 SiLU(W1 phi + b1) + b2 for every row of phi: [P, D_sel] float64.

    W1 [H, F], b1 [H], W2 [D, H], b2 [D] ([Hyena note] listing ``filter_fn``: Linear, SiLU, Linear;
    [EulerStack] YAML ``filter_hidden: 64``).
    """
    W1 = np.asarray(p["W1"], np.float64)
    b1 = np.asarray(p["b1"], np.float64)
    W2 = np.asarray(p["W2"], np.float64)
    b2 = np.asarray(p["b2"], np.float64)
    if channels is not None:
        ch = np.asarray(channels, dtype=np.int64)
        W2, b2 = W2[ch], b2[ch]
    z = phi @ W1.T + b1
    a = silu(z)
    return a @ W2.T + b2


def implicit_filter_1d(p: dict, L: int, channels: Optional[Sequence[int]] = None) -> np.ndarray:
    """h[d, t] = g[d](t) * exp(-alpha_d t / L), t = 0..L-1: [D_sel, L] float64."""
    F = np.asarray(p["W1"]).shape[1]
    g = filter_network(positional_features_1d(L, F), p, channels)      # [L, D_sel]
    alpha = np.asarray(p["alpha"], np.float64)
    if channels is not None:
        alpha = alpha[np.asarray(channels, dtype=np.int64)]
    t = np.arange(L, dtype=np.float64)
    window = np.exp(-np.outer(alpha, t) / L)                             # [D_sel, L]
    return g.T * window


def filter_offsets_3d(n: int) -> np.ndarray:
    """All signed offsets r in [-(n-1), n-1]^3, x slowest: [(2n-1)^3, 3] int64."""
    a = np.arange(-(n - 1), n, dtype=np.int64)
    X, Y, Z = np.meshgrid(a, a, a, indexing="ij")
    return np.stack([X.ravel(), Y.ravel(), Z.ravel()], axis=1)


def implicit_filter_3d(p: dict, n: int, channels: Optional[Sequence[int]] = None) -> np.ndarray:
    """h[d, rx, ry, rz] on offsets [-(n-1), n-1]^3: [D_sel, 2n-1, 2n-1, 2n-1] float64.

    h = g(r) * exp(-alpha_d |r/n|_2): a coordinate MLP on the grid offsets times a decaying window
    ([HyenaND] method, kernel on a continuous coordinate grid; the window shape follows the 1-D
    exponential of [Hyena note], step 2).
    """
    F = np.asarray(p["W1"]).shape[1]
    r = filter_offsets_3d(n)
    g = filter_network(positional_features_3d(r, n, F), p, channels)    # [P, D_sel]
    alpha = np.asarray(p["alpha"], np.float64)
    if channels is not None:
        alpha = alpha[np.asarray(channels, dtype=np.int64)]
    rad = np.sqrt(np.sum((r.astype(np.float64) / n) ** 2, axis=1))      # [P]
    h = g.T * np.exp(-np.outer(alpha, rad))
    m = 2 * n - 1
    return h.reshape(-1, m, m, m)


def filter_offsets_3d_circular(n: int) -> np.ndarray:
    """One period of signed offsets, centred: r in [-n/2, n/2)^3, x slowest: [n^3, 3] int64."""
    a = np.arange(-(n // 2), n - n // 2, dtype=np.int64)
    X, Y, Z = np.meshgrid(a, a, a, indexing="ij")
    return np.stack([X.ravel(), Y.ravel(), Z.ravel()], axis=1)


def implicit_filter_3d_circular(p: dict, n: int, channels: Optional[Sequence[int]] = None) -> np.ndarray:
    """Periodic 3-D filter: h[d, i, j, k] = g(r) exp(-alpha_d |r/n|_2) at the centred offset r with
    r = (i, j, k) mod n: [D_sel, n, n, n] float64 (same network and window as the zero-padded mode)."""
    F = np.asarray(p["W1"]).shape[1]
    r = filter_offsets_3d_circular(n)
    g = filter_network(positional_features_3d(r, n, F), p, channels)    # [n^3, D_sel]
    alpha = np.asarray(p["alpha"], np.float64)
    if channels is not None:
        alpha = alpha[np.asarray(channels, dtype=np.int64)]
    rad = np.sqrt(np.sum((r.astype(np.float64) / n) ** 2, axis=1))
    vals = g.T * np.exp(-np.outer(alpha, rad))                          # [D_sel, n^3]
    h = np.zeros((vals.shape[0], n, n, n), dtype=np.float64)
    ri = r % n
    h[:, ri[:, 0], ri[:, 1], ri[:, 2]] = vals
    return h


# --------------------------------------------------------------------------------------------
# long convolution  [EulerStack, "how it works" 2: FFT, pointwise product, inverse FFT = convolution;
#                    HyenaND, boundary handling: zero-pad to double size to avoid wrap-around]
# --------------------------------------------------------------------------------------------

def causal_conv_direct(u: np.ndarray, h: np.ndarray) -> np.ndarray:
    """c[t] = sum_{s=0..t} h[t-s] u[s]  (the definition; O(L^2); last axis is time)."""
    u = np.asarray(u, np.float64)
    h = np.asarray(h, np.float64)
    L = u.shape[-1]
    out = np.zeros(np.broadcast_shapes(u.shape, h.shape), dtype=np.float64)
    for t in range(L):
        out[..., t] = np.sum(h[..., t::-1] * u[..., : t + 1], axis=-1)
    return out


def causal_conv_fft(u: np.ndarray, h: np.ndarray) -> np.ndarray:
    """Same result through the convolution theorem on a 2L zero-padded grid, truncated to L."""
    u = np.asarray(u, np.float64)
    h = np.asarray(h, np.float64)
    L = u.shape[-1]
    n = 2 * L
    return np.fft.irfft(np.fft.rfft(u, n) * np.fft.rfft(h, n), n)[..., :L]


def linear_conv3d_direct(u: np.ndarray, h: np.ndarray) -> np.ndarray:
    """c[p] = sum_{q in [0,n)^3} h[p-q] u[q], p in [0,n)^3 (the definition, brute force).

    u: [n, n, n]; h: [2n-1]^3 indexed by offset + (n-1).
    """
    u = np.asarray(u, np.float64)
    h = np.asarray(h, np.float64)
    n = u.shape[0]
    c = np.zeros_like(u)
    for px in range(n):
        for py in range(n):
            for pz in range(n):
                # offsets p - q for q over the grid, shifted into h's index range
                hx = slice(px + n - 1, px - 1 if px > 0 else None, -1)
                hy = slice(py + n - 1, py - 1 if py > 0 else None, -1)
                hz = slice(pz + n - 1, pz - 1 if pz > 0 else None, -1)
                c[px, py, pz] = np.sum(h[hx, hy, hz] * u)
    return c


def linear_conv3d_fft(u: np.ndarray, h: np.ndarray) -> np.ndarray:
    """Same result via 3-D real FFTs on a (2n)^3 grid: h[r] placed at r mod 2n, output cropped to [0,n)^3.

    Exact because |p - q| <= n-1 < 2n - (n-1) on every axis, so no wrapped term lands in the crop.
    Leading axes of u / h are batch axes.
    """
    u = np.asarray(u, np.float64)
    h = np.asarray(h, np.float64)
    n = u.shape[-1]
    m = 2 * n
    hp = np.zeros(h.shape[:-3] + (m, m, m), dtype=np.float64)
    idx = np.arange(-(n - 1), n) % m
    hp[..., idx[:, None, None], idx[None, :, None], idx[None, None, :]] = h
    axes = (-3, -2, -1)
    U = np.fft.rfftn(u, s=(m, m, m), axes=axes)
    Hs = np.fft.rfftn(hp, s=(m, m, m), axes=axes)
    return np.fft.irfftn(U * Hs, s=(m, m, m), axes=axes)[..., :n, :n, :n]


def circular_conv_direct(u: np.ndarray, h: np.ndarray) -> np.ndarray:
    """c[t] = sum_{s=0..L-1} h[(t-s) mod L] u[s]  (periodic boundary, the definition; O(L^2))."""
    u = np.asarray(u, np.float64)
    h = np.asarray(h, np.float64)
    L = u.shape[-1]
    s = np.arange(L)
    out = np.zeros(np.broadcast_shapes(u.shape, h.shape), dtype=np.float64)
    for t in range(L):
        out[..., t] = np.sum(h[..., (t - s) % L] * u, axis=-1)
    return out


def circular_conv_fft(u: np.ndarray, h: np.ndarray) -> np.ndarray:
    """Same result through the convolution theorem on the L-point grid itself (no padding)."""
    u = np.asarray(u, np.float64)
    h = np.asarray(h, np.float64)
    L = u.shape[-1]
    return np.fft.irfft(np.fft.rfft(u) * np.fft.rfft(h), L)


def circular_conv3d_direct(u: np.ndarray, h: np.ndarray) -> np.ndarray:
    """c[p] = sum_{q in [0,n)^3} h[(p-q) mod n] u[q] (periodic on every axis; brute force).

    u, h: [n, n, n]; h indexed by offset mod n.
    """
    u = np.asarray(u, np.float64)
    h = np.asarray(h, np.float64)
    n = u.shape[0]
    q = np.arange(n)
    c = np.zeros_like(u)
    for px in range(n):
        for py in range(n):
            for pz in range(n):
                hx = (px - q) % n
                hy = (py - q) % n
                hz = (pz - q) % n
                c[px, py, pz] = np.sum(h[hx[:, None, None], hy[None, :, None], hz[None, None, :]] * u)
    return c


def circular_conv3d_fft(u: np.ndarray, h: np.ndarray) -> np.ndarray:
    """Same result via 3-D real FFTs on the n^3 grid itself; leading axes are batch axes."""
    u = np.asarray(u, np.float64)
    h = np.asarray(h, np.float64)
    n = u.shape[-1]
    axes = (-3, -2, -1)
    return np.fft.irfftn(np.fft.rfftn(u, axes=axes) * np.fft.rfftn(h, axes=axes), s=(n, n, n), axes=axes)


# --------------------------------------------------------------------------------------------
# input projection  [Hyena note, step 1: v, x_1, ..., x_N = split(W_proj x); listing: x.chunk(N + 1)]
# --------------------------------------------------------------------------------------------

def input_projection(x: np.ndarray, W: np.ndarray, bias: Optional[np.ndarray], order: int) -> List[np.ndarray]:
    """[v, x_1, ..., x_N] from token-major inputs x [B, L, Dm]: u = x W^T (+ bias), u [B, L, (N+1) D],
    split along the channel axis into N + 1 chunks of D in that order (v first), each returned
    channel-major [B, D, L] float64.  W [(N+1) D, Dm] (a learned linear map, weight rows = outputs)."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    u = x @ W.T
    if bias is not None:
        u = u + np.asarray(bias, np.float64)
    D = W.shape[0] // (order + 1)
    return [np.ascontiguousarray(np.swapaxes(u[..., j * D:(j + 1) * D], -1, -2)) for j in range(order + 1)]


# --------------------------------------------------------------------------------------------
# input-dependent filters  [HyenaND, method: registers and FiLM; kernel synthesis K(x) = w(c) f(c; z(x));
#                           kernel parameterisation: coordinate SIREN with multi-frequency omega_0]
# --------------------------------------------------------------------------------------------

def register_summary(registers: np.ndarray, q: np.ndarray) -> np.ndarray:
    """z(x) per sample: the softmax-weighted mean of the R register activations: [B, E] float64.

    registers [B, R, E] (the register tokens after the layers that processed them together with the
    grid), q [E] a learned score vector; weights a[b, r] = softmax over r of q . registers[b, r].
    """
    reg = np.asarray(registers, np.float64)
    s = reg @ np.asarray(q, np.float64)                                  # [B, R] scores
    s = s - s.max(axis=1, keepdims=True)
    a = np.exp(s)
    a = a / a.sum(axis=1, keepdims=True)
    return np.einsum("br,bre->be", a, reg)


def film_siren(coords: np.ndarray, z: np.ndarray, p: dict) -> np.ndarray:
    """f(c; z) for every coordinate row c of coords [P, n] and one sample's z [E]: [P, D] float64.

    Two sine layers, each modulated feature-wise by z (gamma = G z + g scales the pre-activation,
    beta = P z + p shifts it), then a linear read-out to the D channels:
        s1 = omega0 * (A1 c + a1);   h1 = sin(gamma1 * s1 + beta1)
        s2 = A2 h1 + a2;             h2 = sin(gamma2 * s2 + beta2)
        f  = A3 h2 + a3
    omega0 [H] is one frequency scale per first-layer unit (blocks of units at different scales).
    """
    f64 = lambda k: np.asarray(p[k], np.float64)
    z = np.asarray(z, np.float64)
    c = np.asarray(coords, np.float64)
    g1, b1 = f64("G1") @ z + f64("g1"), f64("P1") @ z + f64("p1")
    g2, b2 = f64("G2") @ z + f64("g2"), f64("P2") @ z + f64("p2")
    s1 = f64("omega0") * (c @ f64("A1").T + f64("a1"))
    h1 = np.sin(g1 * s1 + b1)
    s2 = h1 @ f64("A2").T + f64("a2")
    h2 = np.sin(g2 * s2 + b2)
    return h2 @ f64("A3").T + f64("a3")


def gaussian_window(coords: np.ndarray, sigma: np.ndarray) -> np.ndarray:
    """w[d, c] = exp(-|c|^2 / (2 sigma_d^2)) for coords [P, n]: [D, P] float64."""
    r2 = np.sum(np.asarray(coords, np.float64) ** 2, axis=1)
    sig = np.asarray(sigma, np.float64)
    return np.exp(-np.outer(1.0 / (2.0 * sig * sig), r2))


def _input_dependent(p: dict, registers: np.ndarray, coords: np.ndarray) -> np.ndarray:
    z = register_summary(registers, p["q"])
    w = gaussian_window(coords, p["sigma"])                              # [D, P]
    return np.stack([film_siren(coords, z[b], p).T * w for b in range(z.shape[0])])


def input_dependent_filter_1d(p: dict, registers: np.ndarray, L: int) -> np.ndarray:
    """K[b, d, t] = w_d(t/L) f_d(t/L; z_b), t = 0..L-1: [B, D, L] float64 (taps of the causal or
    periodic 1-D convolution; coordinate normalised as t/L like the exponential filter)."""
    c = (np.arange(L, dtype=np.float64) / L)[:, None]
    return _input_dependent(p, registers, c)


def input_dependent_filter_3d(p: dict, registers: np.ndarray, n: int, circular: bool = False) -> np.ndarray:
    """K[b, d, ...] on the 3-D offsets, coordinate r/n per axis: zero-padded [B, D, 2n-1, 2n-1, 2n-1]
    (index = offset + n-1), or periodic [B, D, n, n, n] (centred offsets placed at r mod n)."""
    r = filter_offsets_3d_circular(n) if circular else filter_offsets_3d(n)
    vals = _input_dependent(p, registers, r.astype(np.float64) / n)      # [B, D, P]
    if not circular:
        m = 2 * n - 1
        return vals.reshape(vals.shape[0], vals.shape[1], m, m, m)
    h = np.zeros(vals.shape[:2] + (n, n, n), dtype=np.float64)
    ri = r % n
    h[:, :, ri[:, 0], ri[:, 1], ri[:, 2]] = vals
    return h


# --------------------------------------------------------------------------------------------
# the operator  [Hyena note, step 3 equation and listing ``hyena_operator``:
#                v, x_1..x_N chunks; for (h_i, x_i): v <- (h_i conv v) * x_i]
# --------------------------------------------------------------------------------------------

def hyena_operator_rows(v: np.ndarray, xs: Sequence[np.ndarray], hs: Sequence[np.ndarray],
                        direct: bool = False, circular: bool = False) -> np.ndarray:
    """Order-N recurrence on a batch of independent rows (causal, or periodic with ``circular``).

    v, xs[i]: [..., R, L] (any float dtype, taken as exact values); hs[i]: [R, L] filter per row
    (broadcast over leading axes).  Returns y = u_N as float64.
    """
    if circular:
        conv = circular_conv_direct if direct else circular_conv_fft
    else:
        conv = causal_conv_direct if direct else causal_conv_fft
    u = np.asarray(v, np.float64)
    for h, x in zip(hs, xs):
        u = np.asarray(x, np.float64) * conv(u, h)
    return u


def hyena_decode_stream(v: np.ndarray, xs: Sequence[np.ndarray], hs: Sequence[np.ndarray]) -> np.ndarray:
    """Streaming (token-by-token) evaluation of the causal operator: at each position t, in increasing
    t, every order advances by one token using only positions <= t,

        u_0[t] = v[t],  u_i[t] = x_i[t] * sum_{s=0..t} h_i[t-s] u_{i-1}[s],  y[t] = u_N[t]

    ([Hyena note] step 3 equation, evaluated in generation order; [SPECTRE news] generation support:
    a spectral mixer that decodes one token at a time).  How a decoder caches the prefix changes only
    the rounding order, so this is the plain per-token definition.  v, xs[i]: [R, L]; hs[i]: [R, L]
    (broadcast like hyena_operator_rows).  Returns y [R, L] float64.
    """
    v = np.asarray(v, np.float64)
    xs = [np.asarray(x, np.float64) for x in xs]
    hs = [np.broadcast_to(np.asarray(h, np.float64), v.shape) for h in hs]
    L = v.shape[-1]
    hist = [np.zeros_like(v) for _ in xs]          # hist[i][..., s] = u_i's input u_{i-1}[s]
    y = np.zeros_like(v)
    for t in range(L):
        u = v[..., t]
        for i, (h, x) in enumerate(zip(hs, xs)):
            hist[i][..., t] = u
            c = np.sum(h[..., t::-1] * hist[i][..., : t + 1], axis=-1)
            u = x[..., t] * c
        y[..., t] = u
    return y


def hyena_operator_3d(v: np.ndarray, xs: Sequence[np.ndarray], hs: Sequence[np.ndarray],
                      direct: bool = False, circular: bool = False) -> np.ndarray:
    """Order-N recurrence with non-causal 3-D convolutions: zero-padded, or periodic with ``circular``.

    v, xs[i]: [C, n, n, n]; hs[i]: [C, 2n-1, 2n-1, 2n-1] (zero-padded) or [C, n, n, n] (periodic).
    """
    u = np.asarray(v, np.float64)
    direct_fn = circular_conv3d_direct if circular else linear_conv3d_direct
    fft_fn = circular_conv3d_fft if circular else linear_conv3d_fft
    for h, x in zip(hs, xs):
        if direct:
            c = np.stack([direct_fn(u[j], h[j]) for j in range(u.shape[0])])
        else:
            c = fft_fn(u, h)
        u = np.asarray(x, np.float64) * c
    return u


def rel_l2_per_row(y: np.ndarray, ref: np.ndarray, point_axes: int = 1) -> np.ndarray:
    """||y - ref||_2 / ||ref||_2 per row, where a row is the last ``point_axes`` axes (1 for a
    sequence, 3 for a volume) and every leading index (b, d) names one row."""
    ref = np.asarray(ref, np.float64)
    npts = int(np.prod(ref.shape[ref.ndim - point_axes:]))
    rows = ref.reshape(-1, npts)
    ys = np.asarray(y, np.float64).reshape(rows.shape)
    num = np.sqrt(np.sum((ys - rows) ** 2, axis=1))
    den = np.sqrt(np.sum(rows ** 2, axis=1))
    return num / np.where(den == 0, 1.0, den)
