"""Pins for the CPU oracle: every function is checked against something other than itself
(hand-worked examples, closed forms, library routines, brute force, invariants)."""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal

from oracle import hyena_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _params(F, H, D, rng, alpha=(0.3, 3.0)):
    return dict(W1=rng.standard_normal((H, F)) * 0.3, b1=rng.standard_normal(H) * 0.1,
                W2=rng.standard_normal((D, H)) * 0.3, b2=rng.standard_normal(D) * 0.1,
                alpha=rng.uniform(*alpha, size=D))


# ---------------------------------------------------------------- worked examples (by hand)

def test_golden_causal_conv(golden):
    g = golden["causal_conv_4"]
    np.testing.assert_array_equal(orc.causal_conv_direct(g["u"], g["h"]), g["c"])
    np.testing.assert_allclose(orc.causal_conv_fft(np.array(g["u"], float), np.array(g["h"], float)), g["c"],
                               rtol=0, atol=1e-13)


def test_golden_order2_operator(golden):
    g = golden["order2_operator_3"]
    for direct in (True, False):
        y = orc.hyena_operator_rows(np.array([g["v"]], float), [np.array([g["x1"]], float), np.array([g["x2"]], float)],
                                    [np.array([g["h1"]], float), np.array([g["h2"]], float)], direct=direct)
        np.testing.assert_allclose(y[0], g["y"], rtol=0, atol=1e-13)


def test_golden_conv3d_point_sources(golden):
    g = golden["conv3d_point_sources_n2"]
    n = g["n"]
    r = np.arange(-(n - 1), n)
    h = (100 * (r[:, None, None] + 1) + 10 * (r[None, :, None] + 1) + (r[None, None, :] + 1)).astype(float)
    for key, q in (("delta_at_000", (0, 0, 0)), ("delta_at_111", (1, 1, 1))):
        u = np.zeros((n, n, n))
        u[q] = 1.0
        np.testing.assert_array_equal(orc.linear_conv3d_direct(u, h), g[key])
        np.testing.assert_allclose(orc.linear_conv3d_fft(u, h), g[key], rtol=0, atol=1e-11)


def test_golden_features(golden):
    g = golden["features_quarter_period"]
    phi = orc.positional_features_1d(g["L"], 64, t=np.array([g["t"]]))[0]
    np.testing.assert_allclose(phi[:8], g["sin_first8"], atol=1e-14)
    np.testing.assert_allclose(phi[32:40], g["cos_first8"], atol=1e-14)


# ---------------------------------------------------------------- convolution pins

@pytest.mark.parametrize("L", [1, 2, 3, 17, 64, 257])
def test_direct_matches_fft(L):
    rng = np.random.default_rng(L)
    u = rng.standard_normal((3, L))
    h = rng.standard_normal((3, L))
    d = orc.causal_conv_direct(u, h)
    f = orc.causal_conv_fft(u, h)
    assert np.max(np.abs(d - f)) <= 1e-12 * max(1.0, np.max(np.abs(d)))


@pytest.mark.parametrize("L", [5, 128, 1000])
def test_order1_equals_numpy_convolve(L):
    rng = np.random.default_rng(7 + L)
    u = rng.standard_normal(L)
    h = rng.standard_normal(L)
    ref = np.convolve(u, h)[:L]
    for direct in (True, False):
        y = orc.hyena_operator_rows(u[None], [np.ones((1, L))], [h[None]], direct=direct)[0]
        np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-11)


def _exp_filter_params(D, alpha, F=64, H=64):
    """W1 = 0, b1 = 0, W2 = 0, b2 = 1: the network is the constant 1, so h[t] = exp(-alpha t/L)."""
    return dict(W1=np.zeros((H, F)), b1=np.zeros(H), W2=np.zeros((D, H)), b2=np.ones(D), alpha=np.asarray(alpha, float))


@pytest.mark.parametrize("L", [64, 4096, 1 << 16])
def test_exponential_filter_is_first_order_recurrence(L):
    """h[t] = a^t, a = exp(-alpha/L): the causal convolution equals y[t] = a y[t-1] + u[t] (scipy lfilter)."""
    alpha = np.array([0.01, 0.7, 3.0])
    h = orc.implicit_filter_1d(_exp_filter_params(3, alpha), L)
    a = np.exp(-alpha / L)
    np.testing.assert_allclose(h[:, 1], a, rtol=1e-15)
    rng = np.random.default_rng(L)
    u = rng.standard_normal((3, L))
    got = orc.causal_conv_fft(u, h)
    for d in range(3):
        ref = scipy.signal.lfilter([1.0], [1.0, -a[d]], u[d])
        assert np.linalg.norm(got[d] - ref) <= 1e-12 * np.linalg.norm(ref)


@pytest.mark.slow
def test_exponential_filter_full_length_1M():
    """The same closed form at the 1M-token length of the DNA workload."""
    L = 1 << 20
    alpha = np.array([0.01])
    h = orc.implicit_filter_1d(_exp_filter_params(1, alpha), L)
    u = np.random.default_rng(3).standard_normal((1, L))
    got = orc.causal_conv_fft(u, h)[0]
    ref = scipy.signal.lfilter([1.0], [1.0, -math.exp(-0.01 / L)], u[0])
    assert np.linalg.norm(got - ref) <= 1e-10 * np.linalg.norm(ref)


def test_geometric_sum_closed_form():
    """Constant input with h[t] = a^t gives (1 - a^(t+1)) / (1 - a)."""
    L = 2048
    alpha = np.array([0.5, 2.5])
    h = orc.implicit_filter_1d(_exp_filter_params(2, alpha), L)
    got = orc.causal_conv_fft(np.ones((2, L)), h)
    t = np.arange(L)
    for d in range(2):
        a = math.exp(-alpha[d] / L)
        ref = (1 - a ** (t + 1)) / (1 - a)
        np.testing.assert_allclose(got[d], ref, rtol=1e-11)


def test_delta_filter_gives_product_of_gates():
    rng = np.random.default_rng(11)
    L, N = 300, 3
    v = rng.standard_normal((2, L))
    xs = [rng.standard_normal((2, L)) for _ in range(N)]
    delta = np.zeros((2, L))
    delta[:, 0] = 1
    for direct in (True, False):
        y = orc.hyena_operator_rows(v, xs, [delta] * N, direct=direct)
        np.testing.assert_allclose(y, v * xs[0] * xs[1] * xs[2], rtol=1e-12, atol=1e-12)


def test_unit_delay_shifts_by_one():
    rng = np.random.default_rng(12)
    L = 100
    u = rng.standard_normal((1, L))
    h = np.zeros((1, L))
    h[0, 1] = 1
    for conv in (orc.causal_conv_direct, orc.causal_conv_fft):
        c = conv(u, h)
        np.testing.assert_allclose(c[0, 1:], u[0, :-1], atol=1e-12)
        assert abs(c[0, 0]) < 1e-12


def test_linearity_and_multilinearity():
    rng = np.random.default_rng(13)
    L = 200
    v1, v2 = rng.standard_normal((2, 1, L))
    xs = [rng.standard_normal((1, L)) for _ in range(2)]
    hs = [rng.standard_normal((1, L)) for _ in range(2)]
    op = orc.hyena_operator_rows
    np.testing.assert_allclose(op(2 * v1 - 3 * v2, xs, hs), 2 * op(v1, xs, hs) - 3 * op(v2, xs, hs), rtol=1e-10, atol=1e-9)
    np.testing.assert_allclose(op(v1, [xs[0] * 5, xs[1]], hs), 5 * op(v1, xs, hs), rtol=1e-11, atol=1e-9)
    np.testing.assert_allclose(op(v1, xs, [hs[0], hs[1] * -2]), -2 * op(v1, xs, hs), rtol=1e-11, atol=1e-9)


def test_causality():
    rng = np.random.default_rng(14)
    L, t0 = 256, 97
    v = rng.standard_normal((1, L))
    xs = [rng.standard_normal((1, L)) for _ in range(2)]
    hs = [rng.standard_normal((1, L)) for _ in range(2)]
    v2 = v.copy()
    v2[0, t0] += 10.0
    y1 = orc.hyena_operator_rows(v, xs, hs, direct=True)
    y2 = orc.hyena_operator_rows(v2, xs, hs, direct=True)
    np.testing.assert_array_equal(y1[0, :t0], y2[0, :t0])
    assert np.any(y1[0, t0:] != y2[0, t0:])
    f1 = orc.hyena_operator_rows(v, xs, hs)
    f2 = orc.hyena_operator_rows(v2, xs, hs)
    assert np.max(np.abs(f1[0, :t0] - f2[0, :t0])) < 1e-10


# ---------------------------------------------------------------- filter pins

def test_features_at_zero_and_period():
    phi = orc.positional_features_1d(1024, 64)
    np.testing.assert_array_equal(phi[0], np.r_[np.zeros(32), np.ones(32)])
    # cos block at t=L/2: cos(pi f) = (-1)^f
    np.testing.assert_allclose(phi[512, 32:], (-1.0) ** np.arange(1, 33), atol=1e-13)
    # the features are a function of t/L: t=256 at L=1024 equals t=2 at L=8
    np.testing.assert_allclose(orc.positional_features_1d(8, 64, t=np.array([2]))[0], phi[256], atol=1e-13)


def test_silu_identities():
    z = np.linspace(-30, 30, 1001)
    s = orc.silu(z)
    assert orc.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(s - orc.silu(-z), z, atol=1e-12)      # z*sig(z) + z*sig(-z) = z
    assert abs(orc.silu(np.array([30.0]))[0] - 30.0) < 1e-10
    assert abs(orc.silu(np.array([-30.0]))[0]) < 1e-10


def test_filter_network_single_path():
    """W1 with one entry (hidden j <- feature k) and W2 with one entry (channel d <- hidden j):
    g[d](t) = w2 * SiLU(w1 * phi_k(t)); every other channel is its bias."""
    F = H = 64
    D, L = 5, 64
    j, k, d = 3, 40, 2          # feature 40 = cos of frequency 9
    W1 = np.zeros((H, F)); W1[j, k] = 1.5
    W2 = np.zeros((D, H)); W2[d, j] = -2.0
    b2 = np.arange(D, dtype=float)
    p = dict(W1=W1, b1=np.zeros(H), W2=W2, b2=b2, alpha=np.zeros(D))
    h = orc.implicit_filter_1d(p, L)
    t = np.arange(L)
    zz = 1.5 * np.cos(2 * np.pi * 9 * t / L)
    np.testing.assert_allclose(h[d], -2.0 * zz / (1 + np.exp(-zz)) + b2[d], atol=1e-13)
    for other in range(D):
        if other != d:
            np.testing.assert_array_equal(h[other], np.full(L, b2[other]))


def test_filter_network_hidden_bias_single_path():
    """The hidden-layer bias b1 enters before the SiLU, one value per hidden unit: unit j carries a feature
    plus its bias, unit m carries its bias alone (a constant SiLU(b1[m]) at every position), and channel d
    reads both through W2.  A dropped b1, a b1 added after the SiLU, or a b1 indexed by channel instead of
    by unit gives a different value."""
    F = H = 64
    D, L = 5, 64
    j, m, k, d = 3, 17, 40, 2       # feature 40 = cos of frequency 9
    W1 = np.zeros((H, F)); W1[j, k] = 1.5
    b1 = np.linspace(-1.0, 1.0, H); b1[j] = 0.7; b1[m] = -1.2
    W2 = np.zeros((D, H)); W2[d, j] = -2.0; W2[d, m] = 0.5
    b2 = np.arange(D, dtype=float) * 0.25
    p = dict(W1=W1, b1=b1, W2=W2, b2=b2, alpha=np.zeros(D))
    h = orc.implicit_filter_1d(p, L)
    t = np.arange(L)
    zz = 1.5 * np.cos(2 * np.pi * 9 * t / L) + 0.7
    const = 0.5 * (-1.2) / (1 + np.exp(1.2))
    np.testing.assert_allclose(h[d], -2.0 * zz / (1 + np.exp(-zz)) + const + b2[d], atol=1e-13)
    for other in range(D):
        if other != d:
            np.testing.assert_array_equal(h[other], np.full(L, b2[other]))
    # at t = 0 the cosine feature is 1: a value checked by hand, SiLU(2.2) = 2.2 / (1 + e^-2.2)
    assert h[d, 0] == pytest.approx(-2.0 * 2.2 / (1 + math.exp(-2.2)) + 0.5 * -1.2 / (1 + math.exp(1.2)) + 0.5,
                                    abs=1e-13)


def test_filter_network_hidden_bias_3d():
    """The same hidden bias through the 3-D features: unit m with W1 row zero contributes W2[d, m] SiLU(b1[m])
    at every offset, so the filter minus its window-free constant part is the single-feature path."""
    n, D = 4, 3
    F, H = 96, 64
    W1 = np.zeros((H, F)); W1[5, 0] = 2.0             # unit 5 <- sin(2 pi r_x / n)
    b1 = np.zeros(H); b1[5] = -0.3; b1[9] = 0.8
    W2 = np.zeros((D, H)); W2[1, 5] = 1.0; W2[1, 9] = -1.0
    p = dict(W1=W1, b1=b1, W2=W2, b2=np.zeros(D), alpha=np.zeros(D))
    h = orc.implicit_filter_3d(p, n)                  # [D, 7, 7, 7]
    rx = np.arange(-(n - 1), n)
    zz = 2.0 * np.sin(2 * np.pi * rx / n) - 0.3       # depends on r_x only
    ref = zz / (1 + np.exp(-zz)) - 0.8 / (1 + np.exp(-0.8))
    np.testing.assert_allclose(h[1], np.broadcast_to(ref[:, None, None], h[1].shape), atol=1e-13)
    np.testing.assert_array_equal(h[0], 0.0)


def test_window_closed_form_and_channel_subset():
    rng = np.random.default_rng(15)
    p = _params(64, 64, 6, rng)
    L = 512
    h = orc.implicit_filter_1d(p, L)
    g = orc.filter_network(orc.positional_features_1d(L), p)
    t = np.arange(L)
    for d in range(6):
        np.testing.assert_allclose(h[d], g[:, d] * np.exp(-p["alpha"][d] * t / L), rtol=1e-14)
    assert h[3, 0] == pytest.approx(g[0, 3], rel=1e-15)         # window is 1 at t = 0
    np.testing.assert_allclose(orc.implicit_filter_1d(p, L, channels=[4, 1]), h[[4, 1]], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- 3-D pins

@pytest.mark.parametrize("n", [1, 3, 4])
def test_conv3d_brute_force_matches_fft(n):
    rng = np.random.default_rng(20 + n)
    u = rng.standard_normal((n, n, n))
    h = rng.standard_normal((2 * n - 1,) * 3)
    np.testing.assert_allclose(orc.linear_conv3d_fft(u, h), orc.linear_conv3d_direct(u, h), rtol=1e-11, atol=1e-11)


def test_conv3d_separable_is_product_of_1d():
    n = 6
    rng = np.random.default_rng(31)
    a, b, c = rng.standard_normal((3, 2 * n - 1))
    p, q, r = rng.standard_normal((3, n))
    h = np.einsum("i,j,k->ijk", a, b, c)
    u = np.einsum("i,j,k->ijk", p, q, r)

    def same1d(sig, ker):  # c[i] = sum_j ker[i-j] sig[j], ker indexed by offset + n-1
        return np.convolve(sig, ker)[n - 1:2 * n - 1]

    ref = np.einsum("i,j,k->ijk", same1d(p, a), same1d(q, b), same1d(r, c))
    np.testing.assert_allclose(orc.linear_conv3d_fft(u, h), ref, rtol=1e-11, atol=1e-12)


def test_conv3d_point_source_returns_cropped_filter():
    n = 8
    rng = np.random.default_rng(32)
    h = rng.standard_normal((2 * n - 1,) * 3)
    q = (3, 5, 1)
    u = np.zeros((n, n, n)); u[q] = 1.0
    c = orc.linear_conv3d_fft(u, h)
    P = np.arange(n)
    ref = h[np.ix_(P - q[0] + n - 1, P - q[1] + n - 1, P - q[2] + n - 1)]
    np.testing.assert_allclose(c, ref, atol=1e-12)


def test_filter3d_features_and_window():
    n = 4
    rng = np.random.default_rng(33)
    p = _params(96, 64, 3, rng)
    h = orc.implicit_filter_3d(p, n)
    assert h.shape == (3, 7, 7, 7)
    phi0 = orc.positional_features_3d(np.zeros((1, 3), int), n)[0]
    np.testing.assert_array_equal(phi0, np.r_[np.zeros(16), np.ones(16)].tolist() * 3)
    # offset (n/2, 0, 0): x-sines sin(pi f) = 0, x-cosines (-1)^f; window exp(-alpha/2)
    phi = orc.positional_features_3d(np.array([[2, 0, 0]]), n)[0]
    np.testing.assert_allclose(phi[16:32], (-1.0) ** np.arange(1, 17), atol=1e-13)
    g = orc.filter_network(phi[None], p)[0]
    np.testing.assert_allclose(h[:, 2 + 3, 3, 3], g * np.exp(-p["alpha"] * 0.5), rtol=1e-14)
    # W2 = 0, b2 = 1: h = exp(-alpha |r|/n), a radial closed form
    pe = dict(p, W2=np.zeros_like(p["W2"]), b2=np.ones(3))
    he = orc.implicit_filter_3d(pe, n)
    rr = np.arange(-3, 4)
    rad = np.sqrt(rr[:, None, None] ** 2 + rr[None, :, None] ** 2 + rr[None, None, :] ** 2) / n
    for d in range(3):
        np.testing.assert_allclose(he[d], np.exp(-p["alpha"][d] * rad), rtol=1e-14)


def test_operator3d_delta_and_direct():
    n = 3
    rng = np.random.default_rng(34)
    v = rng.standard_normal((2, n, n, n))
    xs = [rng.standard_normal((2, n, n, n)) for _ in range(2)]
    delta = np.zeros((2,) + (2 * n - 1,) * 3)
    delta[:, n - 1, n - 1, n - 1] = 1.0
    np.testing.assert_allclose(orc.hyena_operator_3d(v, xs, [delta, delta]), v * xs[0] * xs[1], atol=1e-12)
    hs = [rng.standard_normal((2,) + (2 * n - 1,) * 3) for _ in range(2)]
    np.testing.assert_allclose(orc.hyena_operator_3d(v, xs, hs), orc.hyena_operator_3d(v, xs, hs, direct=True),
                               rtol=1e-10, atol=1e-10)


def test_rel_l2_per_row():
    ref = np.array([[[3.0, 4.0]], [[1.0, 0.0]]])
    y = ref + np.array([[[0.3, 0.4]], [[0.0, 0.5]]])
    np.testing.assert_allclose(orc.rel_l2_per_row(y, ref), [0.1, 0.5])


# ---------------------------------------------------------------- circular (periodic) mode

def test_golden_circular_conv(golden):
    g = golden["circular_conv_4"]
    np.testing.assert_array_equal(orc.circular_conv_direct(g["u"], g["h"]), g["c"])
    np.testing.assert_allclose(orc.circular_conv_fft(np.array(g["u"], float), np.array(g["h"], float)), g["c"],
                               rtol=0, atol=1e-13)


def test_golden_conv3d_circular_point_sources(golden):
    g = golden["conv3d_circular_point_sources_n2"]
    n = g["n"]
    digit = np.array([2.0, 1.0])          # index 0 <-> offset 0, index 1 <-> offset -1
    h = 100 * digit[:, None, None] + 10 * digit[None, :, None] + digit[None, None, :]
    for key, q in (("delta_at_000", (0, 0, 0)), ("delta_at_111", (1, 1, 1))):
        u = np.zeros((n, n, n))
        u[q] = 1.0
        np.testing.assert_array_equal(orc.circular_conv3d_direct(u, h), g[key])
        np.testing.assert_allclose(orc.circular_conv3d_fft(u, h), g[key], rtol=0, atol=1e-11)


@pytest.mark.parametrize("L", [5, 16, 64])
def test_circular_direct_matches_fft(L):
    rng = np.random.default_rng(L)
    u = rng.standard_normal((3, L))
    h = rng.standard_normal((3, L))
    np.testing.assert_allclose(orc.circular_conv_fft(u, h), orc.circular_conv_direct(u, h), rtol=0, atol=1e-12)


@pytest.mark.parametrize("k", [0, 1, 7, 31])
def test_circular_delta_filter_is_cyclic_shift(k):
    L = 32
    u = np.random.default_rng(k).standard_normal(L)
    h = np.zeros(L)
    h[k] = 1.0
    want = np.roll(u, k)                     # c[t] = u[(t - k) mod L]
    np.testing.assert_array_equal(orc.circular_conv_direct(u, h), want)
    np.testing.assert_allclose(orc.circular_conv_fft(u, h), want, rtol=0, atol=1e-13)


def test_circular_equals_linear_when_nothing_wraps():
    # u and h supported on [0, L/2): no product lands beyond L-1, so the periodic sum is the plain one
    L = 64
    rng = np.random.default_rng(3)
    u = np.zeros(L)
    h = np.zeros(L)
    u[: L // 2] = rng.standard_normal(L // 2)
    h[: L // 2] = rng.standard_normal(L // 2)
    want = np.convolve(u[: L // 2], h[: L // 2])             # length L - 1
    got = orc.circular_conv_direct(u, h)
    np.testing.assert_allclose(got[: L - 1], want, rtol=0, atol=1e-12)
    assert abs(got[L - 1]) < 1e-12


@pytest.mark.parametrize("k", [0, 3, 10])
def test_circular_geometric_filter_eigenvalue(k):
    # h[t] = r^t on one period: a sinusoid of frequency k is an eigenvector of the periodic convolution with
    # eigenvalue H_k = sum_t r^t w^t = (1 - r^L) / (1 - r w), w = exp(-2 pi i k / L) (geometric sum).
    L, r, phase = 24, 0.8, 0.4
    t = np.arange(L)
    h = r ** t
    u = np.cos(2 * math.pi * k * t / L + phase)
    w = np.exp(-2j * math.pi * k / L)
    Hk = (1 - r ** L) / (1 - r * w)
    want = np.real(Hk * np.exp(1j * (2 * math.pi * k * t / L + phase)))
    np.testing.assert_allclose(orc.circular_conv_direct(u, h), want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(orc.circular_conv_fft(u, h), want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [3, 4])
def test_circular3d_brute_force_matches_fft(n):
    rng = np.random.default_rng(n)
    u = rng.standard_normal((n, n, n))
    h = rng.standard_normal((n, n, n))
    np.testing.assert_allclose(orc.circular_conv3d_fft(u, h), orc.circular_conv3d_direct(u, h), rtol=0, atol=1e-12)


def test_circular3d_delta_is_roll():
    n = 4
    u = np.random.default_rng(9).standard_normal((n, n, n))
    h = np.zeros((n, n, n))
    h[1, 3, 2] = 1.0
    want = np.roll(u, (1, 3, 2), axis=(0, 1, 2))
    np.testing.assert_array_equal(orc.circular_conv3d_direct(u, h), want)
    np.testing.assert_allclose(orc.circular_conv3d_fft(u, h), want, rtol=0, atol=1e-13)


def test_circular3d_separable_is_product_of_1d():
    n = 4
    rng = np.random.default_rng(11)
    a, b, c = (rng.standard_normal(n) for _ in range(3))
    f, g, k = (rng.standard_normal(n) for _ in range(3))
    u = np.einsum("i,j,k->ijk", a, b, c)
    h = np.einsum("i,j,k->ijk", f, g, k)
    want = np.einsum("i,j,k->ijk", orc.circular_conv_direct(a, f), orc.circular_conv_direct(b, g),
                     orc.circular_conv_direct(c, k))
    np.testing.assert_allclose(orc.circular_conv3d_direct(u, h), want, rtol=0, atol=1e-12)


def test_filter3d_circular_matches_linear_at_shared_offsets():
    # the periodic filter is the same network and window, evaluated on one centred period of offsets
    n = 6
    rng = np.random.default_rng(5)
    p = _params(96, 64, 3, rng)
    hc = orc.implicit_filter_3d_circular(p, n)
    hl = orc.implicit_filter_3d(p, n)                       # offsets [-(n-1), n-1]^3 at index r + n - 1
    for r in [(0, 0, 0), (-3, 2, 1), (2, -1, -3), (-3, -3, -3), (1, 2, 2)]:
        ci = tuple(x % n for x in r)
        li = tuple(x + n - 1 for x in r)
        np.testing.assert_allclose(hc[(slice(None),) + ci], hl[(slice(None),) + li], rtol=1e-13, atol=0)
    offs = orc.filter_offsets_3d_circular(n)
    assert offs.shape == (n ** 3, 3) and offs.min() == -(n // 2) and offs.max() == n - n // 2 - 1
    assert len({tuple(x % n) for x in offs}) == n ** 3


def test_operator_circular_direct_vs_fft_and_delta():
    rng = np.random.default_rng(21)
    L = 32
    v = rng.standard_normal((2, L))
    xs = [rng.standard_normal((2, L)) for _ in range(2)]
    hs = [rng.standard_normal((2, L)) for _ in range(2)]
    y_d = orc.hyena_operator_rows(v, xs, hs, direct=True, circular=True)
    y_f = orc.hyena_operator_rows(v, xs, hs, circular=True)
    np.testing.assert_allclose(y_f, y_d, rtol=0, atol=1e-12)
    delta = np.zeros((2, L))
    delta[:, 0] = 1.0
    np.testing.assert_allclose(orc.hyena_operator_rows(v, xs, [delta, delta], circular=True), xs[1] * xs[0] * v,
                               rtol=0, atol=1e-14)
    n = 3
    v3 = rng.standard_normal((2, n, n, n))
    x3 = [rng.standard_normal((2, n, n, n)) for _ in range(2)]
    h3 = [rng.standard_normal((2, n, n, n)) for _ in range(2)]
    np.testing.assert_allclose(orc.hyena_operator_3d(v3, x3, h3, circular=True),
                               orc.hyena_operator_3d(v3, x3, h3, direct=True, circular=True), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- spot checks and equivariance

def test_fft_form_spot_checked_by_direct_sums_at_1M():
    # the FFT form at the 1M-token length against O(L) direct dot products at 64 random positions
    L = 1 << 20
    rng = np.random.default_rng(20)
    u = rng.standard_normal(L)
    t = np.arange(L)
    h = np.exp(-0.7 * t / L) * np.cos(2 * math.pi * 5 * t / L)
    c = orc.causal_conv_fft(u, h)
    for t0 in rng.integers(0, L, size=64):
        want = np.dot(h[t0::-1], u[: t0 + 1])
        assert abs(c[t0] - want) <= 1e-9 * (1 + abs(want)), (t0, c[t0], want)


def test_causal_shift_equivariance():
    # delaying the input by s (zero history) delays the causal output by s
    L, s = 256, 37
    rng = np.random.default_rng(22)
    u = rng.standard_normal(L)
    h = rng.standard_normal(L)
    us = np.concatenate([np.zeros(s), u[: L - s]])
    c = orc.causal_conv_direct(u, h)
    cs = orc.causal_conv_direct(us, h)
    np.testing.assert_allclose(cs[s:], c[: L - s], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(cs[:s], np.zeros(s))


def test_circular_shift_equivariance():
    L, s = 64, 23
    rng = np.random.default_rng(23)
    u = rng.standard_normal(L)
    h = rng.standard_normal(L)
    np.testing.assert_allclose(orc.circular_conv_direct(np.roll(u, s), h), np.roll(orc.circular_conv_direct(u, h), s),
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(orc.circular_conv_fft(np.roll(u, s), h), np.roll(orc.circular_conv_fft(u, h), s),
                               rtol=0, atol=1e-12)


# ---------------------------------------------------------------- input-dependent filters (HyenaND registers,
# FiLM-modulated SIREN, Gaussian window)

def test_register_summary_equal_scores_is_plain_mean():
    rng = np.random.default_rng(40)
    reg = rng.standard_normal((3, 5, 4))
    np.testing.assert_allclose(orc.register_summary(reg, np.zeros(4)), reg.mean(axis=1), rtol=0, atol=1e-15)


def test_register_summary_two_registers_logistic_weights():
    # two registers: the softmax weights are the logistic function of the score difference
    reg = np.array([[[1.0, 0.0, 2.0], [0.0, 1.0, -1.0]]])
    q = np.array([0.5, -0.25, 1.0])
    s1, s2 = 0.5 + 2.0, -0.25 - 1.0
    a1 = 1.0 / (1.0 + math.exp(-(s1 - s2)))
    want = a1 * reg[0, 0] + (1.0 - a1) * reg[0, 1]
    np.testing.assert_allclose(orc.register_summary(reg, q)[0], want, rtol=0, atol=1e-15)


def test_register_summary_permutation_invariant_and_dominant_register():
    rng = np.random.default_rng(41)
    reg = rng.standard_normal((2, 6, 8))
    q = rng.standard_normal(8)
    perm = rng.permutation(6)
    np.testing.assert_allclose(orc.register_summary(reg[:, perm], q), orc.register_summary(reg, q), rtol=0, atol=1e-14)
    # one register with a score far above the others takes all the weight
    big = reg.copy()
    big[:, 2] = 50.0 * q / np.linalg.norm(q)
    np.testing.assert_allclose(orc.register_summary(big, q), big[:, 2], rtol=0, atol=1e-12)


def _siren_closed_form_params(w):
    # H = 2 units, one coordinate, D = 3 channels, FiLM switched off (gamma = 1, beta = 0)
    return dict(A1=np.array([[1.0], [0.0]]), a1=np.array([0.0, 0.5]), omega0=np.array([w, 1.0]),
                A2=np.eye(2), a2=np.zeros(2), A3=np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]),
                a3=np.array([0.0, 0.0, 0.25]), G1=np.zeros((2, 2)), g1=np.ones(2), P1=np.zeros((2, 2)),
                p1=np.zeros(2), G2=np.zeros((2, 2)), g2=np.ones(2), P2=np.zeros((2, 2)), p2=np.zeros(2),
                q=np.zeros(2), sigma=np.array([0.3, 0.5, 1.0]))


def test_siren_without_modulation_closed_form():
    w = 7.0
    p = _siren_closed_form_params(w)
    c = np.linspace(-1, 1, 9)[:, None]
    f = orc.film_siren(c, np.array([0.3, -0.2]), p)
    u = np.sin(np.sin(w * c[:, 0]))
    k = math.sin(math.sin(0.5))
    np.testing.assert_allclose(f, np.stack([u, np.full(9, k), u + k + 0.25], axis=1), rtol=0, atol=1e-15)


def test_film_scales_preactivation_and_shifts_it():
    # gamma multiplies omega0 * (A1 c + a1) (bias included), beta is added after the scaling
    w = 3.0
    p = _siren_closed_form_params(w)
    p.update(omega0=np.array([w, 2.0]), G1=np.array([[1.0, 0.0], [0.0, 0.0]]), g1=np.array([0.0, 1.0]),
             P1=np.array([[0.0, 0.0], [0.0, 2.0]]), p1=np.array([0.0, 0.1]),
             g2=np.array([3.0, 1.0]), P2=np.array([[0.0, 1.0], [0.0, 0.0]]),
             A3=np.eye(2), a3=np.zeros(2), sigma=np.array([1.0, 1.0]))
    z = np.array([2.0, -0.5])                 # gamma1 = (2, 1), beta1 = (0, -0.9), beta2 = (-0.5, 0)
    c = np.linspace(0, 1, 5)[:, None]
    f = orc.film_siren(c, z, p)
    h1a = np.sin(2.0 * w * c[:, 0])
    h1b = math.sin(1.0 * 2.0 * 0.5 - 0.9)
    np.testing.assert_allclose(f[:, 0], np.sin(3.0 * h1a - 0.5), rtol=0, atol=1e-15)
    np.testing.assert_allclose(f[:, 1], np.full(5, math.sin(h1b)), rtol=0, atol=1e-15)


def test_gaussian_window_against_normal_density():
    import scipy.stats
    rng = np.random.default_rng(42)
    c = rng.uniform(-1, 1, size=(50, 3))
    sigma = np.array([0.2, 0.5, 1.5])
    w = orc.gaussian_window(c, sigma)
    r = np.linalg.norm(c, axis=1)
    for d, s in enumerate(sigma):
        np.testing.assert_allclose(w[d], scipy.stats.norm.pdf(r, scale=s) / scipy.stats.norm.pdf(0.0, scale=s),
                                   rtol=1e-13, atol=0)
        # separable over the axes; one sigma away from the origin the window is exp(-1/2)
        prod = np.prod(np.exp(-c ** 2 / (2 * s * s)), axis=1)
        np.testing.assert_allclose(w[d], prod, rtol=1e-13, atol=0)
    assert abs(orc.gaussian_window(np.array([[0.0, 0.6, 0.8]]), np.array([1.0]))[0, 0] - math.exp(-0.5)) < 1e-15


def test_input_dependent_filter_1d_closed_form_without_conditioning():
    # G = P = 0: every sample gets the same kernel, window(t/L) * closed-form SIREN(t/L)
    w, L = 5.0, 16
    p = _siren_closed_form_params(w)
    reg = np.random.default_rng(43).standard_normal((3, 4, 2))
    K = orc.input_dependent_filter_1d(p, reg, L)
    assert K.shape == (3, 3, L)
    c = np.arange(L) / L
    u, k = np.sin(np.sin(w * c)), math.sin(math.sin(0.5))
    f = np.stack([u, np.full(L, k), u + k + 0.25])
    want = f * np.exp(-c[None, :] ** 2 / (2 * p["sigma"][:, None] ** 2))
    for b in range(3):
        np.testing.assert_allclose(K[b], want, rtol=0, atol=1e-15)


def test_input_dependent_filter_follows_registers():
    rng = np.random.default_rng(44)
    H, E, D = 8, 6, 5
    p = dict(A1=rng.uniform(-1, 1, (H, 1)), a1=rng.uniform(-1, 1, H), omega0=np.full(H, 4.0),
             A2=rng.standard_normal((H, H)) * 0.3, a2=rng.standard_normal(H) * 0.1,
             A3=rng.standard_normal((D, H)) * 0.3, a3=rng.standard_normal(D) * 0.1,
             G1=rng.standard_normal((H, E)) * 0.2, g1=np.ones(H), P1=rng.standard_normal((H, E)) * 0.2,
             p1=np.zeros(H), G2=rng.standard_normal((H, E)) * 0.2, g2=np.ones(H),
             P2=rng.standard_normal((H, E)) * 0.2, p2=np.zeros(H), q=rng.standard_normal(E),
             sigma=rng.uniform(0.2, 0.6, D))
    reg = rng.standard_normal((3, 4, E))
    reg[2] = reg[0]                          # samples 0 and 2 carry the same registers
    K = orc.input_dependent_filter_1d(p, reg, 32)
    np.testing.assert_array_equal(K[0], K[2])
    assert np.max(np.abs(K[0] - K[1])) > 1e-3
    # each sample's kernel is the FiLM-SIREN at that sample's z, times the window
    z1 = orc.register_summary(reg, p["q"])[1]
    c = (np.arange(32) / 32.0)[:, None]
    np.testing.assert_allclose(K[1], orc.film_siren(c, z1, p).T * orc.gaussian_window(c, p["sigma"]), rtol=0,
                               atol=1e-15)


def test_input_dependent_filter_3d_axes_and_periodic_offsets():
    # a network that sees only the x coordinate gives taps that vary along x alone (x is the slowest
    # tap axis); the periodic filter equals the zero-padded one at every shared offset
    rng = np.random.default_rng(45)
    H, E, D, n = 4, 3, 2, 4
    A1 = np.zeros((H, 3))
    A1[:, 0] = rng.uniform(-1, 1, H)
    p = dict(A1=A1, a1=rng.uniform(-1, 1, H), omega0=np.full(H, 3.0), A2=rng.standard_normal((H, H)) * 0.3,
             a2=np.zeros(H), A3=rng.standard_normal((D, H)), a3=np.zeros(D), G1=rng.standard_normal((H, E)) * 0.1,
             g1=np.ones(H), P1=np.zeros((H, E)), p1=np.zeros(H), G2=np.zeros((H, E)), g2=np.ones(H),
             P2=np.zeros((H, E)), p2=np.zeros(H), q=np.zeros(E), sigma=np.array([1e6, 1e6]))
    reg = rng.standard_normal((2, 2, E))
    K = orc.input_dependent_filter_3d(p, reg, n)
    assert K.shape == (2, D, 7, 7, 7)
    np.testing.assert_allclose(K, np.broadcast_to(K[:, :, :, :1, :1], K.shape), rtol=0, atol=1e-9)
    assert np.max(np.abs(K[:, :, 0] - K[:, :, 6])) > 1e-3
    p["sigma"] = np.array([0.4, 0.7])
    p["A1"] = rng.uniform(-1, 1, (H, 3))
    Kl = orc.input_dependent_filter_3d(p, reg, n)
    Kc = orc.input_dependent_filter_3d(p, reg, n, circular=True)
    for r in orc.filter_offsets_3d_circular(n):
        np.testing.assert_allclose(Kc[:, :, r[0] % n, r[1] % n, r[2] % n], Kl[:, :, r[0] + n - 1, r[1] + n - 1,
                                   r[2] + n - 1], rtol=0, atol=0)


def test_per_sample_filters_in_the_operator_match_row_by_row_sums():
    # one filter per (b, d): the operator with [B, D, L] filters equals the definition applied row by row
    rng = np.random.default_rng(46)
    B, D, L = 2, 3, 12
    v = rng.standard_normal((B, D, L))
    xs = [rng.standard_normal((B, D, L)) for _ in range(2)]
    hs = [rng.standard_normal((B, D, L)) for _ in range(2)]
    y = orc.hyena_operator_rows(v, xs, hs)
    for b in range(B):
        for d in range(D):
            u = v[b, d]
            for h, x in zip(hs, xs):
                u = x[b, d] * np.array([sum(h[b, d, t - s] * u[s] for s in range(t + 1)) for t in range(L)])
            np.testing.assert_allclose(y[b, d], u, rtol=1e-12, atol=1e-12)
    # 3-D periodic with per-sample filters, against the brute-force definition per volume
    n = 3
    v3 = rng.standard_normal((B * D, n, n, n))
    x3 = [rng.standard_normal((B * D, n, n, n))]
    h3 = [rng.standard_normal((B * D, n, n, n))]
    y3 = orc.hyena_operator_3d(v3, x3, h3, circular=True)
    for j in range(B * D):
        np.testing.assert_allclose(y3[j], x3[0][j] * orc.circular_conv3d_direct(v3[j], h3[0][j]), rtol=1e-12,
                                   atol=1e-12)


# ---------------------------------------------------------------- input projection

def test_projection_against_triple_loop():
    rng = np.random.default_rng(50)
    B, L, Dm, D, order = 2, 3, 4, 2, 2
    x = rng.standard_normal((B, L, Dm))
    W = rng.standard_normal(((order + 1) * D, Dm))
    bias = rng.standard_normal((order + 1) * D)
    outs = orc.input_projection(x, W, bias, order)
    assert len(outs) == order + 1 and all(o.shape == (B, D, L) for o in outs)
    for j in range(order + 1):
        for b in range(B):
            for d in range(D):
                for t in range(L):
                    want = bias[j * D + d] + sum(W[j * D + d, k] * x[b, t, k] for k in range(Dm))
                    assert abs(outs[j][b, d, t] - want) < 1e-12


def test_projection_block_identity_splits_in_order():
    # W = [I; 2I; 3I]: v is x transposed, x_1 twice it, x_2 three times (v comes first)
    rng = np.random.default_rng(51)
    x = rng.standard_normal((2, 5, 3))
    W = np.concatenate([np.eye(3), 2 * np.eye(3), 3 * np.eye(3)])
    v, x1, x2 = orc.input_projection(x, W, None, 2)
    np.testing.assert_array_equal(v, np.swapaxes(x, 1, 2))
    np.testing.assert_array_equal(x1, 2 * np.swapaxes(x, 1, 2))
    np.testing.assert_array_equal(x2, 3 * np.swapaxes(x, 1, 2))


# ---------------------------------------------------------------- streaming decode

def test_decode_stream_matches_whole_sequence_operator():
    # token-by-token evaluation (all orders advancing together) against the order-by-order FFT form
    rng = np.random.default_rng(61)
    R, L = 5, 96
    v = rng.standard_normal((R, L))
    xs = [rng.standard_normal((R, L)) for _ in range(3)]
    hs = [rng.standard_normal((R, L)) * np.exp(-np.arange(L) / 20.0) for _ in range(3)]
    y = orc.hyena_decode_stream(v, xs, hs)
    np.testing.assert_allclose(y, orc.hyena_operator_rows(v, xs, hs), rtol=1e-10, atol=1e-12)


def test_decode_stream_unit_delay_filters_shift_each_order():
    # h_i = delta(t - 1): u_1[t] = x_1[t] v[t-1], y[t] = x_2[t] x_1[t-1] v[t-2] (zero history)
    rng = np.random.default_rng(62)
    L = 12
    v, x1, x2 = (rng.standard_normal(L) for _ in range(3))
    h = np.zeros(L)
    h[1] = 1.0
    y = orc.hyena_decode_stream(v[None], [x1[None], x2[None]], [h[None], h[None]])[0]
    want = np.zeros(L)
    want[2:] = x2[2:] * (x1[1:-1] * v[:-2])
    np.testing.assert_array_equal(y, want)


def test_decode_stream_delta_filters_are_pointwise():
    rng = np.random.default_rng(63)
    R, L = 3, 10
    v = rng.standard_normal((R, L))
    xs = [rng.standard_normal((R, L)) for _ in range(2)]
    h = np.zeros((R, L))
    h[:, 0] = [2.0, -1.0, 0.5]
    y = orc.hyena_decode_stream(v, xs, [h, h])
    np.testing.assert_allclose(y, v * xs[0] * xs[1] * (h[:, :1] ** 2), rtol=1e-14)


def test_decode_stream_prefix_is_stable():
    # outputs before t0 depend on inputs before t0 only (what lets a decoder emit them early)
    rng = np.random.default_rng(64)
    R, L, t0 = 2, 40, 23
    v = rng.standard_normal((R, L))
    xs = [rng.standard_normal((R, L)) for _ in range(2)]
    hs = [rng.standard_normal((R, L)) for _ in range(2)]
    y = orc.hyena_decode_stream(v, xs, hs)
    v2, xs2 = v.copy(), [x.copy() for x in xs]
    v2[:, t0:] = rng.standard_normal((R, L - t0))
    for x in xs2:
        x[:, t0:] = rng.standard_normal((R, L - t0))
    y2 = orc.hyena_decode_stream(v2, xs2, hs)
    np.testing.assert_array_equal(y2[:, :t0], y[:, :t0])
    assert np.abs(y2[:, t0:] - y[:, t0:]).max() > 1e-3
