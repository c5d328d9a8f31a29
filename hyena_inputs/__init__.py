"""Seeded synthetic workloads for the Hyena operator.

This module only draws random numbers and names shapes. It holds none of the
operator's arithmetic (no features, no filter network, no transform, no
convolution), so both the CPU oracle and the HIP path may take their inputs
from it without sharing any of the method.

Workloads (the five shapes the Hyena operator is exercised on):

  0  order 2, B=1, D=16,  L=1024,      fp32, v, x_i ~ N(0,1)
  1  order 2, B=4, D=768, L=8192,      bf16 storage, v, x_i ~ N(0,1)
  2  order 3, B=2, D=1024, L=65536,    bf16 storage, v, x_i ~ N(0,1)
  3  order 2, B=1, D=256, L=1048576,   fp32, DNA tokens through a 4x768 embedding
  4  order 2, B=1, D=128, grid 64^3,   fp32, non-causal 3-D (padded to 128^3)
  5  order 2, B=4, D=768, L=8192,      fp32, periodic 1-D (no padding)
  6  order 2, B=1, D=128, grid 64^3,   fp32, periodic 3-D (no padding)
  7  order 2, B=2, D=128, grid 64^3,   fp32, non-causal 3-D with input-dependent filters: 8 register
     tokens per sample, a FiLM-modulated SIREN (64 units) and a Gaussian window, one filter per (b, d)
  8  order 2, B=4, D=768, L=8192,      bf16 storage, from token-major inputs x [B, L, 768] through the
     input projection (W_proj [3 * 768, 768]) to v, x_1, x_2, then the operator
  9  order 2, B=4, D=768, L=8192,      fp32, streaming decode: the sequence fed one token at a time
     (prefix blocks of 256 tokens), v, x_i ~ N(0,1)

Random streams: ``numpy.random.default_rng([seed, stream])``.  Stream 0 draws
the activations (v, x_1 .. x_N in that order, or tokens then the embedding for
the DNA workload); stream 1 draws the filter parameters (per order: W1, W2,
alpha).  Biases are zero.  Xavier-uniform bounds use sqrt(6/(fan_in+fan_out)).
For input-dependent filters stream 1 draws, per order, the SIREN and FiLM parameters (see
``draw_film_params``) and stream 2 the register activations [B, R, D] ~ N(0,1).  For workloads that
start from the input projection, stream 3 draws the token-major inputs x [B, L, d_model] ~ N(0,1), then
W_proj [(N+1) D, d_model] (Xavier uniform); its bias is zero.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "draw_activations", "draw_filter_params",
    "bf16_bits_rne", "bf16_bits_to_f32", "seeded_rng", "draw_film_params", "draw_registers",
    "FILM_OMEGA0_BLOCKS", "draw_projection",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    order: int
    B: int
    D: int
    dims: tuple            # (L,) for 1-D, (nx, ny, nz) for 3-D
    dtype: str             # storage of v, x_i, y: "f32" or "bf16"
    mode: str              # "causal" (1-D), "linear" (3-D, zero-padded "same") or "circular" (periodic)
    alpha_lo: float
    alpha_hi: float
    features: int          # width of the positional-feature vector
    hidden: int            # width of the filter network's hidden layer
    activations: str = "normal"   # "normal" or "dna"
    filter: str = "exp"           # "exp": FFN x exponential window; "film": input-dependent (per sample)
    registers: int = 0            # register tokens per sample (input-dependent filters)
    sigma_lo: float = 0.2         # Gaussian window widths (input-dependent filters)
    sigma_hi: float = 0.8
    d_model: int = 0              # width of the token-major input of the projection (0: none)
    decode_block: int = 0         # streaming decode: tokens per prefix block (0: whole-sequence workload)

    @property
    def ndim(self) -> int:
        return len(self.dims)

    @property
    def points(self) -> int:
        p = 1
        for n in self.dims:
            p *= n
        return p

    @property
    def tokens_channels(self) -> int:
        return self.B * self.D * self.points

    @property
    def shape(self) -> tuple:
        return (self.B, self.D) + tuple(self.dims)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def support(self) -> int:
        """Number of filter taps per channel (L in 1-D; (2n-1)^3 offsets in 3-D, n^3 when periodic)."""
        if self.ndim == 1 or self.mode == "circular":
            return self.points
        p = 1
        for n in self.dims:
            p *= 2 * n - 1
        return p

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: List[Workload] = [
    Workload(0, "order2_B1_D16_L1024_f32", 2, 1, 16, (1024,), "f32", "causal", 0.3, 3.0, 64, 64),
    Workload(1, "order2_B4_D768_L8192_bf16", 2, 4, 768, (8192,), "bf16", "causal", 0.3, 3.0, 64, 64),
    Workload(2, "order3_B2_D1024_L65536_bf16", 3, 2, 1024, (65536,), "bf16", "causal", 0.1, 2.0, 64, 64),
    Workload(3, "hyenadna_order2_B1_D256_L1M_f32", 2, 1, 256, (1 << 20,), "f32", "causal", 0.01, 1.0, 64, 64,
             activations="dna"),
    Workload(4, "hyenand3d_order2_B1_D128_64cubed_f32", 2, 1, 128, (64, 64, 64), "f32", "linear", 0.3, 3.0, 96, 64),
    Workload(5, "periodic_order2_B4_D768_L8192_f32", 2, 4, 768, (8192,), "f32", "circular", 0.3, 3.0, 64, 64),
    Workload(6, "hyenand3d_periodic_order2_B1_D128_64cubed_f32", 2, 1, 128, (64, 64, 64), "f32", "circular",
             0.3, 3.0, 96, 64),
    Workload(7, "hyenand3d_film_order2_B2_D128_64cubed_f32", 2, 2, 128, (64, 64, 64), "f32", "linear",
             0.0, 0.0, 3, 64, filter="film", registers=8),
    Workload(8, "proj_order2_B4_D768_L8192_bf16", 2, 4, 768, (8192,), "bf16", "causal", 0.3, 3.0, 64, 64,
             d_model=768),
    Workload(9, "decode_order2_B4_D768_L8192_f32", 2, 4, 768, (8192,), "f32", "causal", 0.3, 3.0, 64, 64,
             decode_block=256),
]


def workload(i: int) -> Workload:
    return WORKLOADS[i]


def seeded_rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the uint16 bit patterns.

    Data preparation for bf16 storage: the upper 16 bits of the fp32 pattern after
    adding 0x7FFF plus the lowest kept bit.  NaNs are kept quiet NaNs.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = r.copy()
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def draw_activations(w: Workload, seed: Optional[int] = None):
    """Return (v, [x_1..x_N]) as float32 arrays of shape [B, D, *dims].

    For bf16 workloads the returned float32 values are already rounded to bf16
    (every value is exactly representable in bf16), so that both sides see the
    same stored numbers.  Use :func:`bf16_bits_rne` to get the bit patterns.
    """
    seed = w.index if seed is None else seed
    rng = seeded_rng(seed, 0)
    shape = w.shape
    if w.activations == "dna":
        # tokens uniform over {A,C,G,T}, embedding E ~ N(0,1) of shape [4, (N+1)*D];
        # column block j of E feeds stream j (v, x_1, ..., x_N), channel-major after the gather.
        L = w.points
        tok = rng.integers(0, 4, size=(w.B, L), dtype=np.int64)
        E = rng.standard_normal((4, (w.order + 1) * w.D), dtype=np.float32)
        streams = []
        for j in range(w.order + 1):
            Ej = np.ascontiguousarray(E[:, j * w.D:(j + 1) * w.D].T)      # [D, 4]
            a = np.empty(shape, dtype=np.float32)
            for b in range(w.B):
                a[b] = Ej[:, tok[b]]
            streams.append(a)
    else:
        streams = [_normal(rng, shape) for _ in range(w.order + 1)]
    if w.dtype == "bf16":
        streams = [bf16_bits_to_f32(bf16_bits_rne(a)) for a in streams]
    return streams[0], streams[1:]


def draw_filter_params(w: Workload, seed: Optional[int] = None) -> List[dict]:
    """Per-order filter parameters as float32 arrays.

    W1 [H, F], b1 [H] (zeros), W2 [D, H], b2 [D] (zeros), alpha [D] ~ U[alpha_lo, alpha_hi).
    """
    seed = w.index if seed is None else seed
    rng = seeded_rng(seed, 1)
    F, H, D = w.features, w.hidden, w.D
    out = []
    for _ in range(w.order):
        a1 = np.float32(np.sqrt(6.0 / (F + H)))
        W1 = ((rng.random((H, F), dtype=np.float32) * 2 - 1) * a1).astype(np.float32)
        a2 = np.float32(np.sqrt(6.0 / (H + D)))
        W2 = ((rng.random((D, H), dtype=np.float32) * 2 - 1) * a2).astype(np.float32)
        alpha = rng.uniform(w.alpha_lo, w.alpha_hi, size=D).astype(np.float32)
        out.append(dict(W1=W1, b1=np.zeros(H, np.float32), W2=W2, b2=np.zeros(D, np.float32), alpha=alpha))
    return out


FILM_OMEGA0_BLOCKS = (1.0, 3.0, 10.0, 30.0)


def draw_film_params(w: Workload, seed: Optional[int] = None) -> List[dict]:
    """Per-order input-dependent filter parameters as float32 arrays (H = w.hidden units, n = w.ndim
    coordinates, E = D register width):

    q [E] ~ N(0, 1/E); A1 [H, n], a1 [H] ~ U(-1/n, 1/n); omega0 [H]: the units in equal blocks at the
    scales FILM_OMEGA0_BLOCKS; A2 [H, H] ~ U(+-sqrt(6/H)), a2 [H] ~ U(+-1/sqrt(H)); A3 [D, H] Xavier
    uniform, a3 [D] zeros; FiLM maps G1, P1, G2, P2 [H, E] ~ N(0, 0.25/E), g1 = g2 = 1, p1 = p2 = 0;
    sigma [D] ~ U[sigma_lo, sigma_hi).
    """
    seed = w.index if seed is None else seed
    rng = seeded_rng(seed, 1)
    H, D, n, E = w.hidden, w.D, w.ndim, w.D
    f32 = lambda a: np.asarray(a, dtype=np.float32)
    uni = lambda shape, b: f32((rng.random(shape) * 2 - 1) * b)
    nb = len(FILM_OMEGA0_BLOCKS)
    omega0 = f32(np.repeat(FILM_OMEGA0_BLOCKS, -(-H // nb))[:H])
    out = []
    for _ in range(w.order):
        p = dict(q=f32(rng.standard_normal(E) / np.sqrt(E)), A1=uni((H, n), 1.0 / n), a1=uni(H, 1.0 / n),
                 omega0=omega0.copy(), A2=uni((H, H), np.sqrt(6.0 / H)), a2=uni(H, 1.0 / np.sqrt(H)),
                 A3=uni((D, H), np.sqrt(6.0 / (H + D))), a3=np.zeros(D, np.float32))
        for l in (1, 2):
            p[f"G{l}"] = f32(rng.standard_normal((H, E)) * (0.5 / np.sqrt(E)))
            p[f"g{l}"] = np.ones(H, np.float32)
            p[f"P{l}"] = f32(rng.standard_normal((H, E)) * (0.5 / np.sqrt(E)))
            p[f"p{l}"] = np.zeros(H, np.float32)
        p["sigma"] = f32(rng.uniform(w.sigma_lo, w.sigma_hi, size=D))
        out.append(p)
    return out


def draw_registers(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Register activations [B, R, D] ~ N(0,1) as float32 (random stream 2)."""
    seed = w.index if seed is None else seed
    return seeded_rng(seed, 2).standard_normal((w.B, w.registers, w.D), dtype=np.float32)


def draw_projection(w: Workload, seed: Optional[int] = None):
    """(x [B, L, d_model], W_proj [(N+1) D, d_model], bias [(N+1) D]) as float32 (stream 3); x and W are
    rounded to bf16 for bf16 workloads, the bias is zero."""
    seed = w.index if seed is None else seed
    rng = seeded_rng(seed, 3)
    M, K = (w.order + 1) * w.D, w.d_model
    x = rng.standard_normal((w.B, w.points, K), dtype=np.float32)
    W = ((rng.random((M, K), dtype=np.float32) * 2 - 1) * np.float32(np.sqrt(6.0 / (M + K)))).astype(np.float32)
    if w.dtype == "bf16":
        x = bf16_bits_to_f32(bf16_bits_rne(x))
        W = bf16_bits_to_f32(bf16_bits_rne(W))
    return x, W, np.zeros(M, np.float32)


def sample_rows(w: Workload, count: int, seed: int = 1234) -> np.ndarray:
    """Distinct (b, d) row indices, as a [count, 2] int array, always including the first and last row."""
    total = w.B * w.D
    count = min(count, total)
    rng = seeded_rng(seed, 7)
    pick = set([0, total - 1])
    while len(pick) < count:
        pick.add(int(rng.integers(0, total)))
    flat = np.array(sorted(pick), dtype=np.int64)
    return np.stack([flat // w.D, flat % w.D], axis=1)
