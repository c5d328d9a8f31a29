// Workgroup FFT engines on LDS for the Hyena long convolution (gfx950, wave64).
//
// RowEngine<NB, Radices<R0..RP-1>>: NB independent S-point complex DFTs (S = R0*...*RP-1) held
//   contiguously in LDS (sub-FFT b at [b*S, (b+1)*S)).  Forward passes are in-place decimation in
//   frequency (radix R_j DFT over stride Q_j, then output twiddles W_{S_j}^{n k}); the spectrum stays
//   in digit-reversed positions.  The first pass takes its input from registers and the last pass
//   leaves two radix-RP blocks per thread in registers, so the spectral product happens between the
//   last forward and the first inverse pass without touching LDS.  Inverse passes mirror the forward
//   ones (input twiddles conj(W), inverse DFT) and end in registers.
//
//   Frequency bookkeeping: pass j yields digit d_j; bin k = d_0 + R0 d_1 + R0 R1 d_2 + ...; position
//   p = sum_j d_j S/(R0..Rj).  A last-pass block beta (position beta*RP) holds bins kappa + (S/RP) m,
//   where kappa collects d_0..d_{P-2}.
//
// ColEngine<NL, LP, T, Radices>: NL lines of an N-point DFT laid across LDS with the line index
//   fastest (element (line l, position p) at p*LP + l): the transform runs down the columns of a
//   tile, every pass LDS -> LDS, consecutive lanes on consecutive lines.
#pragma once

#include "fft_core.h"

namespace hyena {

template <int... Rs>
struct Radices {
  static constexpr int P = sizeof...(Rs);
  static constexpr int R[P] = {Rs...};
  static constexpr int S = (Rs * ...);
  static constexpr int RP = R[P - 1];
  // sub-block size seen by pass j
  static constexpr int sub(int j) {
    int s = S;
    for (int i = 0; i < j; ++i) s /= R[i];
    return s;
  }
  // bin offset kappa of last-pass block beta (inverse digit reversal of d_0..d_{P-2})
  __device__ __forceinline__ static int kappa_of_block(int beta) {
    int kap = 0, mul = 1;
    // beta = sum_{j<P-1} d_j * sub(j+1)/RP ; peel the most significant position digit (d_0) first
    static_for<P - 1>([&](auto jj) {
      constexpr int j = jj.value;
      constexpr int c = sub(j + 1) / RP;          // coefficient of d_j in beta
      const int dj = beta / c;
      beta -= dj * c;
      kap += dj * mul;
      mul *= R[j];
    });
    return kap;
  }
  // position of bin k's digit prefix: block index of kappa (digit reversal)
  __device__ __forceinline__ static int block_of_kappa(int kap) {
    int beta = 0;
    static_for<P - 1>([&](auto jj) {
      constexpr int j = jj.value;
      const int dj = kap % R[j];
      kap /= R[j];
      beta += dj * (sub(j + 1) / RP);
    });
    return beta;
  }
  // in-place position of bin k for a full transform (used for the column engine's outputs)
  __host__ __device__ static constexpr int position_of_bin(int k) {
    int p = 0;
    for (int j = 0; j < P; ++j) {
      const int dj = k % R[j];
      k /= R[j];
      p += dj * (sub(j + 1));
    }
    return p;
  }
  __host__ __device__ static constexpr int bin_of_position(int p) {
    int k = 0, mul = 1;
    for (int j = 0; j < P; ++j) {
      const int c = sub(j + 1);
      const int dj = p / c;
      p -= dj * c;
      k += dj * mul;
      mul *= R[j];
    }
    return k;
  }
};

template <int NB, class RL>
struct RowEngine {
  static constexpr int P = RL::P, S = RL::S, RP = RL::RP;
  static constexpr int E = 2 * RP;
  static constexpr int T = NB * S / E;
  static constexpr int NBLK = S / RP;                 // last-pass blocks per sub-FFT
  static constexpr int LDS_ELEMS = lds_padded_size(NB * S);
  static_assert(P >= 2, "at least two passes");

  template <int J>
  __device__ __forceinline__ static int base_of(int b, int& n) {
    constexpr int R = RL::R[J], SJ = RL::sub(J), Q = SJ / R, PER = S / R;
    const int bat = b / PER, rem = b % PER;
    n = rem % Q;
    return bat * S + (rem / Q) * SJ + n;
  }

  // Input of pass 0 for butterfly i of thread t: sub-FFT `bat`, positions n + m*S/R0, m < R0.
  __device__ __forceinline__ static void first_input(int t, int i, int& bat, int& n) {
    constexpr int PER = S / RL::R[0];
    const int b = t + T * i;
    bat = b / PER;
    n = b % PER;
  }

  // Output twiddles of pass J for butterfly index n: p[k] = W_{S_J}^{n k}.  When every butterfly
  // of a thread has the same n (Q divides T) the powers are formed once per pass.
  template <int J>
  __device__ __forceinline__ static void pass_twiddles(const Twiddles& tw, int n, float2 (&p)[RL::R[J]]) {
    constexpr int SJ = RL::sub(J);
    twiddle_powers<RL::R[J]>(twiddle<ilog2(SJ)>(tw, uint32_t(n)), p);
  }

  // forward pass J < P-1; J == 0 reads registers (ZERO_UPPER: inputs m >= R0/2 are zero)
  template <int J, bool ZERO_UPPER = false>
  __device__ __forceinline__ static void fwd(float2 (&x)[E], float2* lds, const Twiddles& tw, int t) {
    constexpr int R = RL::R[J], SJ = RL::sub(J), Q = SJ / R, NBT = E / R;
    constexpr bool SHARED = (T % Q == 0);
    static_assert(E % R == 0, "radix must divide the per-thread element count");
    if constexpr (J > 0) {
      static_for<NBT>([&](auto ii) {
        int n;
        const int base = base_of<J>(t + T * ii.value, n);
        static_for<R>([&](auto m) { x[ii.value * R + m.value] = lds[lds_pad(base + m.value * Q)]; });
      });
    }
    float2 wp[R];
    if constexpr (SHARED) {
      int n;
      base_of<J>(t, n);
      pass_twiddles<J>(tw, n, wp);
    }
    static_for<NBT>([&](auto ii) {
      constexpr int i = ii.value;
      int n;
      const int base = base_of<J>(t + T * i, n);
      if constexpr (!SHARED) pass_twiddles<J>(tw, n, wp);
      dft_sub<R, false, ZERO_UPPER && J == 0, false, i * R, 1>(x);
      static_for<R>([&](auto kk) {
        constexpr int k = kk.value;
        float2 v = x[i * R + k];
        if constexpr (k != 0) v = cmul(v, wp[k]);
        lds[lds_pad(base + k * Q)] = v;
      });
    });
  }
  // last forward pass: blocks bA, bB (indices over all NB*NBLK blocks) into x[0..RP), x[RP..2RP)
  __device__ __forceinline__ static void fwd_last(float2 (&x)[E], const float2* lds, int bA, int bB) {
    static_for<RP>([&](auto m) {
      x[m.value] = lds[lds_pad(bA * RP + m.value)];
      x[RP + m.value] = lds[lds_pad(bB * RP + m.value)];
    });
    dft_sub<RP, false, false, false, 0, 1>(x);
    dft_sub<RP, false, false, false, RP, 1>(x);
  }
  __device__ __forceinline__ static void inv_last(float2 (&x)[E], float2* lds, int bA, int bB) {
    dft_sub<RP, true, false, false, 0, 1>(x);
    dft_sub<RP, true, false, false, RP, 1>(x);
    static_for<RP>([&](auto m) {
      lds[lds_pad(bA * RP + m.value)] = x[m.value];
      lds[lds_pad(bB * RP + m.value)] = x[RP + m.value];
    });
  }
  // inverse pass J < P-1 (input twiddles, inverse DFT).  J == 0 leaves the result in registers
  // (HALF_OUT: only outputs m < R0/2, i.e. positions < S/2).
  template <int J, bool HALF_OUT = false>
  __device__ __forceinline__ static void inv(float2 (&x)[E], float2* lds, const Twiddles& tw, int t) {
    constexpr int R = RL::R[J], SJ = RL::sub(J), Q = SJ / R, NBT = E / R;
    constexpr bool SHARED = (T % Q == 0);
    float2 wp[R];
    if constexpr (SHARED) {
      int n;
      base_of<J>(t, n);
      pass_twiddles<J>(tw, n, wp);
    }
    static_for<NBT>([&](auto ii) {
      constexpr int i = ii.value;
      int n;
      const int base = base_of<J>(t + T * i, n);
      if constexpr (!SHARED) pass_twiddles<J>(tw, n, wp);
      static_for<R>([&](auto kk) {
        constexpr int k = kk.value;
        float2 v = lds[lds_pad(base + k * Q)];
        if constexpr (k != 0) v = cmulc(v, wp[k]);
        x[i * R + k] = v;
      });
    });
    static_for<NBT>([&](auto ii) {
      constexpr int i = ii.value;
      dft_sub<R, true, false, HALF_OUT && J == 0, i * R, 1>(x);
      if constexpr (J > 0) {
        int n;
        const int base = base_of<J>(t + T * i, n);
        static_for<R>([&](auto m) { lds[lds_pad(base + m.value * Q)] = x[i * R + m.value]; });
      }
    });
  }

  // forward passes 0..P-2 with barriers; caller then calls fwd_last
  template <bool ZERO_UPPER>
  __device__ __forceinline__ static void forward_to_last(float2 (&x)[E], float2* lds, const Twiddles& tw, int t) {
    static_for<P - 1>([&](auto jj) {
      fwd<jj.value, ZERO_UPPER>(x, lds, tw, t);
      __syncthreads();
    });
  }
  // after inv_last: inverse passes P-2..0 with barriers before each
  template <bool HALF_OUT>
  __device__ __forceinline__ static void inverse_from_last(float2 (&x)[E], float2* lds, const Twiddles& tw, int t) {
    static_for<P - 1>([&](auto jj) {
      constexpr int J = P - 2 - jj.value;
      __syncthreads();
      inv<J, HALF_OUT>(x, lds, tw, t);
    });
  }
};

// Thread -> block pair assignment of the last pass for one whole sub-FFT whose bins pair as
// k <-> S-k ("negation"), with T_neg = S/(2 RP) threads.  Blocks are consecutive across
// consecutive threads (bank-conflict-free reads).  Thread T_neg-1 holds the two self-mirrored
// blocks (kappa = 0 and kappa = S/(2 RP)).
template <class RL>
struct NegPairs {
  static constexpr int P = RL::P, S = RL::S, RP = RL::RP;
  static constexpr int TN = S / (2 * RP);
  struct Pair { int betaA, betaB, kapA, kapB; bool special; };
  __device__ __forceinline__ static Pair of(int t) {
    constexpr int RL2 = RL::R[P - 2];                         // digit with unit stride in beta
    constexpr int KLOW = (S / RP) / RL2;                      // number of kappa_low values
    Pair p;
    int klA, dA, klB, dB;
    p.special = false;
    constexpr int g0 = (KLOW / 2 - 1) * RL2;
    if (KLOW >= 2 && t < g0) {
      klA = 1 + t / RL2; dA = t % RL2; klB = KLOW - klA; dB = RL2 - 1 - dA;
    } else if (KLOW >= 2 && t < g0 + RL2 / 2) {
      const int j = t - g0;
      klA = klB = KLOW / 2; dA = j; dB = RL2 - 1 - j;
    } else if (t < TN - 1) {
      const int j = t - (KLOW >= 2 ? g0 + RL2 / 2 : 0);
      klA = klB = 0; dA = j + 1; dB = RL2 - 1 - j;
    } else {
      klA = klB = 0; dA = 0; dB = RL2 / 2; p.special = true;
    }
    p.kapA = klA + KLOW * dA;
    p.kapB = klB + KLOW * dB;
    p.betaA = RL::block_of_kappa(p.kapA);
    p.betaB = RL::block_of_kappa(p.kapB);
    return p;
  }
};

// Column engine: NL lines of N = RL::S points; element (line l, position p) at
// lds[addr(p * PS + l * LS)], addr = lds_pad when PAD.  Butterflies are enumerated line-fastest, so
// consecutive lanes touch consecutive lines (conflict-free when LS == 1, or when LS is odd).
// NL need not divide the butterfly count evenly among threads (the tail is guarded).
// SWZ16 (16 contiguous lines, LS == 1, no padding): bit 4 of the element index is flipped with bit 7,
// i.e. position rows 8..15 of every 16 store their two half-rows of 8 complex swapped.  A 64-bit access
// serves 32 lanes at once, which here are 16 lines of two rows: rows p and p + 1 (p even) or p and
// p + 8 (the radix-8 passes with unit stride).  Padded rows put one bank pair of the second row on the
// first's; with the swap both pairs of rows fill the 64 banks exactly once.
template <int NL, int PS, int LS, int T, class RL, bool PAD = true, bool SWZ16 = false>
struct ColEngine {
  static constexpr int P = RL::P, N = RL::S;
  static_assert(!SWZ16 || (NL == 16 && PS == 16 && LS == 1 && !PAD), "swizzle layout");
  __device__ __forceinline__ static int addr(int p, int l) {
    const int a = p * PS + l * LS;
    if constexpr (SWZ16) return a ^ ((a >> 3) & 16);
    return PAD ? lds_pad(a) : a;
  }

  template <int J, bool INV, bool ZERO_UPPER, bool HALF_OUT>
  __device__ __forceinline__ static void pass(float2* lds, const Twiddles& tw, int t) {
    constexpr int R = RL::R[J], SJ = RL::sub(J), Q = SJ / R;
    constexpr int NBF = NL * N / R;                      // butterflies in this pass
    constexpr int NBT = (NBF + T - 1) / T;
    constexpr bool EVEN = (NBF % T == 0);
    static_for<NBT>([&](auto ii) {
      const int b = t + T * ii.value;
      if (!EVEN && b >= NBF) return;
      const int l = b % NL, rem = b / NL;
      const int n = rem % Q;
      const int p0 = (rem / Q) * SJ + n;
      float2 wp[R];
      twiddle_powers<R>(twiddle<ilog2(SJ)>(tw, uint32_t(n)), wp);
      float2 v[R];
      static_for<R>([&](auto mm) {
        constexpr int m = mm.value;
        if constexpr (!(ZERO_UPPER && !INV && J == 0 && m >= R / 2)) {
          float2 a = lds[addr(p0 + m * Q, l)];
          if constexpr (INV && m != 0) a = cmulc(a, wp[m]);
          v[m] = a;
        }
      });
      constexpr bool zu = ZERO_UPPER && !INV && J == 0;
      constexpr bool ho = HALF_OUT && INV && J == 0;
      dft<R, INV, zu, ho>(v);
      static_for<R>([&](auto kk) {
        constexpr int k = kk.value;
        if constexpr (!(ho && k >= R / 2)) {
          float2 a = v[k];
          if constexpr (!INV && k != 0) a = cmul(a, wp[k]);
          lds[addr(p0 + k * Q, l)] = a;
        }
      });
    });
  }
  // forward DIF, natural positions in -> digit-reversed positions out
  template <bool ZERO_UPPER>
  __device__ __forceinline__ static void forward(float2* lds, const Twiddles& tw, int t) {
    static_for<P>([&](auto jj) {
      pass<jj.value, false, ZERO_UPPER, false>(lds, tw, t);
      __syncthreads();
    });
  }
  // inverse (mirror), digit-reversed in -> natural out; HALF_OUT keeps positions < N/2 only
  template <bool HALF_OUT>
  __device__ __forceinline__ static void inverse(float2* lds, const Twiddles& tw, int t) {
    static_for<P>([&](auto jj) {
      pass<P - 1 - jj.value, true, false, HALF_OUT>(lds, tw, t);
      __syncthreads();
    });
  }
};

// Real-input split, product with the filter spectrum and re-pack for the inverse, for one pair of
// mirrored bins (k, M-k) of the M-point transform of z[n] = u[2n] + i u[2n+1].
//   A = Z[k], B = Z[M-k] (B == A for a self-mirrored bin), w = W_{2M}^k, hk = Hs[k], hp = Hs[M-k],
//   Hs = H / (4M) with H the 2M-point DFT of the zero-padded filter.
//   X[k] = E + w O, X[M-k] = conj(E - w O), E = (A + conj B)/2, O = (A - conj B)/(2i);  Y = X H;
//   Z'[k] = Ye + i Yo, Ye = (Y[k] + conj Y[M-k])/2, Yo = (Y[k] - conj Y[M-k]) conj(w)/2.
// On return A = Z''[k], B = Z''[M-k] with Z'' = Z'/M: the unnormalised inverse M-point DFT of Z''
// packs the 2M-point real result as (y[2n], y[2n+1]).
__device__ __forceinline__ void spectral_pair(float2& A, float2& B, float2 w, float2 hk, float2 hp) {
  const float2 Bc = cconj(B);
  const float2 E2 = cadd(A, Bc);
  const float2 Dd = csub(A, Bc);
  const float2 O2 = make_float2(Dd.y, -Dd.x);          // -i * Dd
  const float2 wO = cmul(w, O2);
  const float2 Xk = cadd(E2, wO);                      // 2 X[k]
  const float2 Xp = cconj(csub(E2, wO));               // 2 X[M-k]
  const float2 Sk = cmul(Xk, hk);
  const float2 Spc = cconj(cmul(Xp, hp));
  const float2 Ye = cadd(Sk, Spc);
  const float2 Yo = cmulc(csub(Sk, Spc), w);
  A = make_float2(Ye.x - Yo.y, Ye.y + Yo.x);
  B = make_float2(Ye.x + Yo.y, Yo.x - Ye.y);
}

// Spectrum element: fp32 complex, or one word of two bf16 (real part low, imaginary part high).
__device__ __forceinline__ float2 hload(const float2* p) { return *p; }
__device__ __forceinline__ float2 hload(const uint32_t* p) {
  const uint32_t w = *p;
  return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

// Real-input split only: returns 2 X[k] and 2 X[M-k] (used to build filter spectra).
__device__ __forceinline__ void split_pair(float2 A, float2 B, float2 w, float2& Xk, float2& Xp) {
  const float2 Bc = cconj(B);
  const float2 E2 = cadd(A, Bc);
  const float2 Dd = csub(A, Bc);
  const float2 O2 = make_float2(Dd.y, -Dd.x);
  const float2 wO = cmul(w, O2);
  Xk = cadd(E2, wO);
  Xp = cconj(csub(E2, wO));
}

// Spectral step on the two last-pass blocks of one thread, pairing x[m] with x[2RP-1-m]
// ("complement" pairing: block B holds the mirrors of block A in reverse order).
// wA = W_{2M}^{bin of x[0]}; bins of x[m] advance by `step` = M*? via the constant W_{2RP}^m.
// MODE 0: multiply by the spectrum (h from slots), MODE 1: write the split spectrum to `hs_out`.
template <int RP, int MODE, class HT = float2>
__device__ __forceinline__ void spectral_complement(float2 (&x)[2 * RP], float2 wA, const HT* hs, int stride,
                                                    float2* hs_out, float sc) {
  static_for<RP>([&](auto mm) {
    constexpr int m = mm.value, mp = 2 * RP - 1 - m;
    const float2 w = mul_w<m, 2 * RP, false>(wA);
    if constexpr (MODE == 0) {
      spectral_pair(x[m], x[mp], w, hload(hs + m * stride), hload(hs + mp * stride));
    } else {
      float2 Xk, Xp;
      split_pair(x[m], x[mp], w, Xk, Xp);
      hs_out[m * stride] = cscale(Xk, sc);
      hs_out[mp * stride] = cscale(Xp, sc);
    }
  });
}

// Spectral step for the thread that holds the two self-mirrored blocks of a whole transform:
// block A (x[0..RP)) has bins (S/RP) m, mirrored as m <-> RP-m (m = 0: bins 0 and M; m = RP/2: M/2);
// block B (x[RP..2RP)) has bins kB + (S/RP) m mirrored as m <-> RP-1-m.  Slot 0 carries the real
// pair (Hs[0], Hs[M]) as (x, y).  w0 = W_{2M}^{0} = 1, wB = W_{2M}^{kB}.
template <int RP, int MODE, class HT = float2>
__device__ __forceinline__ void spectral_selfmirror(float2 (&x)[2 * RP], float2 wB, const HT* hs, int stride,
                                                    float2* hs_out, float sc) {
  static_for<RP / 2 + 1>([&](auto mm) {
    constexpr int m = mm.value, mp = (RP - m) % RP;
    const float2 w = mul_w<m, 2 * RP, false>(make_float2(1.f, 0.f));
    if constexpr (MODE == 0) {
      if constexpr (m == 0) {
        const float2 s = hload(hs);
        float2 bb = x[0];
        spectral_pair(x[0], bb, w, make_float2(s.x, 0.f), make_float2(s.y, 0.f));
      } else if constexpr (m == RP / 2) {
        float2 bb = x[m];
        const float2 h = hload(hs + m * stride);
        spectral_pair(x[m], bb, w, h, h);
      } else {
        spectral_pair(x[m], x[mp], w, hload(hs + m * stride), hload(hs + mp * stride));
      }
    } else {
      float2 Xk, Xp;
      split_pair(x[m], x[mp], w, Xk, Xp);
      if constexpr (m == 0) {
        hs_out[0] = make_float2(Xk.x * sc, Xp.x * sc);
      } else {
        hs_out[m * stride] = cscale(Xk, sc);
        if constexpr (m != RP / 2) hs_out[mp * stride] = cscale(Xp, sc);
      }
    }
  });
  static_for<RP / 2>([&](auto mm) {
    constexpr int m = RP + mm.value, mp = 2 * RP - 1 - mm.value;
    const float2 w = mul_w<mm.value, 2 * RP, false>(wB);
    if constexpr (MODE == 0) {
      spectral_pair(x[m], x[mp], w, hload(hs + m * stride), hload(hs + mp * stride));
    } else {
      float2 Xk, Xp;
      split_pair(x[m], x[mp], w, Xk, Xp);
      hs_out[m * stride] = cscale(Xk, sc);
      hs_out[mp * stride] = cscale(Xp, sc);
    }
  });
}

}  // namespace hyena
