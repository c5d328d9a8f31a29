// One-workgroup FFT engine for a causal long convolution whose whole transform fits in LDS.
//
// A row u[0..L) (real) is zero-padded to 2L and packed two samples per complex value,
// z[n] = u[2n] + i u[2n+1], n < M = L (z[n] = 0 for n >= M/2).  The M-point complex DFT of z
// runs as three in-place decimation-in-frequency passes (radices R1, R2, R3) with LDS exchanges in
// between; the spectrum is left in digit-reversed order (it is never reordered).  The real-input
// split (bins k and M-k), the product with the filter spectrum and the re-pack for the inverse all
// happen in registers between the last forward pass and the first inverse pass: the last pass
// gives every thread two radix-R3 blocks whose bins are each other's mirror images.  The inverse
// passes mirror the forward ones (input twiddles, inverse DFTs) and only compute the first half of
// the output (the causal part that is kept).
//
// The product of the zero-padded spectra is the linear (non-wrapping) convolution (HyenaND summary,
// boundary handling); keeping outputs [0, L) makes it causal (EulerStack "4. Hyena 상세", how it
// works 2: FFT, elementwise product, inverse FFT).
#pragma once

#include "fft_core.h"

namespace hyena {

template <int LOG2M> struct Plan1;
template <> struct Plan1<10> { static constexpr int R1 = 16, R2 = 8, R3 = 8; };
template <> struct Plan1<11> { static constexpr int R1 = 16, R2 = 16, R3 = 8; };
template <> struct Plan1<12> { static constexpr int R1 = 16, R2 = 16, R3 = 16; };
template <> struct Plan1<13> { static constexpr int R1 = 32, R2 = 16, R3 = 16; };
template <> struct Plan1<14> { static constexpr int R1 = 32, R2 = 32, R3 = 16; };

// Scaled filter spectrum layout ("engine order"): Hs[slot * T + t] for slot < 2*R3, where slot r of
// thread t holds Hs at the bin of that thread's register r in the fused pass (r < R3: block A
// element r, r >= R3: block B element r - R3).  Hs = H / (4M) with H the 2M-point DFT of the
// zero-padded filter.  Thread T-1, slot 0 holds (Hs[0], Hs[M]) as (x, y): both are real.
template <int LOG2M>
struct Engine1 {
  static constexpr int M = 1 << LOG2M;
  static constexpr int R1 = Plan1<LOG2M>::R1, R2 = Plan1<LOG2M>::R2, R3 = Plan1<LOG2M>::R3;
  static constexpr int E = 2 * R3;
  static constexpr int T = M / E;
  static constexpr int Q1 = M / R1;          // stride of pass 1
  static constexpr int S2 = M / R1;          // sub-block size of pass 2
  static constexpr int Q2 = S2 / R2;         // stride of pass 2 (== R3)
  static constexpr int NB1 = E / R1;         // pass-1 butterflies per thread
  static constexpr int NB2 = E / R2;         // pass-2 butterflies per thread
  static constexpr int LDS_ELEMS = lds_padded_size(M);
  static_assert(R1 * R2 * R3 == M, "plan");
  static_assert(Q2 == R3, "three passes");
  static_assert(E % R1 == 0 && E % R2 == 0, "plan");

  // ---- fused-pass block assignment: thread t owns blocks A and B of the last pass
  struct Pair {
    int betaA, betaB;     // block index (LDS position / R3)
    int kapA, kapB;       // frequency offset: bin of element m is kap + (M/R3) m
    bool special;         // thread T-1: both blocks are their own mirror
  };
  __device__ __forceinline__ static Pair pair_of(int t) {
    Pair p;
    int k1A, k2A, k1B, k2B;
    constexpr int g0 = (R1 / 2 - 1) * R2;
    p.special = false;
    if (t < g0) {
      k1A = 1 + t / R2; k2A = t % R2; k1B = R1 - k1A; k2B = R2 - 1 - k2A;
    } else if (t < g0 + R2 / 2) {
      const int j = t - g0;
      k1A = k1B = R1 / 2; k2A = j; k2B = R2 - 1 - j;
    } else if (t < T - 1) {
      const int j = t - g0 - R2 / 2;
      k1A = k1B = 0; k2A = j + 1; k2B = R2 - 1 - j;
    } else {
      k1A = k1B = 0; k2A = 0; k2B = R2 / 2; p.special = true;
    }
    p.betaA = k1A * R2 + k2A; p.betaB = k1B * R2 + k2B;
    p.kapA = k1A + R1 * k2A;  p.kapB = k1B + R1 * k2B;
    return p;
  }
  // bin held by slot r of thread t (slot 0 of thread T-1 holds bins 0 and M)
  __device__ __forceinline__ static int slot_bin(int t, int r) {
    Pair p = pair_of(t);
    return r < R3 ? p.kapA + (M / R3) * r : p.kapB + (M / R3) * (r - R3);
  }

  // ---- forward pass 1: x holds, for butterfly i (b = t + T i), z[b + m Q1] at x[i R1 + m] (m < R1/2)
  __device__ __forceinline__ static void fwd1(float2 (&x)[E], float2* lds, const Twiddles& tw, int t) {
    static_for<NB1>([&](auto ii) {
      constexpr int i = ii.value;
      dft_sub<R1, false, true, false, i * R1, 1>(x);
      const int n = t + T * i;
      static_for<R1>([&](auto kk) {
        constexpr int k = kk.value;
        float2 v = x[i * R1 + k];
        if constexpr (k != 0) v = cmul(v, twiddle<LOG2M>(tw, uint32_t(n * k)));
        lds[lds_pad(n + k * Q1)] = v;
      });
    });
  }
  // ---- forward pass 2 (LDS -> LDS)
  __device__ __forceinline__ static void fwd2(float2 (&x)[E], float2* lds, const Twiddles& tw, int t) {
    static_for<NB2>([&](auto ii) {
      constexpr int i = ii.value;
      const int b = t + T * i;
      const int blk = b / Q2, n = b % Q2;
      const int base = blk * S2 + n;
      static_for<R2>([&](auto m) { x[i * R2 + m.value] = lds[lds_pad(base + m.value * Q2)]; });
    });
    static_for<NB2>([&](auto ii) {
      constexpr int i = ii.value;
      const int b = t + T * i;
      const int n = b % Q2;
      const int base = (b / Q2) * S2 + n;
      dft_sub<R2, false, false, false, i * R2, 1>(x);
      static_for<R2>([&](auto kk) {
        constexpr int k = kk.value;
        float2 v = x[i * R2 + k];
        if constexpr (k != 0) v = cmul(v, twiddle<ilog2(S2)>(tw, uint32_t(n * k)));
        lds[lds_pad(base + k * Q2)] = v;
      });
    });
  }
  // ---- forward pass 3: read blocks A (x[0..R3)) and B (x[R3..2R3)), DFT; no twiddles (S = R3)
  __device__ __forceinline__ static void fwd3(float2 (&x)[E], const float2* lds, const Pair& p) {
    static_for<R3>([&](auto m) {
      x[m.value] = lds[lds_pad(p.betaA * R3 + m.value)];
      x[R3 + m.value] = lds[lds_pad(p.betaB * R3 + m.value)];
    });
    dft_sub<R3, false, false, false, 0, 1>(x);
    dft_sub<R3, false, false, false, R3, 1>(x);
  }
  // ---- inverse pass 3: inverse DFT of both blocks, write back to their LDS positions
  __device__ __forceinline__ static void inv3(float2 (&x)[E], float2* lds, const Pair& p) {
    dft_sub<R3, true, false, false, 0, 1>(x);
    dft_sub<R3, true, false, false, R3, 1>(x);
    static_for<R3>([&](auto m) {
      lds[lds_pad(p.betaA * R3 + m.value)] = x[m.value];
      lds[lds_pad(p.betaB * R3 + m.value)] = x[R3 + m.value];
    });
  }
  // ---- inverse pass 2 (LDS -> LDS): input twiddles conj(W_S2^{nk}), inverse DFT
  __device__ __forceinline__ static void inv2(float2 (&x)[E], float2* lds, const Twiddles& tw, int t) {
    static_for<NB2>([&](auto ii) {
      constexpr int i = ii.value;
      const int b = t + T * i;
      const int n = b % Q2;
      const int base = (b / Q2) * S2 + n;
      static_for<R2>([&](auto kk) {
        constexpr int k = kk.value;
        float2 v = lds[lds_pad(base + k * Q2)];
        if constexpr (k != 0) v = cmulc(v, twiddle<ilog2(S2)>(tw, uint32_t(n * k)));
        x[i * R2 + k] = v;
      });
    });
    static_for<NB2>([&](auto ii) {
      constexpr int i = ii.value;
      const int b = t + T * i;
      const int base = (b / Q2) * S2 + b % Q2;
      dft_sub<R2, true, false, false, i * R2, 1>(x);
      static_for<R2>([&](auto m) { lds[lds_pad(base + m.value * Q2)] = x[i * R2 + m.value]; });
    });
  }
  // ---- inverse pass 1 (LDS -> registers): only outputs m < R1/2 (positions < M/2) are formed;
  //      x[i R1 + m] then holds z'[b + m Q1]
  __device__ __forceinline__ static void inv1(float2 (&x)[E], const float2* lds, const Twiddles& tw, int t) {
    static_for<NB1>([&](auto ii) {
      constexpr int i = ii.value;
      const int n = t + T * i;
      static_for<R1>([&](auto kk) {
        constexpr int k = kk.value;
        float2 v = lds[lds_pad(n + k * Q1)];
        if constexpr (k != 0) v = cmulc(v, twiddle<LOG2M>(tw, uint32_t(n * k)));
        x[i * R1 + k] = v;
      });
      dft_sub<R1, true, false, true, i * R1, 1>(x);
    });
  }
};

// Real-input split, product with the filter spectrum and re-pack for the inverse, for one pair of
// mirrored bins (k, M-k).  A = Z[k], B = Z[M-k] (B == A for a bin that is its own mirror),
// w = W_{2M}^k, hk = Hs[k], hp = Hs[M-k], Hs = H / (4M).  On return A = Z''[k], B = Z''[M-k], where
// the unnormalised inverse M-point DFT of Z'' packs the 2M-point real result (y[2n], y[2n+1]).
//   X[k]   = E + w O,  X[M-k] = conj(E - w O),  E = (A + conj B)/2,  O = (A - conj B)/(2i)
//   Y = X H;  Z'[k] = Ye + i Yo,  Ye = (Y[k] + conj Y[M-k])/2,  Yo = (Y[k] - conj Y[M-k]) conj(w)/2
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

// Real-input split only: returns 2 X[k] and 2 X[M-k] (used to build the filter spectrum).
__device__ __forceinline__ void split_pair(float2 A, float2 B, float2 w, float2& Xk, float2& Xp) {
  const float2 Bc = cconj(B);
  const float2 E2 = cadd(A, Bc);
  const float2 Dd = csub(A, Bc);
  const float2 O2 = make_float2(Dd.y, -Dd.x);
  const float2 wO = cmul(w, O2);
  Xk = cadd(E2, wO);
  Xp = cconj(csub(E2, wO));
}

}  // namespace hyena
