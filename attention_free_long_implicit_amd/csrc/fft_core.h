// Device-side building blocks of the FFT engine used by every Hyena kernel (gfx950, wave64).
//
// * complex helpers on float2 (x = real, y = imaginary), fp32 arithmetic throughout;
// * in-register radix-R DFTs (R = 2..64) whose twiddles are compile-time constants, written as
//   radix-2 decimation-in-time stages on a register renaming of the input (the renaming costs
//   nothing: every index is a compile-time constant after unrolling);
//   pruned forms for an input whose upper half is zero and for an output whose upper half is
//   not needed, which is what zero-padding a length-L signal to 2L and keeping the first L
//   outputs leaves (HyenaND summary, boundary handling: zero-pad to twice the size);
// * twiddle factors W_N^j = exp(-2 pi i j / N) for N = 2^n <= 2^21 from tables the host computes
//   in double precision; within one butterfly the powers w^k of a looked-up w are formed by
//   squaring (a few roundings deep, independent of L);
// * bf16 load/store with round-to-nearest-even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace hyena {

// ------------------------------------------------------------------ complex helpers
__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}
// a * conj(b)
__device__ __forceinline__ float2 cmulc(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, a.y * b.y), fmaf(a.y, b.x, -a.x * b.y));
}
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
__device__ __forceinline__ float2 cscale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }

// ------------------------------------------------------------------ compile-time loops
template <int N, class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------------ compile-time trigonometry
// cos / sin of 2 pi j / n in double, by Taylor series after reduction to [-pi/4, pi/4] with the
// octant symmetries; used only to fold constant twiddles into the instruction stream.
constexpr double kPi = 3.14159265358979323846264338327950288;
constexpr double ce_sin_small(double x) {
  double term = x, sum = x, x2 = x * x;
  for (int k = 1; k < 14; ++k) { term *= -x2 / ((2 * k) * (2 * k + 1)); sum += term; }
  return sum;
}
constexpr double ce_cos_small(double x) {
  double term = 1.0, sum = 1.0, x2 = x * x;
  for (int k = 1; k < 14; ++k) { term *= -x2 / ((2 * k - 1) * (2 * k)); sum += term; }
  return sum;
}
// returns cos(2 pi j / n) (want_sin = false) or sin(2 pi j / n)
constexpr double ce_trig(long j, long n, bool want_sin) {
  j %= n; if (j < 0) j += n;
  // reduce to the first octant using exact integer arithmetic on 8 j / n
  long q8 = 8 * j;                 // angle in units of (2 pi / 8n)
  long oct = q8 / n;               // octant 0..7
  double r = double(q8 - oct * n) / double(n);   // fraction of an octant in [0, 1)
  double th = r * (kPi / 4);
  double c = 0, s = 0;
  // angle = oct * pi/4 + th
  switch (oct) {
    case 0: c = ce_cos_small(th); s = ce_sin_small(th); break;
    case 1: c = ce_sin_small(kPi / 4 - th); s = ce_cos_small(kPi / 4 - th); break;
    case 2: c = -ce_sin_small(th); s = ce_cos_small(th); break;
    case 3: c = -ce_cos_small(kPi / 4 - th); s = ce_sin_small(kPi / 4 - th); break;
    case 4: c = -ce_cos_small(th); s = -ce_sin_small(th); break;
    case 5: c = -ce_sin_small(kPi / 4 - th); s = -ce_cos_small(kPi / 4 - th); break;
    case 6: c = ce_sin_small(th); s = -ce_cos_small(th); break;
    default: c = ce_cos_small(kPi / 4 - th); s = -ce_sin_small(kPi / 4 - th); break;
  }
  return want_sin ? s : c;
}

// v * W_n^j with W = exp(-2 pi i / n) (forward) or exp(+2 pi i / n) (INV); j, n compile-time.
template <long J, long N, bool INV>
__device__ __forceinline__ float2 mul_w(float2 v) {
  constexpr long j = ((J % N) + N) % N;
  if constexpr (j == 0) {
    return v;
  } else if constexpr (4 * j == N) {          // -i (forward) / +i (inverse)
    return INV ? make_float2(-v.y, v.x) : make_float2(v.y, -v.x);
  } else if constexpr (2 * j == N) {
    return make_float2(-v.x, -v.y);
  } else if constexpr (4 * j == 3 * N) {      // +i (forward) / -i (inverse)
    return INV ? make_float2(v.y, -v.x) : make_float2(-v.y, v.x);
  } else {
    constexpr float c = (float)ce_trig(j, N, false);
    constexpr float s0 = (float)ce_trig(j, N, true);
    constexpr float s = INV ? s0 : -s0;       // W = c + i s
    return make_float2(fmaf(v.x, c, -v.y * s), fmaf(v.x, s, v.y * c));
  }
}

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n >> 1); }
constexpr int bitrev(int x, int bits) {
  int r = 0;
  for (int i = 0; i < bits; ++i) r |= ((x >> i) & 1) << (bits - 1 - i);
  return r;
}

// ------------------------------------------------------------------ in-register DFT
// X[k] = sum_m x[m] W_R^{mk}, natural order in and out, as radix-2 decimation-in-time stages on
// the bit-reversed renaming of the input (the renaming is free: all indices are constants).
// A butterfly with a non-trivial twiddle w costs 6 instructions: a' = a + w b as two chained FMAs
// per component, b' = 2a - a' as one FMA per component.
//   ZERO_UPPER: x[m] = 0 for m >= R/2 (those registers are not read; the first stage is a copy).
//   HALF_OUT:   only X[k] for k < R/2 is produced (upper registers are left undefined).
template <long J, long N, bool INV>
__device__ __forceinline__ void bfly_dit(float2& a, float2& b) {
  constexpr long j = ((J % N) + N) % N;
  if constexpr (j == 0) {
    const float2 t = b;
    b = csub(a, t); a = cadd(a, t);
  } else if constexpr (4 * j == N) {            // w = -i (forward) / +i (inverse)
    const float2 t = INV ? make_float2(-b.y, b.x) : make_float2(b.y, -b.x);
    b = csub(a, t); a = cadd(a, t);
  } else {
    constexpr float c = (float)ce_trig(j, N, false);
    constexpr float s0 = (float)ce_trig(j, N, true);
    constexpr float s = INV ? s0 : -s0;         // w = c + i s
    const float ax = fmaf(c, b.x, fmaf(-s, b.y, a.x));
    const float ay = fmaf(c, b.y, fmaf(s, b.x, a.y));
    b = make_float2(fmaf(2.0f, a.x, -ax), fmaf(2.0f, a.y, -ay));
    a = make_float2(ax, ay);
  }
}
template <long J, long N, bool INV>
__device__ __forceinline__ void bfly_dit_top(float2& a, const float2& b) {   // only a' = a + w b
  constexpr long j = ((J % N) + N) % N;
  if constexpr (j == 0) {
    a = cadd(a, b);
  } else if constexpr (4 * j == N) {
    a = cadd(a, INV ? make_float2(-b.y, b.x) : make_float2(b.y, -b.x));
  } else {
    constexpr float c = (float)ce_trig(j, N, false);
    constexpr float s0 = (float)ce_trig(j, N, true);
    constexpr float s = INV ? s0 : -s0;
    a = make_float2(fmaf(c, b.x, fmaf(-s, b.y, a.x)), fmaf(c, b.y, fmaf(s, b.x, a.y)));
  }
}

template <int R, bool INV, bool ZERO_UPPER = false, bool HALF_OUT = false>
__device__ __forceinline__ void dft(float2 (&x)[R]) {
  static_assert(R >= 2 && (R & (R - 1)) == 0 && R <= 64, "radix must be a power of two <= 64");
  constexpr int LR = ilog2(R);
  float2 v[R];
  static_for<R>([&](auto i) {
    constexpr int src = bitrev(i.value, LR);
    if constexpr (!(ZERO_UPPER && src >= R / 2)) v[i.value] = x[src];
  });
  static_for<LR>([&](auto s) {
    constexpr int span = 1 << s.value;
    constexpr bool first = (s.value == 0);
    constexpr bool last = (s.value == LR - 1);
    static_for<R / (2 * span)>([&](auto bi) {
      constexpr int blk = bi.value * 2 * span;
      static_for<span>([&](auto jj) {
        constexpr int j = jj.value;
        constexpr int i0 = blk + j, i1 = blk + j + span;
        if constexpr (first && ZERO_UPPER) {
          v[i1] = v[i0];                       // odd input is zero: both outputs equal the even one
        } else if constexpr (last && HALF_OUT) {
          bfly_dit_top<j, 2 * span, INV>(v[i0], v[i1]);
        } else {
          bfly_dit<j, 2 * span, INV>(v[i0], v[i1]);
        }
      });
    });
  });
  static_for<R>([&](auto k) {
    if constexpr (!HALF_OUT || k.value < R / 2) x[k.value] = v[k.value];
  });
}

// Same on a register sub-array x[OFF + m * STRIDE], m < R, of a larger array.
template <int R, bool INV, bool ZERO_UPPER, bool HALF_OUT, int OFF, int STRIDE, int N>
__device__ __forceinline__ void dft_sub(float2 (&x)[N]) {
  float2 v[R];
  static_for<R>([&](auto m) {
    if constexpr (!(ZERO_UPPER && m.value >= R / 2)) v[m.value] = x[OFF + m.value * STRIDE];
  });
  dft<R, INV, ZERO_UPPER, HALF_OUT>(v);
  static_for<R>([&](auto k) {
    if constexpr (!(HALF_OUT && k.value >= R / 2)) x[OFF + k.value * STRIDE] = v[k.value];
  });
}

// ------------------------------------------------------------------ twiddle tables
// pow2[2^s + j] = W_{2^s}^j for s <= 15, j < 2^s (each size contiguous, so lanes with consecutive j
// read consecutive addresses);  fine[b] = W_{2^21}^b, b < 64, for sizes above 2^15:
//   W_N^j = W_{2^15}^{j >> (n-15)} * W_{2^21}^{(j mod 2^(n-15)) << (21-n)}.
constexpr int kTwPow2Log2 = 15;
constexpr int kTwPow2Entries = 2 << kTwPow2Log2;     // offsets 0..2^16 (entry 0 unused)
constexpr int kTwFineLog2 = 6;
constexpr int kTwFine = 1 << kTwFineLog2;
constexpr int kTwMaxLog2 = kTwPow2Log2 + kTwFineLog2;   // 21

struct Twiddles {
  const float2* __restrict__ pow2;   // [kTwPow2Entries]
  const float2* __restrict__ fine;   // [kTwFine]
};

// W_{2^LOG2N}^j (forward sign), j taken mod 2^LOG2N.
template <int LOG2N>
__device__ __forceinline__ float2 twiddle(const Twiddles& tw, uint32_t j) {
  static_assert(LOG2N <= kTwMaxLog2, "twiddle table too small");
  j &= (1u << LOG2N) - 1u;
  if constexpr (LOG2N <= kTwPow2Log2) {
    return tw.pow2[(1u << LOG2N) + j];
  } else {
    constexpr int sh = LOG2N - kTwPow2Log2;
    const float2 c = tw.pow2[(1u << kTwPow2Log2) + (j >> sh)];
    const uint32_t r = j & ((1u << sh) - 1u);
    return r ? cmul(c, tw.fine[r << (kTwMaxLog2 - LOG2N)]) : c;
  }
}

__device__ __forceinline__ float2 csq(float2 a) { return make_float2(fmaf(a.x, a.x, -a.y * a.y), 2.0f * a.x * a.y); }

// p[k] = w^k, k < R (p[0] = 1), by repeated squaring / one extra product: depth about 2 log2 k.
template <int R>
__device__ __forceinline__ void twiddle_powers(float2 w, float2 (&p)[R]) {
  p[0] = make_float2(1.f, 0.f);
  if constexpr (R > 1) p[1] = w;
  static_for<R>([&](auto kk) {
    constexpr int k = kk.value;
    if constexpr (k >= 2) {
      if constexpr (k % 2 == 0) p[k] = csq(p[k / 2]);
      else p[k] = cmul(p[k - 1], w);
    }
  });
}

// ------------------------------------------------------------------ storage types
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
// bf16 rounding to nearest even (the hardware conversion; NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t b = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, b);
}

// Block scaling of fp16 intermediates: e such that m * 2^-e lies in [2^14, 2^15) (fp16 holds up to 65504);
// 0 for a zero or non-finite m (which then passes through unscaled).  e >= -112 keeps 2^-e finite.
__device__ __forceinline__ int h16_exponent(float m) {
  if (!(m > 0.0f) || !(m <= 3.0e38f)) return 0;
  const int e = __builtin_amdgcn_frexp_expf(m) - 15;
  return e < -112 ? -112 : e;
}

// Two consecutive stored elements (one packed complex sample) <-> float2.
template <bool BF16> struct Store;
template <> struct Store<false> {
  using elem = float;
  __device__ __forceinline__ static float2 load2(const float* p) { return *reinterpret_cast<const float2*>(p); }
  __device__ __forceinline__ static void store2(float* p, float2 v) { *reinterpret_cast<float2*>(p) = v; }
};
template <> struct Store<true> {
  using elem = uint16_t;
  __device__ __forceinline__ static float2 load2(const uint16_t* p) {
    uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
  }
  __device__ __forceinline__ static void store2(uint16_t* p, float2 v) {
    *reinterpret_cast<uint32_t*>(p) = f32x2_to_bf16x2_rne(v.x, v.y);
  }
};

// ------------------------------------------------------------------ LDS padding
// One float2 of padding after every 16: rows of 16 contiguous elements read by consecutive lanes
// then fall on distinct banks.
__device__ __forceinline__ int lds_pad(int p) { return p + (p >> 4); }
constexpr int lds_padded_size(int n) { return n + (n >> 4); }

// ------------------------------------------------------------------ XCD-aware block order
// Consecutive workgroups are dealt round-robin to the 8 XCDs; remap so that each XCD receives a
// contiguous run of logical block ids (rows that share a filter then share that XCD's L2).
__device__ __forceinline__ int xcd_logical_block(int bid, int nblk) {
  constexpr int kXcd = 8;
  const int per = nblk / kXcd;
  if (bid >= per * kXcd) return bid;        // tail keeps its identity
  return (bid % kXcd) * per + bid / kXcd;
}

}  // namespace hyena
