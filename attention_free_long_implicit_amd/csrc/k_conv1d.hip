// Single-pass kernels for 1-D causal long convolution, L <= 16384 (the transform lives in LDS):
//   k_conv1d       y = gate * (h conv u)[0:L) for every (b, d) row, one workgroup per row
//   k_spectrum1d   filter spectrum in engine order from time-domain taps h[d, 0:L)
//   k_export1d     engine-order spectrum -> natural-order bins H[d, 0..L] (testing aid)
//
// Operation: Hyena study note, step 2 (long convolution with the implicit filter) and step 3
// (multiplicative gate); EulerStack "4. Hyena 상세", how it works 2 (FFT -> elementwise product ->
// inverse FFT); HyenaND summary, nSubQ implementation (forward transform, spectral modulation,
// inverse transform and output cut fused in one kernel with the intermediates on chip).
#include "engine1.h"
#include "launch.h"

namespace hyena {

template <int LOG2M, bool BF16, bool GATE>
__global__ void __launch_bounds__(Engine1<LOG2M>::T)
k_conv1d(const typename Store<BF16>::elem* u, const typename Store<BF16>::elem* gate,
         typename Store<BF16>::elem* y, const float2* __restrict__ Hs, int B, int D, Twiddles tw) {
  using En = Engine1<LOG2M>;
  using St = Store<BF16>;
  constexpr int M = En::M, T = En::T, E = En::E, R1 = En::R1, R3 = En::R3, Q1 = En::Q1;
  __shared__ float2 lds[En::LDS_ELEMS];
  const int t = threadIdx.x;
  const int r = xcd_logical_block(blockIdx.x, B * D);
  const int d = r / B, b = r % B;
  const size_t row = (size_t)b * D + d;
  const auto* urow = u + row * M;
  float2 x[E];
  static_for<En::NB1>([&](auto ii) {
    constexpr int i = ii.value;
    static_for<R1 / 2>([&](auto m) { x[i * R1 + m.value] = St::load2(urow + 2 * (t + T * i + m.value * Q1)); });
  });
  En::fwd1(x, lds, tw, t);
  __syncthreads();
  En::fwd2(x, lds, tw, t);
  __syncthreads();
  const auto P = En::pair_of(t);
  En::fwd3(x, lds, P);

  const float2* hrow = Hs + (size_t)d * M;
  if (!P.special) {
    static_for<R3>([&](auto mm) {
      constexpr int m = mm.value, mp = 2 * R3 - 1 - m;
      const float2 w = twiddle<LOG2M + 1>(tw, uint32_t(P.kapA + (M / R3) * m));
      spectral_pair(x[m], x[mp], w, hrow[m * T + t], hrow[mp * T + t]);
    });
  } else {
    static_for<R3 / 2 + 1>([&](auto mm) {
      constexpr int m = mm.value, mp = (R3 - m) % R3;
      const float2 w = twiddle<LOG2M + 1>(tw, uint32_t((M / R3) * m));
      if constexpr (m == 0) {
        const float2 s = hrow[t];
        float2 bb = x[0];
        spectral_pair(x[0], bb, w, make_float2(s.x, 0.f), make_float2(s.y, 0.f));
      } else if constexpr (m == R3 / 2) {
        float2 bb = x[m];
        const float2 h = hrow[m * T + t];
        spectral_pair(x[m], bb, w, h, h);
      } else {
        spectral_pair(x[m], x[mp], w, hrow[m * T + t], hrow[mp * T + t]);
      }
    });
    static_for<R3 / 2>([&](auto mm) {
      constexpr int m = R3 + mm.value, mp = 2 * R3 - 1 - mm.value;
      const float2 w = twiddle<LOG2M + 1>(tw, uint32_t(P.kapB + (M / R3) * mm.value));
      spectral_pair(x[m], x[mp], w, hrow[m * T + t], hrow[mp * T + t]);
    });
  }

  En::inv3(x, lds, P);
  __syncthreads();
  En::inv2(x, lds, tw, t);
  __syncthreads();
  En::inv1(x, lds, tw, t);

  auto* yrow = y + row * M;
  const auto* grow = GATE ? gate + row * M : nullptr;
  static_for<En::NB1>([&](auto ii) {
    constexpr int i = ii.value;
    static_for<R1 / 2>([&](auto m) {
      const int j = t + T * i + m.value * Q1;
      float2 v = x[i * R1 + m.value];
      if constexpr (GATE) {
        const float2 g = St::load2(grow + 2 * j);
        v = make_float2(v.x * g.x, v.y * g.y);
      }
      St::store2(yrow + 2 * j, v);
    });
  });
}

// Filter spectrum in engine order: Hs = DFT_{2L}(h || 0) / (4L), see Engine1.
template <int LOG2M>
__global__ void __launch_bounds__(Engine1<LOG2M>::T)
k_spectrum1d(const float* __restrict__ h, float2* __restrict__ Hs, Twiddles tw) {
  using En = Engine1<LOG2M>;
  constexpr int M = En::M, T = En::T, E = En::E, R1 = En::R1, R3 = En::R3, Q1 = En::Q1;
  __shared__ float2 lds[En::LDS_ELEMS];
  const int t = threadIdx.x;
  const int d = blockIdx.x;
  const float* hrow = h + (size_t)d * M;
  float2 x[E];
  static_for<En::NB1>([&](auto ii) {
    constexpr int i = ii.value;
    static_for<R1 / 2>([&](auto m) {
      x[i * R1 + m.value] = Store<false>::load2(hrow + 2 * (t + T * i + m.value * Q1));
    });
  });
  En::fwd1(x, lds, tw, t);
  __syncthreads();
  En::fwd2(x, lds, tw, t);
  __syncthreads();
  const auto P = En::pair_of(t);
  En::fwd3(x, lds, P);
  const float sc = 1.0f / (8.0f * M);
  float2* out = Hs + (size_t)d * M;
  if (!P.special) {
    static_for<R3>([&](auto mm) {
      constexpr int m = mm.value, mp = 2 * R3 - 1 - m;
      const float2 w = twiddle<LOG2M + 1>(tw, uint32_t(P.kapA + (M / R3) * m));
      float2 Xk, Xp;
      split_pair(x[m], x[mp], w, Xk, Xp);
      out[m * T + t] = cscale(Xk, sc);
      out[mp * T + t] = cscale(Xp, sc);
    });
  } else {
    static_for<R3 / 2 + 1>([&](auto mm) {
      constexpr int m = mm.value, mp = (R3 - m) % R3;
      const float2 w = twiddle<LOG2M + 1>(tw, uint32_t((M / R3) * m));
      float2 Xk, Xp;
      split_pair(x[m], x[mp], w, Xk, Xp);
      if constexpr (m == 0) {
        out[t] = make_float2(Xk.x * sc, Xp.x * sc);
      } else {
        out[m * T + t] = cscale(Xk, sc);
        if constexpr (m != R3 / 2) out[mp * T + t] = cscale(Xp, sc);
      }
    });
    static_for<R3 / 2>([&](auto mm) {
      constexpr int m = R3 + mm.value, mp = 2 * R3 - 1 - mm.value;
      const float2 w = twiddle<LOG2M + 1>(tw, uint32_t(P.kapB + (M / R3) * mm.value));
      float2 Xk, Xp;
      split_pair(x[m], x[mp], w, Xk, Xp);
      out[m * T + t] = cscale(Xk, sc);
      out[mp * T + t] = cscale(Xp, sc);
    });
  }
}

// Engine-order spectrum -> H[d, k], k = 0..L (unscaled 2L-point DFT bins).
template <int LOG2M>
__global__ void k_export1d(const float2* __restrict__ Hs, float2* __restrict__ H) {
  using En = Engine1<LOG2M>;
  constexpr int M = En::M, T = En::T, E = En::E;
  const int d = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;   // slot * T + t
  if (idx >= M) return;
  const int slot = idx / T, t = idx % T;
  const float sc = 4.0f * M;
  const float2 v = Hs[(size_t)d * M + idx];
  float2* out = H + (size_t)d * (M + 1);
  if (t == T - 1 && slot == 0) {
    out[0] = make_float2(v.x * sc, 0.f);
    out[M] = make_float2(v.y * sc, 0.f);
  } else {
    out[En::slot_bin(t, slot)] = cscale(v, sc);
  }
  (void)E;
}

// ------------------------------------------------------------------ host launchers
namespace {
template <int LOG2M>
hipError_t conv1d_launch(int bf16, bool gate, const void* u, const void* g, void* y, const float2* Hs, int B,
                         int D, const Twiddles& tw, hipStream_t s) {
  using En = Engine1<LOG2M>;
  dim3 grid(B * D), block(En::T);
  if (bf16) {
    using E = uint16_t;
    if (gate)
      hipLaunchKernelGGL((k_conv1d<LOG2M, true, true>), grid, block, 0, s, (const E*)u, (const E*)g, (E*)y, Hs, B, D, tw);
    else
      hipLaunchKernelGGL((k_conv1d<LOG2M, true, false>), grid, block, 0, s, (const E*)u, (const E*)g, (E*)y, Hs, B, D, tw);
  } else {
    using E = float;
    if (gate)
      hipLaunchKernelGGL((k_conv1d<LOG2M, false, true>), grid, block, 0, s, (const E*)u, (const E*)g, (E*)y, Hs, B, D, tw);
    else
      hipLaunchKernelGGL((k_conv1d<LOG2M, false, false>), grid, block, 0, s, (const E*)u, (const E*)g, (E*)y, Hs, B, D, tw);
  }
  return hipGetLastError();
}
template <int LOG2M>
hipError_t spectrum1d_launch(const float* h, float2* Hs, int D, const Twiddles& tw, hipStream_t s) {
  hipLaunchKernelGGL((k_spectrum1d<LOG2M>), dim3(D), dim3(Engine1<LOG2M>::T), 0, s, h, Hs, tw);
  return hipGetLastError();
}
template <int LOG2M>
hipError_t export1d_launch(const float2* Hs, float2* H, int D, hipStream_t s) {
  constexpr int M = 1 << LOG2M;
  hipLaunchKernelGGL((k_export1d<LOG2M>), dim3((M + 255) / 256, D), dim3(256), 0, s, Hs, H);
  return hipGetLastError();
}
}  // namespace

bool single_pass_supported(int log2L) { return log2L >= 10 && log2L <= 14; }

hipError_t launch_conv1d_single(int log2L, int bf16, const void* u, const void* gate, void* y, const float2* Hs,
                                int B, int D, const Twiddles& tw, hipStream_t s) {
  const bool g = gate != nullptr;
  switch (log2L) {
    case 10: return conv1d_launch<10>(bf16, g, u, gate, y, Hs, B, D, tw, s);
    case 11: return conv1d_launch<11>(bf16, g, u, gate, y, Hs, B, D, tw, s);
    case 12: return conv1d_launch<12>(bf16, g, u, gate, y, Hs, B, D, tw, s);
    case 13: return conv1d_launch<13>(bf16, g, u, gate, y, Hs, B, D, tw, s);
    case 14: return conv1d_launch<14>(bf16, g, u, gate, y, Hs, B, D, tw, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_spectrum1d_single(int log2L, const float* h, float2* Hs, int D, const Twiddles& tw,
                                    hipStream_t s) {
  switch (log2L) {
    case 10: return spectrum1d_launch<10>(h, Hs, D, tw, s);
    case 11: return spectrum1d_launch<11>(h, Hs, D, tw, s);
    case 12: return spectrum1d_launch<12>(h, Hs, D, tw, s);
    case 13: return spectrum1d_launch<13>(h, Hs, D, tw, s);
    case 14: return spectrum1d_launch<14>(h, Hs, D, tw, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_export1d_single(int log2L, const float2* Hs, float2* H, int D, hipStream_t s) {
  switch (log2L) {
    case 10: return export1d_launch<10>(Hs, H, D, s);
    case 11: return export1d_launch<11>(Hs, H, D, s);
    case 12: return export1d_launch<12>(Hs, H, D, s);
    case 13: return export1d_launch<13>(Hs, H, D, s);
    case 14: return export1d_launch<14>(Hs, H, D, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace hyena
