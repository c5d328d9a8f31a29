// Single-pass kernels for 1-D long convolution whose transform lives in LDS: causal for L <= 16384,
// periodic (circular) for L <= 32768:
//   k_conv1d       y = gate * (h conv u)[0:L) for every (b, d) row, one workgroup per row
//   k_spectrum1d   filter spectrum in engine order from time-domain taps h[d, 0:L)
//   k_export1d     engine-order spectrum -> natural-order bins H[d, 0..L] (testing aid)
//
// Operation: Hyena study note, step 2 (long convolution with the implicit filter) and step 3
// (multiplicative gate); EulerStack "4. Hyena 상세", how it works 2 (FFT -> elementwise product ->
// inverse FFT); HyenaND summary, nSubQ implementation (forward transform, spectral modulation,
// inverse transform and output cut fused in one kernel with the intermediates on chip).
//
// A row u[0..L) is zero-padded to 2L and packed two samples per complex value,
// z[n] = u[2n] + i u[2n+1] (n < L/2; zero above), so the M = L point complex transform of z gives
// the 2L-point real transform after the mirrored-bin split (spectral_pair).  The product of the
// zero-padded spectra is the linear convolution; keeping outputs [0, L) makes it causal.
//
// Periodic boundary (FULL = true; HyenaND summary, boundary handling: circular convolution for
// periodic systems, no padding): a row of L = 2M samples fills all M packed values, so the same
// M-point transform and split give the L-point real transform; the product is the circular
// convolution and every output is kept.  The filter spectrum is that of the L taps, unpadded.
//
// Spectrum layout ("engine order"), per channel: Hs[slot * T + t], slot < 2 RP, holding Hs = H/(4L)
// at the bin of register `slot` of thread t in the fused pass; thread T-1, slot 0 holds the two
// real bins (Hs[0], Hs[L]).
#include "engine.h"
#include "launch.h"

namespace hyena {

template <int LOG2M> struct SinglePlan;
template <> struct SinglePlan<10> { using RL = Radices<16, 8, 8>; };
template <> struct SinglePlan<11> { using RL = Radices<16, 16, 8>; };
template <> struct SinglePlan<12> { using RL = Radices<16, 4, 8, 8>; };
template <> struct SinglePlan<13> { using RL = Radices<16, 8, 8, 8>; };
template <> struct SinglePlan<14> { using RL = Radices<16, 16, 8, 8>; };

template <int LOG2M>
struct Single {
  using RL = typename SinglePlan<LOG2M>::RL;
  using En = RowEngine<1, RL>;
  using NP = NegPairs<RL>;
  static constexpr int M = 1 << LOG2M, T = En::T, E = En::E, R0 = RL::R[0], RP = RL::RP, Q0 = M / R0;
  static constexpr int NB0 = E / R0;          // pass-0 butterflies per thread
  static_assert(RL::S == M && NP::TN == T, "plan");
};

// Orders i = 0..order-1 back to back in one launch (the cross-order fusion of the nSubQ pattern: one
// HBM read of the row and of each gate, one store of the result).  Between orders u_i stays in registers
// in fp32 -- also for bf16 storage, where only v, the gates and y are bf16 -- so for fp32 storage a chain
// equals `order` one-order launches bit for bit.  GATE = false only for a single order without a gate.
template <int LOG2M, bool BF16, bool GATE, bool FULL>
__global__ void __launch_bounds__(Single<LOG2M>::T, 4)
k_conv1d(const typename Store<BF16>::elem* u, ConvChain ch, int order, typename Store<BF16>::elem* y, int B,
         int D, int hsb, Twiddles tw0) {
  using C = Single<LOG2M>;
  using En = typename C::En;
  using St = Store<BF16>;
  using Elem = typename St::elem;
  constexpr int M = C::M, T = C::T, E = C::E, R0 = C::R0, RP = C::RP, Q0 = C::Q0;
  __shared__ float2 lds[En::LDS_ELEMS];
  const int t = threadIdx.x;
  const int r = xcd_logical_block(blockIdx.x, B * D);
  const int d = r / B, b = r % B;
  const size_t row = (size_t)b * D + d;
  constexpr int RS = FULL ? 2 * M : M;        // samples per row
  constexpr int NIN = FULL ? R0 : R0 / 2;     // nonzero inputs (and kept outputs) per first-pass butterfly
  const auto* urow = u + row * RS;
  float2 x[E];
  static_for<C::NB0>([&](auto ii) {
    constexpr int i = ii.value;
    static_for<NIN>([&](auto m) { x[i * R0 + m.value] = St::load2(urow + 2 * (t + T * i + m.value * Q0)); });
  });
  const size_t hrow = (size_t)(d + b * hsb) * M;             // hsb = 0: one filter per channel; D: per (b, d)
  for (int o = 0; o < order; ++o) {
    if (o > 0) __syncthreads();               // the previous order's last inverse pass read the LDS
    // Everything derived from the thread index and the twiddle tables is recomputed per order: kept live
    // across the loop it would not fit the register budget next to the row.
    int t = threadIdx.x;
    Twiddles tw = tw0;
    asm volatile("" : "+v"(t));
    asm volatile("" : "+s"(tw.pow2), "+s"(tw.fine));
    t &= T - 1;                               // restores the range the index arithmetic is specialised on
    const auto P = C::NP::of(t);
    En::template forward_to_last<!FULL>(x, lds, tw, t);
    En::fwd_last(x, lds, P.betaA, P.betaB);
    const float2* hs = ch.spectrum[o] + hrow + t;
    if (!P.special) {
      spectral_complement<RP, 0>(x, twiddle<LOG2M + 1>(tw, uint32_t(P.kapA)), hs, T, nullptr, 0.f);
    } else {
      spectral_selfmirror<RP, 0>(x, twiddle<LOG2M + 1>(tw, uint32_t(P.kapB)), hs, T, nullptr, 0.f);
    }
    En::inv_last(x, lds, P.betaA, P.betaB);
    En::template inverse_from_last<!FULL>(x, lds, tw, t);

    const bool last = o + 1 == order;
    const auto* grow = GATE ? static_cast<const Elem*>(ch.gate[o]) + row * RS : nullptr;
    auto* yrow = y + row * RS;
    static_for<C::NB0>([&](auto ii) {
      constexpr int i = ii.value;
      static_for<NIN>([&](auto m) {
        const int j = t + T * i + m.value * Q0;
        float2 v = x[i * R0 + m.value];
        if constexpr (GATE) {
          const float2 g = St::load2(grow + 2 * j);
          v = make_float2(v.x * g.x, v.y * g.y);
        }
        if (last) St::store2(yrow + 2 * j, v);
        else x[i * R0 + m.value] = v;
      });
    });
  }
}

// Filter spectrum in engine order: Hs = DFT_{2M}(h || 0) / (4M) from M taps, or (FULL) Hs = DFT_{2M}(h) / (4M)
// from 2M taps (periodic boundary).
template <int LOG2M, bool FULL>
__global__ void __launch_bounds__(Single<LOG2M>::T)
k_spectrum1d(const float* __restrict__ h, float2* __restrict__ Hs, Twiddles tw) {
  using C = Single<LOG2M>;
  using En = typename C::En;
  constexpr int M = C::M, T = C::T, E = C::E, R0 = C::R0, RP = C::RP, Q0 = C::Q0;
  __shared__ float2 lds[En::LDS_ELEMS];
  const int t = threadIdx.x;
  const int d = blockIdx.x;
  const float* hrow = h + (size_t)d * (FULL ? 2 * M : M);
  float2 x[E];
  static_for<C::NB0>([&](auto ii) {
    constexpr int i = ii.value;
    static_for<FULL ? R0 : R0 / 2>([&](auto m) {
      x[i * R0 + m.value] = Store<false>::load2(hrow + 2 * (t + T * i + m.value * Q0));
    });
  });
  En::template forward_to_last<!FULL>(x, lds, tw, t);
  const auto P = C::NP::of(t);
  En::fwd_last(x, lds, P.betaA, P.betaB);
  const float sc = 1.0f / (8.0f * M);
  float2* out = Hs + (size_t)d * M + t;
  if (!P.special)
    spectral_complement<RP, 1, float2>(x, twiddle<LOG2M + 1>(tw, uint32_t(P.kapA)), nullptr, T, out, sc);
  else
    spectral_selfmirror<RP, 1, float2>(x, twiddle<LOG2M + 1>(tw, uint32_t(P.kapB)), nullptr, T, out, sc);
}

// Engine-order spectrum -> H[d, k], k = 0..L (unscaled 2L-point DFT bins).
template <int LOG2M>
__global__ void k_export1d(const float2* __restrict__ Hs, float2* __restrict__ H) {
  using C = Single<LOG2M>;
  constexpr int M = C::M, T = C::T, RP = C::RP;
  const int d = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;   // slot * T + t
  if (idx >= M) return;
  const int slot = idx / T, t = idx % T;
  const float sc = 4.0f * M;
  const float2 v = Hs[(size_t)d * M + idx];
  float2* out = H + (size_t)d * (M + 1);
  const auto P = C::NP::of(t);
  if (P.special && slot == 0) {
    out[0] = make_float2(v.x * sc, 0.f);
    out[M] = make_float2(v.y * sc, 0.f);
    return;
  }
  const int k = slot < RP ? P.kapA + (M / RP) * slot : P.kapB + (M / RP) * (slot - RP);
  out[k] = cscale(v, sc);
}

// ------------------------------------------------------------------ host launchers
namespace {
template <int LOG2M, bool BF16, bool FULL>
void conv1d_launch_t(bool gate, const void* u, const ConvChain& ch, int order, void* y, int B, int D, int hsb,
                     const Twiddles& tw, hipStream_t s) {
  using E = typename Store<BF16>::elem;
  dim3 grid(B * D), block(Single<LOG2M>::T);
  if (gate)
    hipLaunchKernelGGL((k_conv1d<LOG2M, BF16, true, FULL>), grid, block, 0, s, (const E*)u, ch, order, (E*)y, B, D,
                       hsb, tw);
  else
    hipLaunchKernelGGL((k_conv1d<LOG2M, BF16, false, FULL>), grid, block, 0, s, (const E*)u, ch, order, (E*)y, B, D,
                       hsb, tw);
}
template <int LOG2M>
hipError_t conv1d_launch(int bf16, bool gate, bool full, const void* u, const ConvChain& ch, int order, void* y,
                         int B, int D, int hsb, const Twiddles& tw, hipStream_t s) {
  if (bf16)
    full ? conv1d_launch_t<LOG2M, true, true>(gate, u, ch, order, y, B, D, hsb, tw, s)
         : conv1d_launch_t<LOG2M, true, false>(gate, u, ch, order, y, B, D, hsb, tw, s);
  else
    full ? conv1d_launch_t<LOG2M, false, true>(gate, u, ch, order, y, B, D, hsb, tw, s)
         : conv1d_launch_t<LOG2M, false, false>(gate, u, ch, order, y, B, D, hsb, tw, s);
  return hipGetLastError();
}
template <int LOG2M>
hipError_t spectrum1d_launch(const float* h, float2* Hs, int D, bool full, const Twiddles& tw, hipStream_t s) {
  if (full)
    hipLaunchKernelGGL((k_spectrum1d<LOG2M, true>), dim3(D), dim3(Single<LOG2M>::T), 0, s, h, Hs, tw);
  else
    hipLaunchKernelGGL((k_spectrum1d<LOG2M, false>), dim3(D), dim3(Single<LOG2M>::T), 0, s, h, Hs, tw);
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

#define HYENA_SINGLE_CASES(X) X(10) X(11) X(12) X(13) X(14)

hipError_t launch_conv1d_chain(int log2L, int bf16, const void* u, const void* const* gates,
                               const float2* const* spectra, int order, void* y, int B, int D, const Twiddles& tw,
                               hipStream_t s, int full, int hsb) {
  if (order < 1 || order > kConvMaxChain) return hipErrorInvalidValue;
  ConvChain ch{};
  bool g = true;
  for (int i = 0; i < order; ++i) {
    ch.gate[i] = gates[i];
    ch.spectrum[i] = spectra[i];
    g = g && gates[i] != nullptr;
  }
  if (!g && order != 1) return hipErrorInvalidValue;   // only a single order may run without a gate
  switch (log2L) {
#define X(n) case n: return conv1d_launch<n>(bf16, g, full != 0, u, ch, order, y, B, D, hsb, tw, s);
    HYENA_SINGLE_CASES(X)
#undef X
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv1d_single(int log2L, int bf16, const void* u, const void* gate, void* y, const float2* Hs,
                                int B, int D, const Twiddles& tw, hipStream_t s, int full, int hsb) {
  const void* g[1] = {gate};
  const float2* h[1] = {Hs};
  return launch_conv1d_chain(log2L, bf16, u, g, h, 1, y, B, D, tw, s, full, hsb);
}

hipError_t launch_spectrum1d_single(int log2L, const float* h, float2* Hs, int D, const Twiddles& tw,
                                    hipStream_t s, int full) {
  switch (log2L) {
#define X(n) case n: return spectrum1d_launch<n>(h, Hs, D, full != 0, tw, s);
    HYENA_SINGLE_CASES(X)
#undef X
  }
  return hipErrorInvalidValue;
}

hipError_t launch_export1d_single(int log2L, const float2* Hs, float2* H, int D, hipStream_t s) {
  switch (log2L) {
#define X(n) case n: return export1d_launch<n>(Hs, H, D, s);
    HYENA_SINGLE_CASES(X)
#undef X
  }
  return hipErrorInvalidValue;
}

}  // namespace hyena
