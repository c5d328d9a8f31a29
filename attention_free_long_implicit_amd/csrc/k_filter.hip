// Implicit filter taps (Hyena study note, step 2: h(t) = FFN(pos_enc(t)) * w(t), w(t) = exp(-alpha t);
// listing ImplicitFilter: Linear(F -> hidden), SiLU, Linear(hidden -> D); EulerStack YAML
// filter_hidden = 64).  Positions are normalised, t/L, so the same parameters serve any length.
//
//   phi(t) = [sin(2 pi f t/L), f = 1..F/2] ++ [cos(2 pi f t/L), f = 1..F/2]
//   g(t)   = W2 SiLU(W1 phi(t) + b1) + b2            W1 [H, F], W2 [D, H]
//   h[d,t] = g_d(t) exp(-alpha_d t / L)
//
// The phase f t is reduced modulo L in integers before the sine, so every angle is exact.
// One workgroup computes a tile of 64 positions for all D channels.
#include "launch.h"

namespace hyena {

template <int F, int H>
__global__ void __launch_bounds__(256)
k_filter1d(FilterArgs a, int L, float* __restrict__ h) {
  constexpr int TP = 64;
  __shared__ float phi[TP][F + 1];
  __shared__ float w1t[F][H + 1];
  __shared__ float act[TP][H + 1];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TP;
  for (int i = tid; i < F * H; i += 256) {
    const int j = i / F, f = i % F;
    w1t[f][j] = a.W1[i];
  }
  for (int i = tid; i < TP * (F / 2); i += 256) {
    const int p = i / (F / 2), f = i % (F / 2);
    const int t = t0 + p;
    const long long ph = ((long long)(f + 1) * t) % L;
    float s, c;
    sincospif(2.0f * (float)ph / (float)L, &s, &c);
    phi[p][f] = s;
    phi[p][F / 2 + f] = c;
  }
  __syncthreads();
  for (int i = tid; i < TP * H; i += 256) {
    const int p = i / H, j = i % H;
    float z = a.b1[j];
#pragma unroll 8
    for (int f = 0; f < F; ++f) z = fmaf(w1t[f][j], phi[p][f], z);
    act[p][j] = z / (1.0f + expf(-z));
  }
  __syncthreads();
  const int p = tid % TP, wv = tid / TP;
  float av[H];
#pragma unroll
  for (int j = 0; j < H; ++j) av[j] = act[p][j];
  const int t = t0 + p;
  const float tn = (float)t / (float)L;
  for (int d = wv; d < a.D; d += 4) {
    const float* w2 = a.W2 + (size_t)d * H;
    float g = a.b2[d];
#pragma unroll
    for (int j = 0; j < H; ++j) g = fmaf(w2[j], av[j], g);
    h[(size_t)d * L + t] = g * expf(-a.alpha[d] * tn);
  }
}

hipError_t launch_filter1d(const FilterArgs& a, int L, float* h, hipStream_t s) {
  if (a.F != 64 || a.H != 64 || L % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_filter1d<64, 64>), dim3(L / 64), dim3(256), 0, s, a, L, h);
  return hipGetLastError();
}

}  // namespace hyena
