// Streaming (token-by-token) evaluation of the causal operator with a prefix-spectrum cache: the
// decode-time counterpart of the whole-sequence kernels (SPECTRE digest, token mixer and generation
// support: a cache that plays the role of the KV cache, so that generating a token does not redo the
// transform of the whole prefix; Hyena study note, step 3 equation for what each token computes).
//
// For each (b, d) row and order i the causal sum at position t splits at the start T0 of t's block:
//
//   (h_i conv u_{i-1})[t] = F_i[t] + sum_{j=0..t-T0} h_i[j] u_{i-1}[t-j],
//   F_i[t] = sum_{s<T0} h_i[t-s] u_{i-1}[s],
//
// F_i is produced once per block by the FFT convolution of the whole stored prefix (the cached filter
// spectrum against the history row, zero past T0), and the in-block part is a direct sum of at most
// one block of taps.  Every term with j >= 1 reads history written by earlier tokens, so the sums of all
// orders are formed together and only the j = 0 terms chain the orders within the token:
//
//   u_i[t] = x_i[t] * (S_i + h_i[0] u_{i-1}[t]),   S_i = F_i[t] + sum_{j=1..t-T0} h_i[j] u_{i-1}[t-j].
//
// One wave per (b, d) row; its lanes split the in-block taps (consecutive j, so the tap and history
// reads are coalesced) and the partial sums are reduced across the wave.
#include "launch.h"

namespace hyena {

namespace {

struct DecodePtrs {
  const float* p[kDecodeMaxOrder];
};
struct DecodeTok {
  const void* p[kDecodeMaxOrder];
};

// one token value of row r: fp32, or bf16 widened exactly
template <bool BF16>
__device__ __forceinline__ float dec_load(const void* p, int r) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[r]);
  else return static_cast<const float*>(p)[r];
}

__device__ __forceinline__ float dec_wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// hist, fut: [N][rows][L] fp32 (history of u_{i-1}, prefix contributions); taps[i]: [D][L] fp32, or
// [rows][L] with per-sample filters.  With bf16 tokens only v_t, the gates and y_t are bf16: the
// intermediates u_i stay fp32, as in the whole-sequence operator.
template <int N, bool BF16>
__global__ void __launch_bounds__(256)
k_decode_step(const void* __restrict__ v_t, DecodeTok x_t, DecodePtrs taps, float* hist,
              const float* __restrict__ fut, void* __restrict__ y_t, int rows, int D, int L, int t, int t0,
              int per_sample) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;                                  // uniform per wave
  const int d = per_sample ? r : r % D;                   // tap row: one filter per channel, or per (b, d)
  const int n = t - t0;                                   // earlier positions of this block
  const size_t rowL = (size_t)r * L;
  const size_t plane = (size_t)rows * L;

  // everything the token needs besides the in-block history, requested before the sums
  float xg[N], h0[N], pre[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    xg[i] = dec_load<BF16>(x_t.p[i], r);
    h0[i] = taps.p[i][(size_t)d * L];
    pre[i] = t0 > 0 ? fut[i * plane + rowL + t] : 0.0f;
  }
  float u = dec_load<BF16>(v_t, r);

  float acc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = 0.0f;
#pragma unroll 4
  for (int j = 1 + lane; j <= n; j += 64) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      acc[i] = fmaf(taps.p[i][(size_t)d * L + j], hist[i * plane + rowL + (t - j)], acc[i]);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = dec_wave_sum(acc[i]) + pre[i];
  // the chain through the orders: u_0 = v, u_i = x_i (S_i + h_i[0] u_{i-1})
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (lane == 0) hist[i * plane + rowL + t] = u;        // u_{i-1}[t] joins order i's history
    u = xg[i] * fmaf(h0[i], u, acc[i]);
  }
  if (lane == 0) {
    if constexpr (BF16) static_cast<uint16_t*>(y_t)[r] = f32_to_bf16_rne(u);
    else static_cast<float*>(y_t)[r] = u;
  }
}

// Prompt (prefill) staging, one element of a row per thread, rows of L: position t < P takes the prompt
// value, t >= P is zero (the history past the last token is zero).  MODE 0: dst = v (the input of order
// 1).  MODE 1: c holds the convolution of order i over its history; dst = x_i * c (the input of order
// i + 1, fp32), or, with y (the last order), y[b, d, t < P] = x_N * c.
// a (v or x_i) and y: [rows][P] of the token type.
template <int MODE, bool BF16>
__global__ void __launch_bounds__(256)
k_decode_prefill(const void* __restrict__ a, const float* c, float* dst, void* __restrict__ y, int L, int P) {
  const int r = blockIdx.x;
  const int t = blockIdx.y * 256 + threadIdx.x;
  if (t >= L) return;
  const size_t at = (size_t)r * L + t;
  const size_t ap = (size_t)r * P + t;
  float u = 0.0f;
  if (t < P) {
    const float in = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(a)[ap]) : static_cast<const float*>(a)[ap];
    u = MODE == 0 ? in : in * c[at];
  }
  if (MODE == 1 && y) {
    if (t < P) {
      if constexpr (BF16) static_cast<uint16_t*>(y)[ap] = f32_to_bf16_rne(u);
      else static_cast<float*>(y)[ap] = u;
    }
    return;
  }
  dst[at] = u;
}

}  // namespace

hipError_t launch_decode_prefill(int mode, int bf16, const void* a, const float* c, float* dst, void* y, int rows,
                                 int L, int P, hipStream_t s) {
  const dim3 grid(rows, (L + 255) / 256), block(256);
  if (mode == 0) {
    if (bf16) hipLaunchKernelGGL((k_decode_prefill<0, true>), grid, block, 0, s, a, c, dst, y, L, P);
    else hipLaunchKernelGGL((k_decode_prefill<0, false>), grid, block, 0, s, a, c, dst, y, L, P);
  } else {
    if (bf16) hipLaunchKernelGGL((k_decode_prefill<1, true>), grid, block, 0, s, a, c, dst, y, L, P);
    else hipLaunchKernelGGL((k_decode_prefill<1, false>), grid, block, 0, s, a, c, dst, y, L, P);
  }
  return hipGetLastError();
}

hipError_t launch_decode_step(int order, int bf16, const void* v_t, const void* const* x_t,
                              const float* const* taps, float* hist, const float* fut, void* y_t, int rows, int D,
                              int L, int t, int t0, int per_sample, hipStream_t s) {
  DecodeTok xp{};
  DecodePtrs tp{};
  for (int i = 0; i < order; ++i) {
    xp.p[i] = x_t[i];
    tp.p[i] = taps[i];
  }
  const dim3 grid((rows + 3) / 4), block(256);
  switch (order) {
#define X(n)                                                                                                     \
  case n:                                                                                                        \
    if (bf16) hipLaunchKernelGGL((k_decode_step<n, true>), grid, block, 0, s, v_t, xp, tp, hist, fut, y_t, rows, D, L, \
                                 t, t0, per_sample);                                                                        \
    else hipLaunchKernelGGL((k_decode_step<n, false>), grid, block, 0, s, v_t, xp, tp, hist, fut, y_t, rows, D, L, \
                            t, t0, per_sample);                                                                            \
    break;
    X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8)
#undef X
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hyena
