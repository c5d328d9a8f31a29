// Implicit filter taps (Hyena study note, step 2: h(t) = FFN(pos_enc(t)) * w(t), w(t) = exp(-alpha t);
// listing ImplicitFilter: Linear(F -> hidden), SiLU, Linear(hidden -> D); EulerStack YAML
// filter_hidden = 64; HyenaND summary, method: a coordinate network on the grid offsets).
// Positions are normalised (t/L, r/n), so the same parameters serve any grid.
//
//   1-D: phi(t) = [sin(2 pi f t/L), f = 1..F/2] ++ [cos(2 pi f t/L), f = 1..F/2],   window exp(-alpha t/L)
//   3-D: per axis (x, y, z) [sin, cos](2 pi f r_a/n), f = 1..F/6, F/6 sines then F/6 cosines,
//        window exp(-alpha |r|/n); offsets r on [-(n-1), n-1]^3 (zero-padded grid) or the centred
//        period [-n/2, n/2)^3 (periodic grid)
//   g = W2 SiLU(W1 phi + b1) + b2,  W1 [H, F], W2 [D, H];  h[d, pos] = g_d(pos) * window_d(pos)
//
// Phases f t (f r) are reduced modulo L (n) in integers before the sine, so every angle is exact.
// A workgroup owns a tile of 64 positions x 128 channels: the hidden layer of its 64 positions is
// formed once (a 4 positions x 4 units register tile per thread), then the second layer runs as a
// small GEMM from LDS with a 4 x 8 register tile per thread; both read their operands as 16-byte
// LDS vectors.  W1 and the features, then W2 and the hidden activations, share one LDS region.
#include "launch.h"

namespace hyena {

namespace flt {
constexpr int TP = 64;     // positions per tile
constexpr int CB = 128;    // channels per tile
constexpr int T = 256;
}  // namespace flt

// 1-D positions t = 0..L-1
struct FilterGrid1D {
  int L;
  __device__ __forceinline__ int count() const { return L; }
  // feature pair q (frequency q + 1): sine at column q, cosine at column F/2 + q
  template <int F>
  __device__ __forceinline__ void pair(int pos, int q, int& col_s, int& col_c, float& s, float& c) const {
    const long long ph = ((long long)(q + 1) * pos) % L;
    sincospif(2.0f * (float)ph / (float)L, &s, &c);
    col_s = q;
    col_c = F / 2 + q;
  }
  __device__ __forceinline__ float window_arg(int pos) const { return (float)pos / (float)L; }
};

// 3-D offsets: W taps per axis, tap index i <-> offset i - R0, grid size n
struct FilterGrid3D {
  int W, R0, n;
  __device__ __forceinline__ int count() const { return W * W * W; }
  __device__ __forceinline__ int off(int pos, int ax) const {
    const int i = ax == 0 ? pos / (W * W) : (ax == 1 ? (pos / W) % W : pos % W);
    return i - R0;
  }
  template <int F>
  __device__ __forceinline__ void pair(int pos, int q, int& col_s, int& col_c, float& s, float& c) const {
    constexpr int PER = F / 6;
    const int ax = q / PER, k = q % PER;
    const int ph = (((k + 1) * off(pos, ax)) % n + n) % n;
    sincospif(2.0f * (float)ph / (float)n, &s, &c);
    col_s = ax * 2 * PER + k;
    col_c = ax * 2 * PER + PER + k;
  }
  __device__ __forceinline__ float window_arg(int pos) const {
    const float fx = (float)off(pos, 0) / n, fy = (float)off(pos, 1) / n, fz = (float)off(pos, 2) / n;
    return sqrtf(fx * fx + fy * fy + fz * fz);
  }
};

template <int F, int H, class G>
__global__ void __launch_bounds__(flt::T)
k_filter_tiles(FilterArgs a, G geo, float* __restrict__ h) {
  using namespace flt;
  static_assert(H == 64 && (TP * H) % T == 0, "tile shape");
  constexpr int PHASE1 = F * H + F * (TP + 4);          // w1t[F][H], phiT[F][TP+4]
  constexpr int PHASE2 = H * CB + H * (TP + 4);         // w2t[H][CB], actT[H][TP+4]
  __shared__ __align__(16) float lds[PHASE1 > PHASE2 ? PHASE1 : PHASE2];
  const int tid = threadIdx.x;
  const int npos = geo.count();
  const int p0 = blockIdx.x * TP, c0 = blockIdx.y * CB;

  // phase 1: W1 transposed and the features of the tile's positions (feature-major)
  float* w1t = lds;
  float* phiT = lds + F * H;
  for (int i = tid; i < F * H; i += T) {
    const int j = i / F, f = i % F;
    w1t[f * H + j] = a.W1[i];
  }
  for (int i = tid; i < TP * (F / 2); i += T) {
    const int p = i / (F / 2), q = i % (F / 2);
    const int pos = min(p0 + p, npos - 1);
    int cs, cc;
    float s, c;
    geo.template pair<F>(pos, q, cs, cc, s, c);
    phiT[cs * (TP + 4) + p] = s;
    phiT[cc * (TP + 4) + p] = c;
  }
  __syncthreads();
  // hidden layer: thread owns positions 4 hp .. 4 hp + 3 and units 4 hj .. 4 hj + 3
  const int hp = tid % (TP / 4), hj = tid / (TP / 4);
  float act[4][4];
  {
    const float bj[4] = {a.b1[4 * hj], a.b1[4 * hj + 1], a.b1[4 * hj + 2], a.b1[4 * hj + 3]};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) act[i][k] = bj[k];
#pragma unroll 4
    for (int f = 0; f < F; ++f) {
      const float4 pv = *reinterpret_cast<const float4*>(phiT + f * (TP + 4) + 4 * hp);
      const float4 wv = *reinterpret_cast<const float4*>(w1t + f * H + 4 * hj);
      const float x[4] = {pv.x, pv.y, pv.z, pv.w};
      const float y[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) act[i][k] = fmaf(x[i], y[k], act[i][k]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) act[i][k] = __fdividef(act[i][k], 1.0f + __expf(-act[i][k]));   // SiLU
  }
  __syncthreads();

  // phase 2: W2 block transposed (zero past D) and the activations, positions contiguous
  float* w2t = lds;
  float* actT = lds + H * CB;
  for (int i = tid; i < H * CB; i += T) {
    const int j = i / CB, c = i % CB;
    w2t[i] = (c0 + c < a.D) ? a.W2[(size_t)(c0 + c) * H + j] : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    *reinterpret_cast<float4*>(actT + (4 * hj + k) * (TP + 4) + 4 * hp) =
        make_float4(act[0][k], act[1][k], act[2][k], act[3][k]);
  __syncthreads();

  // second layer: positions 4 pg .. 4 pg + 3, channels 8 cg .. 8 cg + 7 of the tile
  const int pg = tid % (TP / 4), cg = tid / (TP / 4);
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[i][c] = 0.0f;
#pragma unroll 4
  for (int j = 0; j < H; ++j) {
    const float4 av = *reinterpret_cast<const float4*>(actT + j * (TP + 4) + 4 * pg);
    const float4 wa = *reinterpret_cast<const float4*>(w2t + j * CB + 8 * cg);
    const float4 wb = *reinterpret_cast<const float4*>(w2t + j * CB + 8 * cg + 4);
    const float x[4] = {av.x, av.y, av.z, av.w};
    const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[i][c] = fmaf(x[i], wv[c], acc[i][c]);
  }

  // bias and window; four consecutive positions per channel as one 16-byte store when in range
  const int pos0 = p0 + 4 * pg;
  float wa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wa[i] = geo.window_arg(min(pos0 + i, npos - 1));
  const bool full = pos0 + 3 < npos && (npos & 3) == 0 && (reinterpret_cast<uintptr_t>(h) & 15) == 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int d = c0 + 8 * cg + c;
    if (d >= a.D) break;
    const float b2 = a.b2[d], al = a.alpha[d];
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (acc[i][c] + b2) * __expf(-al * wa[i]);
    float* dst = h + (size_t)d * npos + pos0;
    if (full) {
      *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (pos0 + i < npos) dst[i] = v[i];
    }
  }
}

hipError_t launch_filter1d(const FilterArgs& a, int L, float* h, hipStream_t s) {
  if (a.F != 64 || a.H != 64 || L <= 0) return hipErrorInvalidValue;
  const dim3 grid((L + flt::TP - 1) / flt::TP, (a.D + flt::CB - 1) / flt::CB);
  hipLaunchKernelGGL((k_filter_tiles<64, 64, FilterGrid1D>), grid, dim3(flt::T), 0, s, a, FilterGrid1D{L}, h);
  return hipGetLastError();
}

// 3-D taps on the 64^3 grid: zero-padded offsets [-63, 63]^3 (W = 127) or the periodic centred period
// [-32, 31]^3 (W = 64); h[d, W, W, W] with tap index = offset + R0.
hipError_t launch_filter3d(const FilterArgs& a, float* h, hipStream_t s, int circ) {
  if (a.F != 96 || a.H != 64) return hipErrorInvalidValue;
  constexpr int n = 64;
  const FilterGrid3D geo = circ ? FilterGrid3D{n, n / 2, n} : FilterGrid3D{2 * n - 1, n - 1, n};
  const int np = geo.W * geo.W * geo.W;
  const dim3 grid((np + flt::TP - 1) / flt::TP, (a.D + flt::CB - 1) / flt::CB);
  hipLaunchKernelGGL((k_filter_tiles<96, 64, FilterGrid3D>), grid, dim3(flt::T), 0, s, a, geo, h);
  return hipGetLastError();
}

}  // namespace hyena
