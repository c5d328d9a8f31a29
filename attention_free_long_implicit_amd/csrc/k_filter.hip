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
// The input-dependent filters (one per sample) follow the same tiling; see k_film_tiles below.
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
  static constexpr int NC = 1;
  __device__ __forceinline__ void coords(int pos, float* c) const { c[0] = (float)pos / (float)L; }
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
  static constexpr int NC = 3;
  __device__ __forceinline__ void coords(int pos, float* c) const {
    for (int ax = 0; ax < 3; ++ax) c[ax] = (float)off(pos, ax) / n;
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

// ------------------------------------------------------------------ input-dependent (per-sample) filters
// HyenaND summary, method: R register tokens summarised per sample by a softmax-weighted mean z(x); z
// modulates (FiLM) a coordinate SIREN f(c; z); the kernel is K = w(c) f(c; z) with a Gaussian window w.
//   a[r] = softmax_r(q . reg[b, r]),  z = sum_r a[r] reg[b, r]
//   gamma_l = G_l z + g_l,  beta_l = P_l z + p_l                         (l = 1, 2; H values each)
//   h1 = sin(gamma_1 * omega0 * (A1 c + a1) + beta_1),  h2 = sin(gamma_2 * (A2 h1 + a2) + beta_2)
//   K[b, d, c] = (A3 h2 + a3)_d * exp(-|c|^2 / (2 sigma_d^2))
// Coordinates as for the exponential filter: c = t/L (1-D), c = r/n per axis (3-D offsets).

namespace {
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
}  // namespace

// One workgroup per sample: scores, softmax weights, z, then the four FiLM vectors
// mod[b] = {gamma_1, beta_1, gamma_2, beta_2} (H floats each).
__global__ void __launch_bounds__(256)
k_film_prep(FilmArgs a, const float* __restrict__ reg, int R, float* __restrict__ mod) {
  __shared__ float z[kFilmMaxE];
  __shared__ float wr[kFilmMaxR];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int E = a.E, H = a.H;
  const float* rb = reg + (size_t)b * R * E;
  for (int r = wv; r < R; r += 4) {
    float acc = 0.0f;
    for (int e = lane; e < E; e += 64) acc = fmaf(a.q[e], rb[(size_t)r * E + e], acc);
    acc = wave_sum(acc);
    if (lane == 0) wr[r] = acc;
  }
  __syncthreads();
  float m = -INFINITY;
  for (int r = 0; r < R; ++r) m = fmaxf(m, wr[r]);
  float sum = 0.0f;
  for (int r = 0; r < R; ++r) sum += expf(wr[r] - m);
  __syncthreads();
  for (int r = tid; r < R; r += 256) wr[r] = expf(wr[r] - m) / sum;
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    float acc = 0.0f;
    for (int r = 0; r < R; ++r) acc = fmaf(wr[r], rb[(size_t)r * E + e], acc);
    z[e] = acc;
  }
  __syncthreads();
  const float* Ms[4] = {a.G1, a.P1, a.G2, a.P2};
  const float* vs[4] = {a.g1, a.p1, a.g2, a.p2};
  for (int o = wv; o < 4 * H; o += 4) {
    const float* row = Ms[o / H] + (size_t)(o % H) * E;
    float acc = 0.0f;
    for (int e = lane; e < E; e += 64) acc = fmaf(row[e], z[e], acc);
    acc = wave_sum(acc);
    if (lane == 0) mod[(size_t)b * 4 * H + o] = acc + vs[o / H][o % H];
  }
}

// Taps of sample blockIdx.z: a tile of 64 positions x 128 channels per workgroup.  Layer 1 (NC inputs)
// is evaluated directly into LDS; layer 2 (H x H) and the read-out (H -> D) run as small GEMMs from LDS
// with 4 x 4 and 4 x 8 register tiles, as in the exponential filter's network.
template <int H, class G>
__global__ void __launch_bounds__(flt::T)
k_film_tiles(FilmArgs a, const float* __restrict__ mod, G geo, float* __restrict__ h) {
  using namespace flt;
  constexpr int NC = G::NC;
  static_assert(H == 64 && 4 * H == T, "tile shape");
  constexpr int PHASE1 = H * H + H * (TP + 4);          // a2t[H][H], h1T[H][TP+4]
  constexpr int PHASE2 = H * CB + H * (TP + 4);         // a3t[H][CB], h2T[H][TP+4]
  __shared__ __align__(16) float lds[PHASE1 > PHASE2 ? PHASE1 : PHASE2];
  __shared__ float gm[4 * H];                           // gamma_1, beta_1, gamma_2, beta_2
  __shared__ float crd[NC][TP];
  __shared__ float rsq[TP];
  const int tid = threadIdx.x;
  const int b = blockIdx.z;
  const int npos = geo.count();
  const int p0 = blockIdx.x * TP, c0 = blockIdx.y * CB;

  float* a2t = lds;
  float* h1T = lds + H * H;
  for (int i = tid; i < H * H; i += T) {
    const int j = i / H, k = i % H;
    a2t[k * H + j] = a.A2[i];
  }
  gm[tid] = mod[(size_t)b * 4 * H + tid];
  if (tid < TP) {
    float c[NC];
    geo.coords(min(p0 + tid, npos - 1), c);
    float r2 = 0.0f;
#pragma unroll
    for (int ax = 0; ax < NC; ++ax) {
      crd[ax][tid] = c[ax];
      r2 = fmaf(c[ax], c[ax], r2);
    }
    rsq[tid] = r2;
  }
  __syncthreads();
  // layer 1: unit k of position p, positions fastest
  for (int i = tid; i < TP * H; i += T) {
    const int k = i / TP, p = i % TP;
    float s = a.a1[k];
#pragma unroll
    for (int ax = 0; ax < NC; ++ax) s = fmaf(a.A1[k * NC + ax], crd[ax][p], s);
    h1T[k * (TP + 4) + p] = sinf(fmaf(gm[k], a.omega0[k] * s, gm[H + k]));
  }
  __syncthreads();
  // layer 2: positions 4 hp .. 4 hp + 3, units 4 hj .. 4 hj + 3
  const int hp = tid % (TP / 4), hj = tid / (TP / 4);
  float act[4][4];
  {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float bj = a.a2[4 * hj + k];
#pragma unroll
      for (int i = 0; i < 4; ++i) act[i][k] = bj;
    }
#pragma unroll 4
    for (int k = 0; k < H; ++k) {
      const float4 pv = *reinterpret_cast<const float4*>(h1T + k * (TP + 4) + 4 * hp);
      const float4 wv = *reinterpret_cast<const float4*>(a2t + k * H + 4 * hj);
      const float x[4] = {pv.x, pv.y, pv.z, pv.w};
      const float y[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) act[i][c] = fmaf(x[i], y[c], act[i][c]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float g2 = gm[2 * H + 4 * hj + k], b2 = gm[3 * H + 4 * hj + k];
#pragma unroll
      for (int i = 0; i < 4; ++i) act[i][k] = sinf(fmaf(g2, act[i][k], b2));
    }
  }
  __syncthreads();

  // read-out: A3 block transposed (zero past D) and the layer-2 activations, positions contiguous
  float* a3t = lds;
  float* h2T = lds + H * CB;
  for (int i = tid; i < H * CB; i += T) {
    const int k = i / CB, c = i % CB;
    a3t[i] = (c0 + c < a.D) ? a.A3[(size_t)(c0 + c) * H + k] : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    *reinterpret_cast<float4*>(h2T + (4 * hj + k) * (TP + 4) + 4 * hp) =
        make_float4(act[0][k], act[1][k], act[2][k], act[3][k]);
  __syncthreads();

  const int pg = tid % (TP / 4), cg = tid / (TP / 4);
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[i][c] = 0.0f;
#pragma unroll 4
  for (int k = 0; k < H; ++k) {
    const float4 av = *reinterpret_cast<const float4*>(h2T + k * (TP + 4) + 4 * pg);
    const float4 wa = *reinterpret_cast<const float4*>(a3t + k * CB + 8 * cg);
    const float4 wb = *reinterpret_cast<const float4*>(a3t + k * CB + 8 * cg + 4);
    const float x[4] = {av.x, av.y, av.z, av.w};
    const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[i][c] = fmaf(x[i], wv[c], acc[i][c]);
  }

  const int pos0 = p0 + 4 * pg;
  float* hb = h + (size_t)b * a.D * npos;
  const bool full = pos0 + 3 < npos && (npos & 3) == 0 && (reinterpret_cast<uintptr_t>(h) & 15) == 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int d = c0 + 8 * cg + c;
    if (d >= a.D) break;
    const float a3 = a.a3[d], sg = a.sigma[d];
    const float k2 = -0.5f / (sg * sg);
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (acc[i][c] + a3) * expf(k2 * rsq[4 * pg + i]);
    float* dst = hb + (size_t)d * npos + pos0;
    if (full) {
      *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (pos0 + i < npos) dst[i] = v[i];
    }
  }
}

hipError_t launch_film_prep(const FilmArgs& a, const float* reg, int B, int R, float* mod, hipStream_t s) {
  if (a.H != 64 || a.E < 1 || a.E > kFilmMaxE || R < 1 || R > kFilmMaxR || B < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_film_prep, dim3(B), dim3(256), 0, s, a, reg, R, mod);
  return hipGetLastError();
}

hipError_t launch_film_filter1d(const FilmArgs& a, const float* mod, int B, int L, float* h, hipStream_t s) {
  if (a.H != 64 || a.NC != 1 || L <= 0 || B < 1) return hipErrorInvalidValue;
  const dim3 grid((L + flt::TP - 1) / flt::TP, (a.D + flt::CB - 1) / flt::CB, B);
  hipLaunchKernelGGL((k_film_tiles<64, FilterGrid1D>), grid, dim3(flt::T), 0, s, a, mod, FilterGrid1D{L}, h);
  return hipGetLastError();
}

hipError_t launch_film_filter3d(const FilmArgs& a, const float* mod, int B, float* h, hipStream_t s, int circ) {
  if (a.H != 64 || a.NC != 3 || B < 1) return hipErrorInvalidValue;
  constexpr int n = 64;
  const FilterGrid3D geo = circ ? FilterGrid3D{n, n / 2, n} : FilterGrid3D{2 * n - 1, n - 1, n};
  const int np = geo.W * geo.W * geo.W;
  const dim3 grid((np + flt::TP - 1) / flt::TP, (a.D + flt::CB - 1) / flt::CB, B);
  hipLaunchKernelGGL((k_film_tiles<64, FilterGrid3D>), grid, dim3(flt::T), 0, s, a, mod, geo, h);
  return hipGetLastError();
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
