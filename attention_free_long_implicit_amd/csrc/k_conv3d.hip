// 3-D non-causal ("same") long convolution on a 64^3 grid, zero-padded to 128^3 (HyenaND summary,
// method: native N-D convolution evaluated by an N-D FFT; boundary handling: zero-pad to twice the
// size so nothing wraps), with the Hyena gate (Hyena study note, step 3).
//
//   c[p] = sum_{q in [0,64)^3} h[p-q] u[q],  p in [0,64)^3,  h on offsets [-63, 63]^3 placed at r mod 128
//
// Layout of the transform: every z-line (128 reals, upper half zero) is packed two samples per
// complex value and transformed with 64 points, then split into its 65 real-transform bins; y and x
// are complex 128-point transforms.  Passes (per (b, d) volume):
//   A  k3_planes  one x-slab: z-transform + split + y-transform in an LDS plane [128 y][65 kz]
//   B  k3_cols    64 (y, kz) columns: x-transform, product with the filter spectrum, inverse, keep x < 64
//   C  k3_planes  one x-slab: inverse y (keep y < 64), re-pack, inverse z (keep z < 64), gate; for every
//                 order but the last, the same workgroup then runs the next order's pass A
// Intermediate per volume: [64 x][128 y-position][65 kz] complex fp32 (4.26 MB), processed in chunks.
// Filter spectrum per channel: Hs[tile][x-position][64 columns], 130 tiles, Hs = H / 2^22 where H is
// the 128^3 real-input DFT of the placed filter.
#include "engine.h"
#include "launch.h"

namespace hyena {

namespace k3 {
constexpr int N = 64;              // grid points per axis
constexpr int MP = 128;            // padded length per axis
constexpr int NZC = 64;            // packed complex points per z-line
constexpr int NKZ = 65;            // real-transform bins per z-line
constexpr int PLANE = MP * NKZ;    // 8320 complex per x-slab
constexpr int COLS = 64;           // columns per pass-B workgroup
constexpr int TILES = PLANE / COLS;  // 130
constexpr int T = 512;
using ZRL = Radices<8, 8>;
using YRL = Radices<16, 8>;
using XRL = Radices<16, 8>;
template <int NL>
using ZEng = ColEngine<NL, 1, NKZ, T, ZRL, false>;       // lines = y, positions = packed z
using YEng = ColEngine<NKZ, NKZ, 1, T, YRL, false>;      // lines = kz, positions = y
using XEng = ColEngine<COLS, COLS, 1, T, XRL, true>;     // lines = columns, positions = x
constexpr float kSpecScale = 1.0f / 8388608.0f;          // 2^-23 (the split contributes a factor 2)
}  // namespace k3

// z-line split / re-pack on the plane.  Split: Z (digit-reversed positions 0..63 of each line) ->
// 2 X[kz] at natural columns 0..64.  Re-pack: Y at natural columns 0..64 -> Z'' at digit-reversed
// positions 0..63.  All reads happen before the barrier, all writes after.
template <int NLINES, bool SPLIT>
__device__ __forceinline__ void k3_zline_pairs(float2* plane, const Twiddles& tw, int t) {
  using namespace k3;
  constexpr int ITEMS = NLINES * 33;
  constexpr int PER = (ITEMS + T - 1) / T;
  float2 a[PER], b[PER];
  static_for<PER>([&](auto ii) {
    const int it = t + T * ii.value;
    if (it >= ITEMS) return;
    const int y = it / 33, k = it % 33;
    const int kp = (NZC - k) % NZC;
    float2* line = plane + y * NKZ;
    const float2 w = twiddle<7>(tw, uint32_t(k));
    if constexpr (SPLIT) {
      const float2 A = line[ZRL::position_of_bin(k)];
      const float2 B = line[ZRL::position_of_bin(kp)];
      split_pair(A, B, w, a[ii.value], b[ii.value]);
    } else {
      const float2 Yk = line[k];
      const float2 Yp = line[NZC - k];
      const float2 Ye = cadd(Yk, cconj(Yp));
      const float2 Yo = cmulc(csub(Yk, cconj(Yp)), w);
      a[ii.value] = make_float2(Ye.x - Yo.y, Ye.y + Yo.x);
      b[ii.value] = make_float2(Ye.x + Yo.y, Yo.x - Ye.y);
    }
  });
  __syncthreads();
  static_for<PER>([&](auto ii) {
    const int it = t + T * ii.value;
    if (it >= ITEMS) return;
    const int y = it / 33, k = it % 33;
    float2* line = plane + y * NKZ;
    if constexpr (SPLIT) {
      line[k] = a[ii.value];
      if (k != 0 && k != 32) line[NZC - k] = b[ii.value];
      if (k == 0) line[NZC] = b[ii.value];
    } else {
      line[ZRL::position_of_bin(k)] = a[ii.value];
      if (k != 0 && k != 32) line[ZRL::position_of_bin(NZC - k)] = b[ii.value];
    }
  });
  __syncthreads();
}

// forward half of pass A on a plane whose packed z-lines are in place (lines y < NLINES nonzero)
template <int NLINES>
__device__ __forceinline__ void k3_plane_forward(float2* plane, const Twiddles& tw, int t) {
  using namespace k3;
  constexpr bool HALF = NLINES == N;      // activation slabs: y >= 64 and z >= 64 are zero
  ZEng<NLINES>::template forward<HALF>(plane, tw, t);
  k3_zline_pairs<NLINES, true>(plane, tw, t);
  YEng::template forward<HALF>(plane, tw, t);
}

// Pass A (MODE 0, from activations) or pass C (MODE 1, inverse + gate [+ chained pass A]).
// grid.x = 64 slabs * nq (volume fastest).
template <bool BF16, int MODE, bool GATE, bool CHAIN>
__global__ void __launch_bounds__(k3::T)
k3_planes(const typename Store<BF16>::elem* u, const typename Store<BF16>::elem* gate,
          typename Store<BF16>::elem* y, float2* I, int q0, int nq, int B, int D, Twiddles tw) {
  using namespace k3;
  using St = Store<BF16>;
  __shared__ float2 plane[PLANE];
  const int t = threadIdx.x;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ql = lb % nq, x = lb / nq;
  const int q = q0 + ql;
  const int d = q / B, b = q % B;
  const size_t vol = ((size_t)b * D + d) * (size_t)(N * N * N);
  float2* slab = I + ((size_t)ql * N + x) * PLANE;
  if constexpr (MODE == 0) {
    const auto* src = u + vol + (size_t)x * N * N;
    static_for<(N * NZC / 2) / T>([&](auto ii) {
      const int e = t + T * ii.value;
      const int yy = e / (NZC / 2), m = e % (NZC / 2);
      plane[yy * NKZ + m] = St::load2(src + yy * N + 2 * m);
    });
    __syncthreads();
  } else {
    for (int j = t; j < PLANE; j += T) plane[j] = slab[j];
    __syncthreads();
    YEng::template inverse<true>(plane, tw, t);
    k3_zline_pairs<N, false>(plane, tw, t);
    ZEng<N>::template inverse<true>(plane, tw, t);
    const auto* g = GATE ? gate + vol + (size_t)x * N * N : nullptr;
    auto* dst = CHAIN ? nullptr : y + vol + (size_t)x * N * N;
    static_for<(N * NZC / 2) / T>([&](auto ii) {
      const int e = t + T * ii.value;
      const int yy = e / (NZC / 2), m = e % (NZC / 2);
      float2 v = plane[yy * NKZ + m];
      if constexpr (GATE) {
        const float2 gv = St::load2(g + yy * N + 2 * m);
        v = make_float2(v.x * gv.x, v.y * gv.y);
      }
      if constexpr (CHAIN) {
        if constexpr (BF16) v = make_float2(bf16_to_f32(f32_to_bf16_rne(v.x)), bf16_to_f32(f32_to_bf16_rne(v.y)));
        plane[yy * NKZ + m] = v;
      } else {
        St::store2(dst + yy * N + 2 * m, v);
      }
    });
    if constexpr (!CHAIN) return;
    __syncthreads();
  }
  k3_plane_forward<N>(plane, tw, t);
  for (int j = t; j < PLANE; j += T) slab[j] = plane[j];
}

// Pass A for the filter: taps h[d, 127, 127, 127] (offset + 63) placed at r mod 128; all 128 slabs.
__global__ void __launch_bounds__(k3::T)
k3_planes_taps(const float* __restrict__ h, float2* I, int q0, int nq, Twiddles tw) {
  using namespace k3;
  constexpr int W = 2 * N - 1;     // 127
  __shared__ float2 plane[PLANE];
  const int t = threadIdx.x;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ql = lb % nq, x = lb / nq;
  const int d = q0 + ql;
  const float* hd = h + (size_t)d * W * W * W;
  auto off = [](int i) { return i < N ? i : i - MP; };    // index on the 128-torus -> signed offset
  const int rx = off(x);
  static_for<(MP * NZC) / T>([&](auto ii) {
    const int e = t + T * ii.value;
    const int yy = e / NZC, m = e % NZC;
    const int ry = off(yy);
    float2 v = make_float2(0.f, 0.f);
    if (x != N && yy != N) {
      const float* line = hd + ((size_t)(rx + N - 1) * W + (ry + N - 1)) * W;
      const int z0 = 2 * m, z1 = 2 * m + 1;
      if (z0 != N) v.x = line[off(z0) + N - 1];
      if (z1 != N) v.y = line[off(z1) + N - 1];
    }
    plane[yy * NKZ + m] = v;
  });
  __syncthreads();
  k3_plane_forward<MP>(plane, tw, t);
  float2* slab = I + ((size_t)ql * MP + x) * PLANE;
  for (int j = t; j < PLANE; j += T) slab[j] = plane[j];
}

// Pass B.  MODE 0: x-transform (x >= 64 zero), product with Hs, inverse, keep x < 64 (in place).
//          MODE 1: x-transform of a full filter slab stack, write the scaled spectrum.
// grid.x = 130 tiles * nq (volume fastest).
template <int MODE>
__global__ void __launch_bounds__(k3::T)
k3_cols(float2* I, const float2* __restrict__ Hs, float2* __restrict__ Hs_out, int q0, int nq, int B, Twiddles tw) {
  using namespace k3;
  constexpr int NX = (MODE == 0) ? N : MP;    // slabs present in the intermediate
  __shared__ float2 lds[lds_padded_size(COLS * MP)];
  const int t = threadIdx.x;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ql = lb % nq, tile = lb / nq;
  const int q = q0 + ql;
  const int d = (MODE == 0) ? q / B : q;
  const int j0 = tile * COLS;
  float2* base = I + (size_t)ql * NX * PLANE + j0;
  static_for<(NX * COLS) / T>([&](auto ii) {
    const int e = t + T * ii.value;
    const int xx = e / COLS, l = e % COLS;
    lds[XEng::addr(xx, l)] = base[(size_t)xx * PLANE + l];
  });
  __syncthreads();
  XEng::template forward<MODE == 0>(lds, tw, t);
  const size_t hoff = ((size_t)d * TILES + tile) * (MP * COLS);
  if constexpr (MODE == 1) {
    static_for<(MP * COLS) / T>([&](auto ii) {
      const int e = t + T * ii.value;
      const int p = e / COLS, l = e % COLS;
      Hs_out[hoff + e] = cscale(lds[XEng::addr(p, l)], kSpecScale);
    });
    return;
  }
  static_for<(MP * COLS) / T>([&](auto ii) {
    const int e = t + T * ii.value;
    const int p = e / COLS, l = e % COLS;
    const int a = XEng::addr(p, l);
    lds[a] = cmul(lds[a], Hs[hoff + e]);
  });
  __syncthreads();
  XEng::template inverse<true>(lds, tw, t);
  static_for<(N * COLS) / T>([&](auto ii) {
    const int e = t + T * ii.value;
    const int xx = e / COLS, l = e % COLS;
    base[(size_t)xx * PLANE + l] = lds[XEng::addr(xx, l)];
  });
}

// Engine-order spectrum -> H[d, kx, ky, kz] (128 x 128 x 65, unscaled real-input DFT bins).
__global__ void k3_export(const float2* __restrict__ Hs, float2* __restrict__ H) {
  using namespace k3;
  const int d = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= TILES * MP * COLS) return;
  const int tile = idx / (MP * COLS), rem = idx % (MP * COLS);
  const int p = rem / COLS, l = rem % COLS;
  const int j = tile * COLS + l;
  const int ypos = j / NKZ, kz = j % NKZ;
  const int kx = XRL::bin_of_position(p), ky = YRL::bin_of_position(ypos);
  H[(((size_t)d * MP + kx) * MP + ky) * NKZ + kz] = cscale(Hs[(size_t)d * TILES * MP * COLS + idx], 4194304.0f);
}

// ------------------------------------------------------------------ 3-D filter taps
// h[d, rx, ry, rz] = (W2 SiLU(W1 phi(r) + b1) + b2)_d * exp(-alpha_d |r| / n) on offsets [-(n-1), n-1]^3;
// phi(r): per axis (x, y, z) 16 sines then 16 cosines of 2 pi f r_a / n, f = 1..16 (phases reduced mod n).
template <int F, int H>
__global__ void __launch_bounds__(256)
k_filter3d(FilterArgs a, float* __restrict__ h) {
  using namespace k3;
  constexpr int W = 2 * N - 1, NP = W * W * W, TP = 64, PER_AX = F / 6;
  __shared__ float phi[TP][F + 1];
  __shared__ float w1t[F][H + 1];
  __shared__ float act[TP][H + 1];
  __shared__ float rad[TP];
  const int tid = threadIdx.x;
  const int p0 = blockIdx.x * TP;
  for (int i = tid; i < F * H; i += 256) {
    const int j = i / F, f = i % F;
    w1t[f][j] = a.W1[i];
  }
  for (int i = tid; i < TP * 3 * PER_AX; i += 256) {
    const int pp = i / (3 * PER_AX), rem = i % (3 * PER_AX);
    const int ax = rem / PER_AX, f = rem % PER_AX;
    const int pos = min(p0 + pp, NP - 1);
    const int r3[3] = {pos / (W * W) - (N - 1), (pos / W) % W - (N - 1), pos % W - (N - 1)};
    const int ph = (((f + 1) * r3[ax]) % N + N) % N;
    float s, c;
    sincospif(2.0f * (float)ph / (float)N, &s, &c);
    phi[pp][ax * 2 * PER_AX + f] = s;
    phi[pp][ax * 2 * PER_AX + PER_AX + f] = c;
    if (ax == 0 && f == 0) {
      const float fx = (float)r3[0] / N, fy = (float)r3[1] / N, fz = (float)r3[2] / N;
      rad[pp] = sqrtf(fx * fx + fy * fy + fz * fz);
    }
  }
  __syncthreads();
  for (int i = tid; i < TP * H; i += 256) {
    const int pp = i / H, j = i % H;
    float z = a.b1[j];
#pragma unroll 8
    for (int f = 0; f < F; ++f) z = fmaf(w1t[f][j], phi[pp][f], z);
    act[pp][j] = z / (1.0f + expf(-z));
  }
  __syncthreads();
  const int pp = tid % TP, wv = tid / TP;
  float av[H];
#pragma unroll
  for (int j = 0; j < H; ++j) av[j] = act[pp][j];
  const int pos = p0 + pp;
  if (pos >= NP) return;
  const float rr = rad[pp];
  for (int dd = wv; dd < a.D; dd += 4) {
    const float* w2 = a.W2 + (size_t)dd * H;
    float g = a.b2[dd];
#pragma unroll
    for (int j = 0; j < H; ++j) g = fmaf(w2[j], av[j], g);
    h[(size_t)dd * NP + pos] = g * expf(-a.alpha[dd] * rr);
  }
}

// ------------------------------------------------------------------ host side
bool grid3d_supported(int64_t nx, int64_t ny, int64_t nz) { return nx == k3::N && ny == k3::N && nz == k3::N; }
size_t conv3d_volume_bytes() { return (size_t)k3::N * k3::PLANE * sizeof(float2); }
size_t conv3d_filter_volume_bytes() { return (size_t)k3::MP * k3::PLANE * sizeof(float2); }
size_t conv3d_spectrum_bytes_per_channel() { return (size_t)k3::TILES * k3::MP * k3::COLS * sizeof(float2); }
size_t conv3d_taps_per_channel() { return (size_t)(2 * k3::N - 1) * (2 * k3::N - 1) * (2 * k3::N - 1); }

namespace {
template <bool BF16>
hipError_t conv3d_launch_t(int order, int B, int D, const void* v, const void* const* x, const void* const* spectra,
                           void* y, float2* I, int chunk, const Twiddles& tw, hipStream_t s) {
  using namespace k3;
  using E = typename Store<BF16>::elem;
  const int rows = B * D;
  for (int q0 = 0; q0 < rows; q0 += chunk) {
    const int nq = (rows - q0 < chunk) ? rows - q0 : chunk;
    hipLaunchKernelGGL((k3_planes<BF16, 0, false, false>), dim3(N * nq), dim3(T), 0, s, (const E*)v,
                       (const E*)nullptr, (E*)nullptr, I, q0, nq, B, D, tw);
    for (int i = 0; i < order; ++i) {
      hipLaunchKernelGGL((k3_cols<0>), dim3(TILES * nq), dim3(T), 0, s, I, (const float2*)spectra[i],
                         (float2*)nullptr, q0, nq, B, tw);
      if (i + 1 < order)
        hipLaunchKernelGGL((k3_planes<BF16, 1, true, true>), dim3(N * nq), dim3(T), 0, s, (const E*)nullptr,
                           (const E*)x[i], (E*)nullptr, I, q0, nq, B, D, tw);
      else if (x[i])
        hipLaunchKernelGGL((k3_planes<BF16, 1, true, false>), dim3(N * nq), dim3(T), 0, s, (const E*)nullptr,
                           (const E*)x[i], (E*)y, I, q0, nq, B, D, tw);
      else
        hipLaunchKernelGGL((k3_planes<BF16, 1, false, false>), dim3(N * nq), dim3(T), 0, s, (const E*)nullptr,
                           (const E*)nullptr, (E*)y, I, q0, nq, B, D, tw);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
}  // namespace

hipError_t launch_conv3d(int bf16, int order, int B, int D, const void* v, const void* const* x,
                         const void* const* spectra, void* y, float2* I, int chunk, const Twiddles& tw, hipStream_t s) {
  return bf16 ? conv3d_launch_t<true>(order, B, D, v, x, spectra, y, I, chunk, tw, s)
              : conv3d_launch_t<false>(order, B, D, v, x, spectra, y, I, chunk, tw, s);
}

hipError_t launch_filter3d(const FilterArgs& a, float* h, hipStream_t s) {
  if (a.F != 96 || a.H != 64) return hipErrorInvalidValue;
  const int np = (int)conv3d_taps_per_channel();
  hipLaunchKernelGGL((k_filter3d<96, 64>), dim3((np + 63) / 64), dim3(256), 0, s, a, h);
  return hipGetLastError();
}

hipError_t launch_spectrum3d(const float* h, float2* Hs, int D, float2* I, int chunk, const Twiddles& tw,
                             hipStream_t s) {
  using namespace k3;
  for (int q0 = 0; q0 < D; q0 += chunk) {
    const int nq = (D - q0 < chunk) ? D - q0 : chunk;
    hipLaunchKernelGGL(k3_planes_taps, dim3(MP * nq), dim3(T), 0, s, h, I, q0, nq, tw);
    hipLaunchKernelGGL((k3_cols<1>), dim3(TILES * nq), dim3(T), 0, s, I, (const float2*)nullptr, Hs, q0, nq, 1,
                       tw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_export3d(const float2* Hs, float2* H, int D, hipStream_t s) {
  using namespace k3;
  const int n = TILES * MP * COLS;
  hipLaunchKernelGGL(k3_export, dim3((n + 255) / 256, D), dim3(256), 0, s, Hs, H);
  return hipGetLastError();
}

}  // namespace hyena
