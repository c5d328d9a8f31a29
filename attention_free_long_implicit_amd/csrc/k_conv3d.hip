// 3-D non-causal long convolution on a 64^3 grid (HyenaND summary, method: native N-D convolution
// evaluated by an N-D FFT; boundary handling), with the Hyena gate (Hyena study note, step 3), for two
// boundaries (template geometry G):
//
//   zero-padded "same" (Geo3<false>): c[p] = sum_{q in [0,64)^3} h[p-q] u[q], p in [0,64)^3, h on
//     offsets [-63, 63]^3 placed at r mod 128, transforms on the 128^3 grid (padding to twice the size
//     so nothing wraps);
//   periodic (Geo3<true>): c[p] = sum_q h[(p-q) mod 64] u[q], h on the centred offsets [-32, 31]^3
//     placed at r mod 64, transforms on the 64^3 grid itself (circular convolution for periodic
//     systems).
//
// Two plans.  The periodic geometry (64^3 transform, nothing padded) runs passes A-C below; the
// zero-padded geometry runs passes Z, XY, Z' (further down), which store the volume after its z
// transform only and pad x and y on chip.
//
// Passes A-C (periodic geometry).  Every z-line is packed two samples per complex value and transformed
// with 32 points, then split into its 33 real-transform bins; y and x are complex 64-point transforms.
// Per (b, d) volume:
//   A  k3_planes  one x-slab: z-transform + split + y-transform in an LDS plane [64 y][33 kz]
//   B  k3_cols    64 (y, kz) columns: x-transform, product with the filter spectrum, inverse
//   C  k3_planes  one x-slab: inverse y, re-pack, inverse z, gate; for every order but the last, the same
//                 workgroup then runs the next order's pass A
// Intermediate per volume: [64 x][64 y][33 kz] complex fp32 (1.08 MB), processed in chunks.  Filter
// spectrum per channel: Hs[tile][x-position][64 columns], 33 tiles, Hs = H / 2^19 where H is the 64^3
// real-input DFT of the placed filter.
#include "engine.h"
#include "launch.h"

namespace hyena {

namespace k3 {
constexpr int N = 64;              // grid points per axis
constexpr int T = 512;
constexpr int COLS = 64;           // columns per pass-B workgroup
}  // namespace k3

template <bool CIRC> struct Geo3;
template <> struct Geo3<false> {   // zero-padded to 128^3
  static constexpr bool PAD = true;
  static constexpr int MP = 128;   // transform length per axis
  using ZRL = Radices<8, 8>;       // 64 packed points per z-line
  using YRL = Radices<16, 8>;
  using XRL = Radices<16, 8>;
};
template <> struct Geo3<true> {    // periodic, 64^3
  static constexpr bool PAD = false;
  static constexpr int MP = 64;
  using ZRL = Radices<8, 4>;       // 32 packed points per z-line
  using YRL = Radices<8, 8>;
  using XRL = Radices<8, 8>;
};

template <class G>
struct K3 {
  static constexpr int N = k3::N, T = k3::T, COLS = k3::COLS, MP = G::MP;
  static constexpr bool PAD = G::PAD;
  static constexpr int NZC = MP / 2;            // packed complex points per z-line
  static constexpr int NKZ = NZC + 1;           // real-transform bins per z-line
  static constexpr int PLANE = MP * NKZ;        // complex per x-slab
  static constexpr int TILES = PLANE / COLS;
  static constexpr int NZIN = PAD ? NZC / 2 : NZC;   // packed z values of the activations per line
  static_assert(PLANE % COLS == 0, "tiles");
  using ZRL = typename G::ZRL;
  using YRL = typename G::YRL;
  using XRL = typename G::XRL;
  static_assert(ZRL::S == NZC && YRL::S == MP && XRL::S == MP, "plans");
  template <int NL>
  using ZEng = ColEngine<NL, 1, NKZ, T, ZRL, false>;       // lines = y, positions = packed z
  using YEng = ColEngine<NKZ, NKZ, 1, T, YRL, false>;      // lines = kz, positions = y
  // lines = columns, positions = x; unpadded: a wave's 64 lanes always touch the 64 consecutive
  // columns of one position, which fill the banks exactly (a padded row spilled one bank pair over)
  using XEng = ColEngine<COLS, COLS, 1, T, XRL, false>;
  // Hs = H / (2 MP^3); the filter's own z split contributes a factor 2 (2^-23 for 128^3, 2^-20 for 64^3)
  static constexpr float kSpecScale = 1.0f / (4.0f * MP * MP * MP);
  // signed offset of transform index i on the MP-torus, and whether the filter holds it
  __device__ __forceinline__ static int offset(int i) { return PAD ? (i < N ? i : i - MP) : (i < MP / 2 ? i : i - MP); }
  __device__ __forceinline__ static bool in_filter(int i) { return !PAD || i != N; }
  // filter taps per axis and the tap index of a signed offset
  static constexpr int W = PAD ? 2 * N - 1 : N;
  __device__ __forceinline__ static int tap(int r) { return PAD ? r + N - 1 : r + N / 2; }
};

// z-line split / re-pack on the plane.  Split: Z (digit-reversed positions 0..NZC-1 of each line) ->
// 2 X[kz] at natural columns 0..NZC.  Re-pack: Y at natural columns 0..NZC -> Z'' at digit-reversed
// positions 0..NZC-1.  All reads happen before the barrier, all writes after.
template <class G, int NLINES, bool SPLIT>
__device__ __forceinline__ void k3_zline_pairs(float2* plane, const Twiddles& tw, int t) {
  using C = K3<G>;
  constexpr int NZC = C::NZC, NKZ = C::NKZ, T = C::T, HZ = NZC / 2;
  using ZRL = typename C::ZRL;
  constexpr int ITEMS = NLINES * (HZ + 1);
  constexpr int PER = (ITEMS + T - 1) / T;
  float2 a[PER], b[PER];
  static_for<PER>([&](auto ii) {
    const int it = t + T * ii.value;
    if (it >= ITEMS) return;
    const int y = it % NLINES, k = it / NLINES;   // lanes on consecutive lines: distinct banks
    const int kp = (NZC - k) % NZC;
    float2* line = plane + y * NKZ;
    const float2 w = twiddle<ilog2(2 * NZC)>(tw, uint32_t(k));
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
    const int y = it % NLINES, k = it / NLINES;   // lanes on consecutive lines: distinct banks
    float2* line = plane + y * NKZ;
    if constexpr (SPLIT) {
      line[k] = a[ii.value];
      if (k != 0 && k != HZ) line[NZC - k] = b[ii.value];
      if (k == 0) line[NZC] = b[ii.value];
    } else {
      line[ZRL::position_of_bin(k)] = a[ii.value];
      if (k != 0 && k != HZ) line[ZRL::position_of_bin(NZC - k)] = b[ii.value];
    }
  });
  __syncthreads();
}

// forward half of pass A on a plane whose packed z-lines are in place (lines y < NLINES nonzero)
template <class G, int NLINES>
__device__ __forceinline__ void k3_plane_forward(float2* plane, const Twiddles& tw, int t) {
  using C = K3<G>;
  constexpr bool HALF = C::PAD && NLINES == C::N;   // zero-padded activation slabs: y, z >= 64 are zero
  C::template ZEng<NLINES>::template forward<HALF>(plane, tw, t);
  k3_zline_pairs<G, NLINES, true>(plane, tw, t);
  C::YEng::template forward<HALF>(plane, tw, t);
}

// Pass A (MODE 0, from activations) or pass C (MODE 1, inverse + gate [+ chained pass A]).
// grid.x = 64 slabs * nq (volume fastest).
template <class G, bool BF16, int MODE, bool GATE, bool CHAIN>
__global__ void __launch_bounds__(k3::T)
k3_planes(const typename Store<BF16>::elem* u, const typename Store<BF16>::elem* gate,
          typename Store<BF16>::elem* y, float2* I, int q0, int nq, int B, int D, Twiddles tw) {
  using C = K3<G>;
  constexpr int N = C::N, T = C::T, PLANE = C::PLANE, NKZ = C::NKZ, NZIN = C::NZIN;
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
    static_for<(N * NZIN) / T>([&](auto ii) {
      const int e = t + T * ii.value;
      const int yy = e / NZIN, m = e % NZIN;
      plane[yy * NKZ + m] = St::load2(src + yy * N + 2 * m);
    });
    __syncthreads();
  } else {
    for (int j = t; j < PLANE; j += T) plane[j] = slab[j];
    __syncthreads();
    C::YEng::template inverse<C::PAD>(plane, tw, t);
    k3_zline_pairs<G, N, false>(plane, tw, t);
    C::template ZEng<N>::template inverse<C::PAD>(plane, tw, t);
    const auto* g = GATE ? gate + vol + (size_t)x * N * N : nullptr;
    auto* dst = CHAIN ? nullptr : y + vol + (size_t)x * N * N;
    static_for<(N * NZIN) / T>([&](auto ii) {
      const int e = t + T * ii.value;
      const int yy = e / NZIN, m = e % NZIN;
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
  k3_plane_forward<G, N>(plane, tw, t);
  for (int j = t; j < PLANE; j += T) slab[j] = plane[j];
}

// Pass A for the filter: taps h[d, W, W, W] (tap index of a signed offset: K3::tap) placed at r mod MP;
// all MP slabs.  Zero-padded: W = 127, offsets [-63, 63], index 64 of each axis empty.  Periodic:
// W = 64, offsets [-32, 31].
template <class G>
__global__ void __launch_bounds__(k3::T)
k3_planes_taps(const float* __restrict__ h, float2* I, int q0, int nq, Twiddles tw) {
  using C = K3<G>;
  constexpr int T = C::T, MP = C::MP, NZC = C::NZC, NKZ = C::NKZ, PLANE = C::PLANE, W = C::W;
  __shared__ float2 plane[PLANE];
  const int t = threadIdx.x;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ql = lb % nq, x = lb / nq;
  const int d = q0 + ql;
  const float* hd = h + (size_t)d * W * W * W;
  const int rx = C::offset(x);
  static_for<(MP * NZC) / T>([&](auto ii) {
    const int e = t + T * ii.value;
    const int yy = e / NZC, m = e % NZC;
    const int ry = C::offset(yy);
    float2 v = make_float2(0.f, 0.f);
    if (C::in_filter(x) && C::in_filter(yy)) {
      const float* line = hd + ((size_t)C::tap(rx) * W + C::tap(ry)) * W;
      const int z0 = 2 * m, z1 = 2 * m + 1;
      if (C::in_filter(z0)) v.x = line[C::tap(C::offset(z0))];
      if (C::in_filter(z1)) v.y = line[C::tap(C::offset(z1))];
    }
    plane[yy * NKZ + m] = v;
  });
  __syncthreads();
  k3_plane_forward<G, MP>(plane, tw, t);
  float2* slab = I + ((size_t)ql * MP + x) * PLANE;
  for (int j = t; j < PLANE; j += T) slab[j] = plane[j];
}

// Pass B.  MODE 0: x-transform (zero-padded: x >= 64 zero), product with Hs, inverse, keep x < 64
//          (in place).  MODE 1: x-transform of a full filter slab stack, write the scaled spectrum.
// grid.x = TILES * nq (volume fastest).
template <class G, int MODE>
__global__ void __launch_bounds__(k3::T)
k3_cols(float2* I, const float2* __restrict__ Hs, float2* __restrict__ Hs_out, int q0, int nq, int B, int hsb,
        Twiddles tw) {
  using C = K3<G>;
  constexpr int N = C::N, T = C::T, MP = C::MP, COLS = C::COLS, PLANE = C::PLANE, TILES = C::TILES;
  using XEng = typename C::XEng;
  constexpr int NX = (MODE == 0) ? N : MP;    // slabs present in the intermediate
  __shared__ float2 lds[lds_padded_size(COLS * MP)];
  const int t = threadIdx.x;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ql = lb % nq, tile = lb / nq;
  const int q = q0 + ql;
  // spectrum channel: d (one filter per channel, hsb = 0) or b * D + d (one per (b, d), hsb = D)
  const int d = (MODE == 0) ? q / B + (q % B) * hsb : q;
  const int j0 = tile * COLS;
  float2* base = I + (size_t)ql * NX * PLANE + j0;
  static_for<(NX * COLS) / T>([&](auto ii) {
    const int e = t + T * ii.value;
    const int xx = e / COLS, l = e % COLS;
    lds[XEng::addr(xx, l)] = base[(size_t)xx * PLANE + l];
  });
  __syncthreads();
  XEng::template forward<MODE == 0 && C::PAD>(lds, tw, t);
  const size_t hoff = ((size_t)d * TILES + tile) * (MP * COLS);
  if constexpr (MODE == 1) {
    static_for<(MP * COLS) / T>([&](auto ii) {
      const int e = t + T * ii.value;
      const int p = e / COLS, l = e % COLS;
      Hs_out[hoff + e] = cscale(lds[XEng::addr(p, l)], C::kSpecScale);
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
  XEng::template inverse<C::PAD>(lds, tw, t);
  static_for<(N * COLS) / T>([&](auto ii) {
    const int e = t + T * ii.value;
    const int xx = e / COLS, l = e % COLS;
    base[(size_t)xx * PLANE + l] = lds[XEng::addr(xx, l)];
  });
}

// Engine-order spectrum -> H[d, kx, ky, kz] (MP x MP x (MP/2+1), unscaled real-input DFT bins).
template <class G>
__global__ void k3_export(const float2* __restrict__ Hs, float2* __restrict__ H) {
  using C = K3<G>;
  constexpr int MP = C::MP, COLS = C::COLS, TILES = C::TILES, NKZ = C::NKZ;
  using XRL = typename C::XRL;
  using YRL = typename C::YRL;
  const int d = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= TILES * MP * COLS) return;
  const int tile = idx / (MP * COLS), rem = idx % (MP * COLS);
  const int p = rem / COLS, l = rem % COLS;
  const int j = tile * COLS + l;
  const int ypos = j / NKZ, kz = j % NKZ;
  const int kx = XRL::bin_of_position(p), ky = YRL::bin_of_position(ypos);
  H[(((size_t)d * MP + kx) * MP + ky) * NKZ + kz] =
      cscale(Hs[(size_t)d * TILES * MP * COLS + idx], 0.5f / C::kSpecScale);
}

// ------------------------------------------------------------------ zero-padded plan: z alone, then (x, y)
// Padding doubles the data along each axis it is applied to.  Run on the padded grid, passes A-C would
// store the volume after its z and y transforms (4x the activations).  This plan stores it after the z
// transform only (2x): its middle pass transforms x and y together in one LDS plane [128 x][128 y] per
// z-bin, where both paddings happen on chip.  Passes per (b, d) volume:
//   Z   k3z_lines   one x-slab: z-transform + split on [64 y][65 kz]; stored as J[kz][x][y] (x, y < 64)
//   XY  k3z_planes  one kz: J[kz] (32 KB) into the plane, y- and x-transforms (zero upper halves),
//                   product with the filter spectrum, inverse x and y keeping x, y < 64, back to J[kz]
//   Z'  k3z_lines   one x-slab: re-pack, inverse z (keep z < 64), gate; for every order but the last the
//                   same workgroup then runs the next order's pass Z
// Intermediate per volume: [65 kz][64 x][64 y] complex fp32 (2.13 MB).  Filter spectrum per channel:
// Hz[kz][x-position][y-position] (65 x 128 x 128), Hz = H / 2^22 where H is the 128^3 real-input DFT of the
// placed filter, built by the same two steps over all 128^3 placed taps.
namespace k3z {
constexpr int N = 64, MP = 128, NKZ = 65, T = 512;
constexpr int TXY = 1024;                      // pass XY: one workgroup per CU (its plane takes 129 KB)
constexpr int LSX = MP + 1;                    // plane row stride (odd: both transforms conflict-free)
constexpr int VOL = NKZ * N * N;               // complex per volume in the intermediate
constexpr int FVOL = NKZ * MP * MP;            // complex per channel while building a spectrum
using G = Geo3<false>;
using C = K3<G>;
// lines x (line stride LSX), positions y (contiguous); NL = 64 for activations, 128 for filters
template <int NL>
using YE = ColEngine<NL, 1, LSX, TXY, C::YRL, false>;
using XE = ColEngine<MP, LSX, 1, TXY, C::XRL, false>;   // lines y, positions x
}  // namespace k3z

// one x-slab's [NL y][65 kz] plane -> J[kz][x][y] (rows of NL y values per (kz, x))
template <int NL>
__device__ __forceinline__ void k3z_store_slab(const float2* plane, float2* Jv, int x, int t) {
  for (int e = t; e < k3z::NKZ * NL; e += k3z::T) {
    const int kz = e / NL, yy = e % NL;
    Jv[((size_t)kz * NL + x) * NL + yy] = plane[yy * k3z::NKZ + kz];
  }
}

// Pass Z (MODE 0, from activations) or pass Z' (MODE 1, inverse + gate [+ chained pass Z]).
// grid.x = 64 slabs * nq (volume fastest).
template <bool BF16, int MODE, bool GATE, bool CHAIN>
__global__ void __launch_bounds__(k3z::T)
k3z_lines(const typename Store<BF16>::elem* u, const typename Store<BF16>::elem* gate,
          typename Store<BF16>::elem* y, float2* J, int q0, int nq, int B, int D, Twiddles tw) {
  using namespace k3z;
  using St = Store<BF16>;
  constexpr int NZIN = C::NZIN;
  __shared__ float2 plane[N * NKZ];
  const int t = threadIdx.x;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ql = lb % nq, x = lb / nq;
  const int q = q0 + ql;
  const int d = q / B, b = q % B;
  const size_t vol = ((size_t)b * D + d) * (size_t)(N * N * N);
  float2* Jv = J + (size_t)ql * VOL;
  if constexpr (MODE == 0) {
    const auto* src = u + vol + (size_t)x * N * N;
    static_for<(N * NZIN) / T>([&](auto ii) {
      const int e = t + T * ii.value;
      const int yy = e / NZIN, m = e % NZIN;
      plane[yy * NKZ + m] = St::load2(src + yy * N + 2 * m);
    });
    __syncthreads();
  } else {
    for (int e = t; e < NKZ * N; e += T) {
      const int kz = e / N, yy = e % N;
      plane[yy * NKZ + kz] = Jv[((size_t)kz * N + x) * N + yy];
    }
    __syncthreads();
    k3_zline_pairs<G, N, false>(plane, tw, t);
    C::template ZEng<N>::template inverse<true>(plane, tw, t);
    const auto* g = GATE ? gate + vol + (size_t)x * N * N : nullptr;
    auto* dst = CHAIN ? nullptr : y + vol + (size_t)x * N * N;
    static_for<(N * NZIN) / T>([&](auto ii) {
      const int e = t + T * ii.value;
      const int yy = e / NZIN, m = e % NZIN;
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
  C::template ZEng<N>::template forward<true>(plane, tw, t);
  k3_zline_pairs<G, N, true>(plane, tw, t);
  k3z_store_slab<N>(plane, Jv, x, t);
}

// Pass Z for the filter: taps placed at r mod 128 on all 128 x-slabs and y-lines, half an x-slab (64
// y-lines, a 33 KB plane) per workgroup so that four share a CU.  grid.x = 2 * 128 half-slabs * nq
// (channel fastest).
__global__ void __launch_bounds__(k3z::T)
k3z_taps(const float* __restrict__ h, float2* J, int q0, int nq, Twiddles tw) {
  using namespace k3z;
  constexpr int NZC = C::NZC, W = C::W, NL = MP / 2;
  __shared__ float2 plane[NL * NKZ];
  const int t = threadIdx.x;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ql = lb % nq, hs = lb / nq;
  const int x = hs >> 1, y0 = NL * (hs & 1);
  const int d = q0 + ql;
  const float* hd = h + (size_t)d * W * W * W;
  const int rx = C::offset(x);
  static_for<(NL * NZC) / T>([&](auto ii) {
    const int e = t + T * ii.value;
    const int yl = e / NZC, m = e % NZC, yy = y0 + yl;
    const int ry = C::offset(yy);
    float2 v = make_float2(0.f, 0.f);
    if (C::in_filter(x) && C::in_filter(yy)) {
      const float* line = hd + ((size_t)C::tap(rx) * W + C::tap(ry)) * W;
      const int z0 = 2 * m, z1 = 2 * m + 1;
      if (C::in_filter(z0)) v.x = line[C::tap(C::offset(z0))];
      if (C::in_filter(z1)) v.y = line[C::tap(C::offset(z1))];
    }
    plane[yl * NKZ + m] = v;
  });
  __syncthreads();
  C::template ZEng<NL>::template forward<false>(plane, tw, t);
  k3_zline_pairs<G, NL, true>(plane, tw, t);
  // J[kz][x][y] (128 x 128 per z-bin): this half-slab's 64 y values of row (kz, x)
  float2* Jv = J + (size_t)ql * FVOL;
  for (int e = t; e < NKZ * NL; e += T) {
    const int kz = e / NL, yl = e % NL;
    Jv[((size_t)kz * MP + x) * MP + y0 + yl] = plane[yl * NKZ + kz];
  }
}

// Pass XY.  MODE 0: y- and x-transforms of J[kz] (x, y < 64; upper halves zero), product with Hz,
// inverse x and y keeping x, y < 64 (in place).  MODE 1: the same forward transforms of a full filter
// plane (128 x 128), written as the scaled spectrum.  grid.x = 65 z-bins * nq (volume fastest).
template <int MODE>
__global__ void __launch_bounds__(k3z::TXY)
k3z_planes(float2* J, const float2* __restrict__ Hs, float2* __restrict__ Hs_out, int q0, int nq, int B, int hsb,
           Twiddles tw) {
  using namespace k3z;
  constexpr int NXY = (MODE == 0) ? N : MP;    // x and y extent present in the intermediate
  using Y = YE<NXY>;
  __shared__ float2 lds[MP * LSX];
  const int t = threadIdx.x;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ql = lb % nq, kz = lb / nq;
  const int q = q0 + ql;
  // spectrum channel: d (one filter per channel, hsb = 0) or b * D + d (one per (b, d), hsb = D)
  const int d = (MODE == 0) ? q / B + (q % B) * hsb : q;
  float2* Jp = J + ((size_t)ql * NKZ + kz) * (NXY * NXY);
  static_for<(NXY * NXY) / TXY>([&](auto ii) {
    const int e = t + TXY * ii.value;
    lds[(e / NXY) * LSX + e % NXY] = Jp[e];
  });
  __syncthreads();
  Y::template forward<MODE == 0>(lds, tw, t);
  XE::template forward<MODE == 0>(lds, tw, t);
  const float2* hz = Hs + ((size_t)d * NKZ + kz) * (MP * MP);
  if constexpr (MODE == 1) {
    float2* ho = Hs_out + ((size_t)d * NKZ + kz) * (MP * MP);
    static_for<(MP * MP) / TXY>([&](auto ii) {
      const int e = t + TXY * ii.value;
      ho[e] = cscale(lds[(e / MP) * LSX + e % MP], C::kSpecScale);
    });
    return;
  }
  static_for<(MP * MP) / TXY>([&](auto ii) {
    const int e = t + TXY * ii.value;
    const int a = (e / MP) * LSX + e % MP;
    lds[a] = cmul(lds[a], hz[e]);
  });
  __syncthreads();
  XE::template inverse<true>(lds, tw, t);
  Y::template inverse<true>(lds, tw, t);
  static_for<(N * N) / TXY>([&](auto ii) {
    const int e = t + TXY * ii.value;
    Jp[e] = lds[(e / N) * LSX + e % N];
  });
}

// Hz spectrum -> H[d, kx, ky, kz] (unscaled real-input DFT bins).
__global__ void k3z_export(const float2* __restrict__ Hs, float2* __restrict__ H) {
  using namespace k3z;
  const int d = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= FVOL) return;
  const int kz = idx / (MP * MP), rem = idx % (MP * MP);
  const int kx = C::XRL::bin_of_position(rem / MP), ky = C::YRL::bin_of_position(rem % MP);
  H[(((size_t)d * MP + kx) * MP + ky) * NKZ + kz] = cscale(Hs[(size_t)d * FVOL + idx], 0.5f / C::kSpecScale);
}

// ------------------------------------------------------------------ host side
bool grid3d_supported(int64_t nx, int64_t ny, int64_t nz) { return nx == k3::N && ny == k3::N && nz == k3::N; }
size_t conv3d_volume_bytes(int circ) {
  return circ ? (size_t)k3::N * K3<Geo3<true>>::PLANE * sizeof(float2) : (size_t)k3z::VOL * sizeof(float2);
}
size_t conv3d_filter_volume_bytes(int circ) {
  return circ ? (size_t)K3<Geo3<true>>::MP * K3<Geo3<true>>::PLANE * sizeof(float2)
              : (size_t)k3z::FVOL * sizeof(float2);
}
size_t conv3d_spectrum_bytes_per_channel(int circ) {
  using A = K3<Geo3<true>>;
  return circ ? (size_t)A::TILES * A::MP * A::COLS * sizeof(float2) : (size_t)k3z::FVOL * sizeof(float2);
}
size_t conv3d_taps_per_channel(int circ) {
  return circ ? (size_t)K3<Geo3<true>>::W * K3<Geo3<true>>::W * K3<Geo3<true>>::W
              : (size_t)K3<Geo3<false>>::W * K3<Geo3<false>>::W * K3<Geo3<false>>::W;
}

namespace {
template <class G, bool BF16>
hipError_t conv3d_launch_t(int order, int B, int D, const void* v, const void* const* x, const void* const* spectra,
                           void* y, float2* I0, int chunk, const Twiddles& tw, hipStream_t s0, int hsb,
                           const SideStream* side) {
  using C = K3<G>;
  constexpr int N = C::N, T = C::T, TILES = C::TILES;
  using E = typename Store<BF16>::elem;
  const int rows = B * D;
  const int ways = (side != nullptr && rows > chunk) ? side->ways : 1;
  if (ways > 1) {
    const hipError_t e = side_fork(side, s0);
    if (e != hipSuccess) return e;
  }
  int k = 0;
  for (int q0 = 0; q0 < rows; q0 += chunk, ++k) {
    const int nq = (rows - q0 < chunk) ? rows - q0 : chunk;
    const int j = k % ways;
    const hipStream_t s = j ? side->s[j - 1] : s0;
    float2* I = I0 + (size_t)j * chunk * (conv3d_volume_bytes(G::PAD ? 0 : 1) / sizeof(float2));
    hipLaunchKernelGGL((k3_planes<G, BF16, 0, false, false>), dim3(N * nq), dim3(T), 0, s, (const E*)v,
                       (const E*)nullptr, (E*)nullptr, I, q0, nq, B, D, tw);
    for (int i = 0; i < order; ++i) {
      hipLaunchKernelGGL((k3_cols<G, 0>), dim3(TILES * nq), dim3(T), 0, s, I, (const float2*)spectra[i],
                         (float2*)nullptr, q0, nq, B, hsb, tw);
      if (i + 1 < order)
        hipLaunchKernelGGL((k3_planes<G, BF16, 1, true, true>), dim3(N * nq), dim3(T), 0, s, (const E*)nullptr,
                           (const E*)x[i], (E*)nullptr, I, q0, nq, B, D, tw);
      else if (x[i])
        hipLaunchKernelGGL((k3_planes<G, BF16, 1, true, false>), dim3(N * nq), dim3(T), 0, s, (const E*)nullptr,
                           (const E*)x[i], (E*)y, I, q0, nq, B, D, tw);
      else
        hipLaunchKernelGGL((k3_planes<G, BF16, 1, false, false>), dim3(N * nq), dim3(T), 0, s, (const E*)nullptr,
                           (const E*)nullptr, (E*)y, I, q0, nq, B, D, tw);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return ways > 1 ? side_join(side, s0) : hipSuccess;
}

template <class G>
hipError_t spectrum3d_launch_t(const float* h, float2* Hs, int D, float2* I, int chunk, const Twiddles& tw,
                               hipStream_t s) {
  using C = K3<G>;
  for (int q0 = 0; q0 < D; q0 += chunk) {
    const int nq = (D - q0 < chunk) ? D - q0 : chunk;
    hipLaunchKernelGGL((k3_planes_taps<G>), dim3(C::MP * nq), dim3(C::T), 0, s, h, I, q0, nq, tw);
    hipLaunchKernelGGL((k3_cols<G, 1>), dim3(C::TILES * nq), dim3(C::T), 0, s, I, (const float2*)nullptr, Hs, q0,
                       nq, 1, 0, tw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <class G>
hipError_t export3d_launch_t(const float2* Hs, float2* H, int D, hipStream_t s) {
  using C = K3<G>;
  const int n = C::TILES * C::MP * C::COLS;
  hipLaunchKernelGGL((k3_export<G>), dim3((n + 255) / 256, D), dim3(256), 0, s, Hs, H);
  return hipGetLastError();
}
// zero-padded geometry: passes Z, XY, Z' per chunk of volumes
template <bool BF16>
hipError_t conv3d_pad_launch(int order, int B, int D, const void* v, const void* const* x, const void* const* spectra,
                             void* y, float2* I0, int chunk, const Twiddles& tw, hipStream_t s0, int hsb,
                             const SideStream* side) {
  using namespace k3z;
  using E = typename Store<BF16>::elem;
  const int rows = B * D;
  const int ways = (side != nullptr && rows > chunk) ? side->ways : 1;
  if (ways > 1) {
    const hipError_t e = side_fork(side, s0);
    if (e != hipSuccess) return e;
  }
  int k = 0;
  for (int q0 = 0; q0 < rows; q0 += chunk, ++k) {
    const int nq = (rows - q0 < chunk) ? rows - q0 : chunk;
    const int j = k % ways;
    const hipStream_t s = j ? side->s[j - 1] : s0;
    float2* I = I0 + (size_t)j * chunk * VOL;
    hipLaunchKernelGGL((k3z_lines<BF16, 0, false, false>), dim3(N * nq), dim3(T), 0, s, (const E*)v,
                       (const E*)nullptr, (E*)nullptr, I, q0, nq, B, D, tw);
    for (int i = 0; i < order; ++i) {
      hipLaunchKernelGGL((k3z_planes<0>), dim3(NKZ * nq), dim3(TXY), 0, s, I, (const float2*)spectra[i],
                         (float2*)nullptr, q0, nq, B, hsb, tw);
      if (i + 1 < order)
        hipLaunchKernelGGL((k3z_lines<BF16, 1, true, true>), dim3(N * nq), dim3(T), 0, s, (const E*)nullptr,
                           (const E*)x[i], (E*)nullptr, I, q0, nq, B, D, tw);
      else if (x[i])
        hipLaunchKernelGGL((k3z_lines<BF16, 1, true, false>), dim3(N * nq), dim3(T), 0, s, (const E*)nullptr,
                           (const E*)x[i], (E*)y, I, q0, nq, B, D, tw);
      else
        hipLaunchKernelGGL((k3z_lines<BF16, 1, false, false>), dim3(N * nq), dim3(T), 0, s, (const E*)nullptr,
                           (const E*)nullptr, (E*)y, I, q0, nq, B, D, tw);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return ways > 1 ? side_join(side, s0) : hipSuccess;
}

hipError_t spectrum3d_pad_launch(const float* h, float2* Hs, int D, float2* I, int chunk, const Twiddles& tw,
                                 hipStream_t s) {
  using namespace k3z;
  for (int q0 = 0; q0 < D; q0 += chunk) {
    const int nq = (D - q0 < chunk) ? D - q0 : chunk;
    hipLaunchKernelGGL(k3z_taps, dim3(2 * MP * nq), dim3(T), 0, s, h, I, q0, nq, tw);
    hipLaunchKernelGGL((k3z_planes<1>), dim3(NKZ * nq), dim3(TXY), 0, s, I, (const float2*)nullptr, Hs, q0, nq, 1, 0,
                       tw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
}  // namespace

hipError_t launch_conv3d(int bf16, int order, int B, int D, const void* v, const void* const* x,
                         const void* const* spectra, void* y, float2* I, int chunk, const Twiddles& tw, hipStream_t s,
                         int circ, int hsb, const SideStream* side) {
  if (circ)
    return bf16 ? conv3d_launch_t<Geo3<true>, true>(order, B, D, v, x, spectra, y, I, chunk, tw, s, hsb, side)
                : conv3d_launch_t<Geo3<true>, false>(order, B, D, v, x, spectra, y, I, chunk, tw, s, hsb, side);
  return bf16 ? conv3d_pad_launch<true>(order, B, D, v, x, spectra, y, I, chunk, tw, s, hsb, side)
              : conv3d_pad_launch<false>(order, B, D, v, x, spectra, y, I, chunk, tw, s, hsb, side);
}

hipError_t launch_spectrum3d(const float* h, float2* Hs, int D, float2* I, int chunk, const Twiddles& tw,
                             hipStream_t s, int circ) {
  return circ ? spectrum3d_launch_t<Geo3<true>>(h, Hs, D, I, chunk, tw, s)
              : spectrum3d_pad_launch(h, Hs, D, I, chunk, tw, s);
}

hipError_t launch_export3d(const float2* Hs, float2* H, int D, hipStream_t s, int circ) {
  if (circ) return export3d_launch_t<Geo3<true>>(Hs, H, D, s);
  hipLaunchKernelGGL(k3z_export, dim3((k3z::FVOL + 255) / 256, D), dim3(256), 0, s, Hs, H);
  return hipGetLastError();
}

}  // namespace hyena
