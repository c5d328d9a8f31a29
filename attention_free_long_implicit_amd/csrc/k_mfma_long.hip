// Matrix-core causal long convolution for bf16 storage and long rows (L = 2^15, 2^16), rows taken in pairs.
//
// Operation: Hyena study note, steps 2-3 (long convolution with the implicit filter, gate); EulerStack
// "4. Hyena 상세", how it works 2 (FFT, elementwise product, inverse FFT); HyenaND summary, boundary handling
// (zero-pad to twice the size).  A row of 2L samples is too long for one workgroup, so the transform is split
// four-step style, N = 2L = N1 x N2 with N2 = 16384 the matrix-core transform of the 8192-sample kernel:
//
//   n = m + N2 n0 (n0 < N1, only n0 < N1/2 non-zero: the zero padding), k = k0 + N1 kappa,
//   W_N^{nk} = W_N1^{n0 k0} . W_N^{m k0} . W_N2^{m kappa}.
//
//   column pass (k_mfl_cols): for every column m, the N1-point DFT over n0 and the twiddle W_N^{m k0}
//       -> plane k0, X[k0][m]; in fp32, one thread per four consecutive columns.
//   plane pass  (k_mfl_planes): every plane k0 is an N2-point sequence: forward transform on the matrix
//       cores, product with the filter spectrum at bins k0 + N1 kappa (scaled by 1/N), inverse transform;
//       the passes and the slab decomposition are those of the 8192-sample kernel (16 x 32 x 32), with all
//       16 inputs of the first radix-16 product non-zero and all 16 outputs of the last one kept.
//   column pass again: conjugate twiddle, inverse N1-point DFT over k0, keep n0 < N1/2 (the causal half),
//       gate; for every order but the last the same workgroup then runs the next order's forward column
//       pass on the gated values, so u_i never goes to memory.
//
// Rows are paired as in the 8192-sample kernel: z = u_b0 + i u_b1 for two rows of one channel (h is real, so
// the inverse transform of DFT(z) H is (h * u_b0) + i (h * u_b1)).  A pair's planes live in the workspace as
// fp16 (11-bit significand), real parts and imaginary parts in separate planes, each block of values written
// by one workgroup scaled by a power of two (its exponent stored beside the planes; the reader scales back
// exactly).  Each workgroup of the plane pass takes the two planes k0 and N1 - k0 (0 and N1/2 together), whose
// filter-spectrum bins mirror each other (H[N - k] = conj H[k]), so one stored half serves both.
#include "engine.h"
#include "launch.h"
#include "mfma_core.h"

namespace hyena {

namespace mfl {
constexpr int N2 = 16384;                 // plane length
constexpr int TILE_C = 64;                // column pass: columns c .. c + 63 (mod 1024) for all 16 n1
constexpr int NTILE = 1024 / TILE_C;      // column tiles per pair
constexpr int TC = 256;                   // column-pass threads: four consecutive columns each
constexpr int TP = 512;                   // plane-pass threads: two planes of four waves
// Per pair: N1 planes of N2 fp16 real parts then N2 fp16 imaginary parts (N 32-bit words), then a header of
// HDR 32-bit words: the column pass's tile exponents (H_EA + tile); its per-tile "row is non-zero" bits in two
// slots by order parity (H_NZ + 32 slot + 2 tile + row: the column pass of order i reads slot i % 2 while
// writing slot (i + 1) % 2 for the next order); the plane pass's plane exponents (H_EB + k0).
enum { H_EA = 0, H_NZ = 32, H_EB = 128, HDR = 256 };
template <int N1>
struct Plan {
  static_assert(N1 == 4 || N1 == 8, "L = 2^15 or 2^16");
  static constexpr int N = N1 * N2;
  static constexpr int L = N / 2;
  static constexpr int LOG2N = N1 == 4 ? 16 : 17;
  static constexpr size_t PAIR_WORDS = (size_t)N + HDR;
  // spectrum slots of 16 words x 64 lanes: plane 0 slabs 0..8, plane N1/2 slabs 0..7, planes 1..N1/2-1
  // slabs 0..15; then a 64-word tail (word 0: the exponent of the table's scale back)
  static constexpr int SLOTS = 8 * N1 + 1;
  static constexpr int SPEC_WORDS = SLOTS * 1024 + 64;
};
}  // namespace mfl

// Largest value of a and of b, and the OR of c and of d, over the 256 threads (4 waves) of the workgroup;
// red: 16 words of LDS.  The caller's next barrier must not be this one's.
__device__ __forceinline__ void block_reduce4(float& a, float& b, uint32_t& c, uint32_t& d, uint32_t* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a = fmaxf(a, __shfl_xor(a, o));
    b = fmaxf(b, __shfl_xor(b, o));
    c |= __shfl_xor(c, o);
    d |= __shfl_xor(d, o);
  }
  if ((threadIdx.x & 63) == 0) {
    uint32_t* r = red + 4 * (threadIdx.x >> 6);
    r[0] = __float_as_uint(a);
    r[1] = __float_as_uint(b);
    r[2] = c;
    r[3] = d;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    a = fmaxf(a, __uint_as_float(red[4 * w]));
    b = fmaxf(b, __uint_as_float(red[4 * w + 1]));
    c |= red[4 * w + 2];
    d |= red[4 * w + 3];
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ----------------------------------------------------------------------------------------------
// Column pass.  MODE 0: forward from the bf16 input u (first order).  MODE 1: inverse of the planes, gate
// (GATE), then store y, or (CHAIN) the forward column pass of the next order on the gated values.
// grid.x = NTILE * nq (pair fastest); thread t: n1 = t / 16, columns m = 64 tile + 4 (t % 16) + i + 1024 n1,
// i < 4, so each access of a plane or a row is 8 bytes, 16 threads per 128-byte segment.
template <int N1, int MODE, bool GATE, bool CHAIN>
__global__ void __launch_bounds__(mfl::TC)
k_mfl_cols(const uint16_t* u, const uint16_t* gate, uint16_t* y, uint32_t* W, int q0, int nq, int B, int D,
           int par, Twiddles tw) {
  using namespace mfl;
  using P = Plan<N1>;
  constexpr int N = P::N, L = P::L, H = N1 / 2;
  __shared__ uint32_t red[16];
  const int t = threadIdx.x;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int pl = lb % nq, tile = lb / nq;
  const int q = q0 + pl;
  const int np = B >> 1;
  const int d = q / np, bp = q % np;
  const size_t r0 = (size_t)(2 * bp) * D + d, r1 = r0 + D;
  uint32_t* const Wp = W + (size_t)pl * P::PAIR_WORDS;
  uint16_t* const planes = reinterpret_cast<uint16_t*>(Wp);
  uint32_t* const hdr = Wp + N;
  const int m0 = TILE_C * tile + 4 * (t & 15) + 1024 * (t >> 4);

  float2 z[4][H];   // [column][n0]: row b0 in x, row b1 in y
  if constexpr (MODE == 0) {
#pragma unroll
    for (int n0 = 0; n0 < H; ++n0) {
      const uint2 a = *reinterpret_cast<const uint2*>(u + r0 * L + m0 + N2 * n0);
      const uint2 b = *reinterpret_cast<const uint2*>(u + r1 * L + m0 + N2 * n0);
      z[0][n0] = make_float2(bf16_lo(a.x), bf16_lo(b.x));
      z[1][n0] = make_float2(bf16_hi(a.x), bf16_hi(b.x));
      z[2][n0] = make_float2(bf16_lo(a.y), bf16_lo(b.y));
      z[3][n0] = make_float2(bf16_hi(a.y), bf16_hi(b.y));
    }
  } else {
    uint2 re[N1], im[N1];
#pragma unroll
    for (int k0 = 0; k0 < N1; ++k0) {
      re[k0] = *reinterpret_cast<const uint2*>(planes + (size_t)k0 * 2 * N2 + m0);
      im[k0] = *reinterpret_cast<const uint2*>(planes + (size_t)k0 * 2 * N2 + N2 + m0);
    }
    uint2 g0[H], g1[H];
    if constexpr (GATE) {
#pragma unroll
      for (int n0 = 0; n0 < H; ++n0) {
        g0[n0] = *reinterpret_cast<const uint2*>(gate + r0 * L + m0 + N2 * n0);
        g1[n0] = *reinterpret_cast<const uint2*>(gate + r1 * L + m0 + N2 * n0);
      }
    }
    // exponents of the plane pass's blocks; a row whose input to this order was all zeros gives exact zeros
    float eb[N1];
#pragma unroll
    for (int k0 = 0; k0 < N1; ++k0) eb[k0] = __builtin_ldexpf(1.0f, (int)hdr[H_EB + k0]);
    uint32_t nz0 = 0, nz1 = 0;
#pragma unroll
    for (int k = 0; k < NTILE; ++k) {
      nz0 |= hdr[H_NZ + 32 * par + 2 * k];
      nz1 |= hdr[H_NZ + 32 * par + 2 * k + 1];
    }
    const float keep0 = nz0 ? 1.0f : 0.0f, keep1 = nz1 ? 1.0f : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2 w = twiddle<P::LOG2N>(tw, uint32_t(m0 + i));
      float2 p[N1];
      twiddle_powers<N1>(w, p);
      float2 x[N1];
#pragma unroll
      for (int k0 = 0; k0 < N1; ++k0) {
        const uint32_t rw = (i < 2) ? re[k0].x : re[k0].y, iw = (i < 2) ? im[k0].x : im[k0].y;
        const f16x2 rh = __builtin_bit_cast(f16x2, rw), ih = __builtin_bit_cast(f16x2, iw);
        const float xr = (float)((i & 1) ? rh.y : rh.x), xi = (float)((i & 1) ? ih.y : ih.x);
        x[k0] = cmulc(make_float2(xr * eb[k0], xi * eb[k0]), p[k0]);
      }
      dft<N1, true, false, true>(x);
#pragma unroll
      for (int n0 = 0; n0 < H; ++n0) {
        float a = x[n0].x * keep0, b = x[n0].y * keep1;
        if constexpr (GATE) {
          const uint32_t ga = (i < 2) ? g0[n0].x : g0[n0].y, gb = (i < 2) ? g1[n0].x : g1[n0].y;
          a *= (i & 1) ? bf16_hi(ga) : bf16_lo(ga);
          b *= (i & 1) ? bf16_hi(gb) : bf16_lo(gb);
        }
        z[i][n0] = make_float2(a, b);
      }
    }
    if constexpr (!CHAIN) {
#pragma unroll
      for (int n0 = 0; n0 < H; ++n0) {
        uint2 ya, yb;
        ya.x = f32x2_to_bf16x2_rne(z[0][n0].x, z[1][n0].x);
        ya.y = f32x2_to_bf16x2_rne(z[2][n0].x, z[3][n0].x);
        yb.x = f32x2_to_bf16x2_rne(z[0][n0].y, z[1][n0].y);
        yb.y = f32x2_to_bf16x2_rne(z[2][n0].y, z[3][n0].y);
        *reinterpret_cast<uint2*>(y + r0 * L + m0 + N2 * n0) = ya;
        *reinterpret_cast<uint2*>(y + r1 * L + m0 + N2 * n0) = yb;
      }
      return;
    }
  }

  // forward column pass: the tile's scale from a bound (each output component is at most N1 times the largest
  // input component), and per row whether any input is non-zero
  float a0 = 0.0f, a1 = 0.0f;
  uint32_t o0 = 0, o1 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n0 = 0; n0 < H; ++n0) {
      a0 = fmaxf(a0, fabsf(z[i][n0].x));
      a1 = fmaxf(a1, fabsf(z[i][n0].y));
      o0 |= __float_as_uint(z[i][n0].x) & 0x7fffffffu;
      o1 |= __float_as_uint(z[i][n0].y) & 0x7fffffffu;
    }
  block_reduce4(a0, a1, o0, o1, red);
  const int ex = h16_exponent((float)N1 * fmaxf(a0, a1));
  const float sc = __builtin_ldexpf(1.0f, -ex);
  if (t == 0) {
    const int slot = MODE == 0 ? par : par ^ 1;
    hdr[H_EA + tile] = (uint32_t)ex;
    hdr[H_NZ + 32 * slot + 2 * tile] = o0;
    hdr[H_NZ + 32 * slot + 2 * tile + 1] = o1;
  }
  uint32_t rw[N1][2], iw[N1][2];   // fp16 pairs of columns (0, 1) and (2, 3)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2 w = twiddle<P::LOG2N>(tw, uint32_t(m0 + i));
    float2 p[N1];
    twiddle_powers<N1>(w, p);
    float2 x[N1];
#pragma unroll
    for (int n0 = 0; n0 < H; ++n0) x[n0] = z[i][n0];
    dft<N1, false, true, false>(x);
#pragma unroll
    for (int k0 = 0; k0 < N1; ++k0) {
      const float2 v = cmul(x[k0], p[k0]);
      const _Float16 vr = (_Float16)(v.x * sc), vi = (_Float16)(v.y * sc);
      const uint32_t br = __builtin_bit_cast(uint16_t, vr), bi = __builtin_bit_cast(uint16_t, vi);
      if (i & 1) {
        rw[k0][i >> 1] |= br << 16;
        iw[k0][i >> 1] |= bi << 16;
      } else {
        rw[k0][i >> 1] = br;
        iw[k0][i >> 1] = bi;
      }
    }
  }
#pragma unroll
  for (int k0 = 0; k0 < N1; ++k0) {
    *reinterpret_cast<uint2*>(planes + (size_t)k0 * 2 * N2 + m0) = make_uint2(rw[k0][0], rw[k0][1]);
    *reinterpret_cast<uint2*>(planes + (size_t)k0 * 2 * N2 + N2 + m0) = make_uint2(iw[k0][0], iw[k0][1]);
  }
}

// ----------------------------------------------------------------------------------------------
// Plane pass: workgroup = planes k0 = g and N1 - g of one pair (g = 0: planes 0 and N1/2), 8 waves, one LDS
// plane each.  Waves 4q..4q+3 run pass 1 and pass 1' of plane q; in passes 2..2' wave w owns slabs w and
// w + 8 of both planes, with one set of matrix loads.  The transform steps are those of k_conv_mfma (the
// 8192-sample kernel): pass 1 radix 16 over n1 (all 16 inputs), pass 2 radix 32 with the slab's matrix,
// twiddle W_1024, pass 3 radix 32 -> bins kappa = k1 + 16 k2 + 512 k3; product; passes 3', 2', 1' inverse.
//
// Scaling (all exact powers of two): the column pass's tiles have exponents e_A; the plane's input is read
// as fp16 and its first product's accumulators are scaled by 2^(e_A - E - 16), E = max e_A, which puts every
// input component below 1/2 (with all 16 inputs non-zero, no intermediate then exceeds 2^14.5); the spectrum
// table holds c H / N; the output block is stored as fp16 scaled by 2^-e', e' chosen from a bound (each
// output component is at most 32 times the largest value pass 2' leaves), with
// e_B = e' + 10 + log2(1/c) + E + 16 recorded for the column pass.
template <int N1>
__global__ void __launch_bounds__(mfl::TP, 1)
k_mfl_planes(uint32_t* W, const uint32_t* __restrict__ spec, const u32x4* __restrict__ mats, int q0, int nq, int B) {
  using namespace mf;
  using P = mfl::Plan<N1>;
  constexpr int N2 = mfl::N2, NW = 8, NIT = 2, G = N1 / 2;
  __shared__ uint32_t S[2 * PLANE];
  __shared__ float red[2 * NW];
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int pl = lb / G, g = lb % G;
  const int d = (q0 + pl) / (B >> 1);
  uint32_t* const Wp = W + (size_t)pl * P::PAIR_WORDS;
  uint16_t* const planes = reinterpret_cast<uint16_t*>(Wp);
  uint32_t* const hdr = Wp + P::N;
  const int mine = (int)(threadIdx.x >> 8);
  auto plane_of = [&](int qq) { return qq == 0 ? g : (g == 0 ? N1 / 2 : N1 - g); };

  const int t = threadIdx.x, w = t >> 6, wq = w & 3, l = t & 63, j = l & 31, h = l >> 5;
  const int c0 = 256 * wq + 8 * j;
  const int n2c = 8 * wq + (j >> 2), n3c = 8 * (j & 3);
  uint32_t* const Sm = S + mine * PLANE;
  uint16_t* const Pm = planes + (size_t)plane_of(mine) * 2 * N2;   // this group's plane (real parts first)

  // pass 1 input: lanes h = 0 / 1 carry the real / imaginary parts, n1 = e, 8 consecutive columns each
  u32x4 VA[8], VB[8];   // n1 = e, n1 = 8 + e
  {
    const uint16_t* src = Pm + h * N2 + c0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      VA[e] = *reinterpret_cast<const u32x4*>(src + 1024 * e);
      VB[e] = *reinterpret_cast<const u32x4*>(src + 1024 * (8 + e));
    }
  }
  const u32x4 m1a = mats[M1F_H * 64 + l], m1b = mats[M1F_H2 * 64 + l];
  const u32x4 m1r = mats[M1I_R * 64 + l], m1i = mats[M1I_I * 64 + l];
  f16x2 pc[8], ps[8];
  {
    const u32x4 a0 = mats[TW_C0 * 64 + l], a1 = mats[TW_C1 * 64 + l];
    const u32x4 s0 = mats[TW_S0 * 64 + l], s1 = mats[TW_S1 * 64 + l];
    // (through scalars: a bit cast of a subscripted vector element reads element 0 with this compiler)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = a0[q], b = a1[q], e = s0[q], f = s1[q];
      pc[q] = __builtin_bit_cast(f16x2, a);
      pc[4 + q] = __builtin_bit_cast(f16x2, b);
      ps[q] = __builtin_bit_cast(f16x2, e);
      ps[4 + q] = __builtin_bit_cast(f16x2, f);
    }
  }
  int E = -1000;
#pragma unroll
  for (int k = 0; k < mfl::NTILE; ++k) E = max(E, (int)hdr[mfl::H_EA + k]);
  const float f_in = __builtin_ldexpf(1.0f, (int)hdr[mfl::H_EA + (c0 >> 6)] - E - 16);
  const uint32_t* __restrict__ Hc = spec + (size_t)d * P::SPEC_WORDS;
  const int eH = (int)Hc[P::SLOTS * 1024];

  f16x8 Ma[NBLK], Mb[NBLK];
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(mats + NFIX * 64), (short)0, 16 * SLAB_TABLE * 64 * 16, kRawBufferWord3);
  const int mvo = l * 16;
  auto load_mat = [&](int k1s_, int which, f16x8 (&M)[NBLK]) {
#pragma unroll
    for (int b = 0; b < NBLK; ++b)
      M[b] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                           mrs, mvo, ((k1s_ * SLAB_TABLE + which * NBLK + b) * 64) * 16, 0));
  };
  // Spectrum slot of plane qq's slab k1 and whether it is read mirrored.  Bin N - k of (plane k0, slab k1,
  // lane l, register v) is register 15 - v of lane 63 - l in plane N1 - k0, slab 15 - k1 (slab 16 - k1 for
  // plane 0, whose mirror is itself): a mirrored read takes word 7 - q / 23 - q of lane 63 - l and uses it
  // with the halves swapped and conjugated.  All wave-uniform.
  auto slot_of = [&](int qq, int k1, bool& mir) {
    if (g == 0) {
      if (qq == 0) {
        mir = k1 > 8;
        return mir ? 16 - k1 : k1;
      }
      mir = k1 > 7;
      return 9 + (mir ? 15 - k1 : k1);
    }
    mir = qq == 1;
    return 17 + 16 * (g - 1) + (mir ? 15 - k1 : k1);
  };
  uint32_t hw[2][16];
  const __amdgpu_buffer_rsrc_t hrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)Hc, (short)0, P::SLOTS * 1024 * 4, kRawBufferWord3);
  const int ws = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto load_spectrum = [&](int k1s) {
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      bool mir;
      const int slot = slot_of(qq, k1s, mir);
      const int vo = (mir ? 63 - l : l) * 4;
#pragma unroll
      for (int k = 0; k < 16; ++k)
        hw[qq][k] = __builtin_amdgcn_raw_buffer_load_b32(hrs, vo, slot * 4096 + (mir ? (k < 8 ? 7 - k : 23 - k) : k) * 256, 0);
    }
  };
  load_mat(ws, MF2, Ma);
  load_mat(ws, MF3, Mb);
  load_spectrum(ws);
  // pass 1: both halves of the radix-16 input (n1 < 8, n1 >= 8), accumulators scaled into range
  static_for<8>([&](auto tt) {
    constexpr int TT = tt.value;
    const f32x16 z = {};
    f32x16 D1 = mfma(as_h(m1a), as_h(column8<TT>(VA)), z);
    D1 = mfma(as_h(m1b), as_h(column8<TT>(VB)), D1);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      Sm[acc_row(e, h) * SLAB + n2c * ROW + n3c + TT] = pack2h(D1[e] * f_in, D1[8 + e] * f_in);
  });
  __syncthreads();

  float vm[2] = {0.0f, 0.0f};   // largest |value| pass 2' leaves, per plane
  auto slab_step = [&](auto itc) {
    constexpr int it = decltype(itc)::value;
    const int k1 = w + NW * it;
    const int k1s = ws + NW * it;
    f16x8 xr_lo[2], xr_hi[2], xi_lo[2], xi_hi[2];
    f32x16 dr[2], di[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t* sl = S + q * PLANE + k1 * SLAB;
      uint32_t clo[8], chi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        clo[e] = sl[(8 * h + e) * ROW + j];
        chi[e] = sl[(16 + 8 * h + e) * ROW + j];
      }
      split8(clo, xr_lo[q], xi_lo[q]);
      split8(chi, xr_hi[q], xi_hi[q]);
      dft32<false, true>(Ma, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q], dr[q], di[q]);
    }
    load_mat(k1s, MI3, Ma);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      f16x2 ar[8], ai[8];
      to_pairs(dr[q], ar);
      to_pairs(di[q], ai);
      cmul_pairs<false>(ar, ai, pc, ps, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q]);
      dft32<false, false>(Mb, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q], dr[q], di[q]);
    }
    load_mat(k1s, MI2, Mb);
    // spectral product, plane by plane (bin k0 + N1 (k1 + 16 j + 512 k3(v)))
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      f16x2 hr[8], hi[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        hr[k] = __builtin_bit_cast(f16x2, hw[q][k]);
        hi[k] = __builtin_bit_cast(f16x2, hw[q][8 + k]);
      }
      f16x2 ar[8], ai[8];
      to_pairs(dr[q], ar);
      to_pairs(di[q], ai);
      bool mir;
      slot_of(q, k1s, mir);
      if (mir) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          hr[k] = hr[k].yx;
          hi[k] = hi[k].yx;
        }
        cmul_pairs<true>(ar, ai, hr, hi, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q]);
      } else {
        cmul_pairs<false>(ar, ai, hr, hi, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q]);
      }
    }
    if (it + 1 < NIT) load_spectrum(k1s + NW);
#pragma unroll
    for (int q = 0; q < 2; ++q) dft32<true, true>(Ma, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q], dr[q], di[q]);
    if (it + 1 < NIT) load_mat(k1s + NW, MF2, Ma);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      f16x2 ar[8], ai[8];
      to_pairs(dr[q], ar);
      to_pairs(di[q], ai);
      cmul_pairs<true>(ar, ai, pc, ps, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q]);
      dft32<true, false>(Mb, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q], dr[q], di[q]);
    }
    if (it + 1 < NIT) load_mat(k1s + NW, MF3, Mb);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t* sl = S + q * PLANE + k1 * SLAB;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        vm[q] = fmaxf(vm[q], fmaxf(fabsf(dr[q][v]), fabsf(di[q][v])));
        sl[acc_row(v, h) * ROW + j] = pack2h(dr[q][v], di[q][v]);
      }
    }
  };
  static_for<NIT>([&](auto itc) { slab_step(itc); });
#pragma unroll
  for (int q = 0; q < 2; ++q) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) vm[q] = fmaxf(vm[q], __shfl_xor(vm[q], o));
  }
  if (l == 0) {
    red[2 * w] = vm[0];
    red[2 * w + 1] = vm[1];
  }
  __syncthreads();

  // pass 1': all 16 outputs n1 of tile TT: register s < 8 of a lane is the real part of n1(s), register
  // 8 + s the imaginary part, n1(s) = 4h + s (s < 4) or 8 + 4h + s - 4; stored as fp16, two tiles per word
  float mp = 0.0f;
#pragma unroll
  for (int k = 0; k < NW; ++k) mp = fmaxf(mp, red[2 * k + mine]);
  const int eo = h16_exponent(32.0f * mp);
  const float so = __builtin_ldexpf(1.0f, -eo);
  u32x4 outR[8], outI[8];
  static_for<4>([&](auto tp) {
    constexpr int TP2 = tp.value;
    f32x16 o[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int TT = 2 * TP2 + u;
      uint32_t cw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cw[e] = Sm[(8 * h + e) * SLAB + n2c * ROW + n3c + TT];
      f16x8 xr, xi;
      split8(cw, xr, xi);
      const f32x16 z = {};
      o[u] = mfma(as_h(m1r), xr, z);
      o[u] = mfma(as_h(m1i), xi, o[u]);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      outR[s][TP2] = pack2h(o[0][s] * so, o[1][s] * so);
      outI[s][TP2] = pack2h(o[0][8 + s] * so, o[1][8 + s] * so);
    }
  });
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int n1 = s < 4 ? 4 * h + s : 8 + 4 * h + (s - 4);
    *reinterpret_cast<u32x4*>(Pm + c0 + 1024 * n1) = outR[s];
    *reinterpret_cast<u32x4*>(Pm + N2 + c0 + 1024 * n1) = outI[s];
  }
  if ((threadIdx.x & 255) == 0) hdr[mfl::H_EB + plane_of(mine)] = (uint32_t)(eo + 10 + eH + E + 16);
}

// Spectrum copy of one channel per workgroup from the natural-order bins 0..L of the 2L-point DFT (upper bins
// by conjugate symmetry): slot s (see Plan) of plane k0, slab k1: word q < 8 of lane l holds the real parts of
// c H[k(2q)] / N and c H[k(2q + 1)] / N as fp16 (register 2q low), word 8 + q their imaginary parts,
// k(v) = k0 + N1 (k1 + 16 (l % 32) + 512 k3(v, l / 32)); then the tail, word 0 = log2(1/c).  c is the power of
// two that brings the channel's largest |H[k]| / N into [0.5, 1).
template <int N1>
__global__ void __launch_bounds__(256) k_mfl_spectrum(const float2* __restrict__ Hnat, uint32_t* __restrict__ Hc) {
  using namespace mf;
  using P = mfl::Plan<N1>;
  constexpr int L = P::L, N = P::N;
  __shared__ float red[4];
  const int d = blockIdx.x;
  const float2* hn = Hnat + (size_t)d * (L + 1);
  float m = 0.0f;
  for (int k = threadIdx.x; k <= L; k += 256) m = fmaxf(m, fmaxf(fabsf(hn[k].x), fabsf(hn[k].y)));
  const float c = range_scale(block_max4(m * (1.0f / N), red));
  const float sc = c * (1.0f / N);
  uint32_t* out = Hc + (size_t)d * P::SPEC_WORDS;
  auto bin = [&](int k) { return k <= L ? hn[k] : cconj(hn[N - k]); };
  for (int idx = threadIdx.x; idx < P::SLOTS * 1024; idx += 256) {   // (slot, word, lane)
    const int slot = idx / 1024, wd = (idx / 64) % 16, l = idx % 64;
    int k0, k1;
    if (slot < 9) {
      k0 = 0;
      k1 = slot;
    } else if (slot < 17) {
      k0 = N1 / 2;
      k1 = slot - 9;
    } else {
      k0 = 1 + (slot - 17) / 16;
      k1 = (slot - 17) % 16;
    }
    const int q = wd & 7;
    const int base = k0 + N1 * (k1 + 16 * (l & 31));
    const float2 a = bin(base + N1 * 512 * acc_row(2 * q, l >> 5));
    const float2 b = bin(base + N1 * 512 * acc_row(2 * q + 1, l >> 5));
    out[idx] = wd < 8 ? pack2h(a.x * sc, b.x * sc) : pack2h(a.y * sc, b.y * sc);
  }
  if (threadIdx.x < 64)
    out[P::SLOTS * 1024 + threadIdx.x] =
        threadIdx.x == 0 ? (uint32_t)(__builtin_amdgcn_frexp_expf(1.0f / c) - 1) : 0u;
}

// ------------------------------------------------------------------ host side
namespace {

template <int N1>
hipError_t mfl_conv_launch(int order, int B, int D, const void* v, const void* const* x, const void* const* spectra,
                           void* y, uint32_t* W0, int chunk, const void* mats, const Twiddles& tw, hipStream_t s0,
                           const SideStream* side) {
  using P = mfl::Plan<N1>;
  const int pairs = (B / 2) * D;
  const int ways = (side != nullptr && pairs > chunk) ? side->ways : 1;
  if (ways > 1) {
    const hipError_t e = side_fork(side, s0);
    if (e != hipSuccess) return e;
  }
  const u32x4* mt = (const u32x4*)mats;
  const uint16_t* vv = (const uint16_t*)v;
  uint16_t* yy = (uint16_t*)y;
  int k = 0;
  for (int q0 = 0; q0 < pairs; q0 += chunk, ++k) {
    const int nq = (pairs - q0 < chunk) ? pairs - q0 : chunk;
    const int j = k % ways;
    const hipStream_t s = j ? side->s[j - 1] : s0;
    uint32_t* W = W0 + (size_t)j * chunk * P::PAIR_WORDS;
    const dim3 gc(mfl::NTILE * nq), gp((N1 / 2) * nq);
    hipLaunchKernelGGL((k_mfl_cols<N1, 0, false, false>), gc, dim3(mfl::TC), 0, s, vv, (const uint16_t*)nullptr,
                       (uint16_t*)nullptr, W, q0, nq, B, D, 0, tw);
    for (int i = 0; i < order; ++i) {
      hipLaunchKernelGGL((k_mfl_planes<N1>), gp, dim3(mfl::TP), 0, s, W, (const uint32_t*)spectra[i], mt, q0, nq, B);
      const uint16_t* g = (const uint16_t*)x[i];
      if (i + 1 < order)
        hipLaunchKernelGGL((k_mfl_cols<N1, 1, true, true>), gc, dim3(mfl::TC), 0, s, (const uint16_t*)nullptr, g,
                           (uint16_t*)nullptr, W, q0, nq, B, D, i & 1, tw);
      else if (g)
        hipLaunchKernelGGL((k_mfl_cols<N1, 1, true, false>), gc, dim3(mfl::TC), 0, s, (const uint16_t*)nullptr, g,
                           yy, W, q0, nq, B, D, i & 1, tw);
      else
        hipLaunchKernelGGL((k_mfl_cols<N1, 1, false, false>), gc, dim3(mfl::TC), 0, s, (const uint16_t*)nullptr,
                           (const uint16_t*)nullptr, yy, W, q0, nq, B, D, i & 1, tw);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return ways > 1 ? side_join(side, s0) : hipSuccess;
}

}  // namespace

bool mfl_supported(int log2L, int B) { return (log2L == 15 || log2L == 16) && B % 2 == 0; }

size_t mfl_pair_bytes(int log2L) {
  return ((size_t)2 << log2L) * 4 + (size_t)mfl::HDR * 4;
}

size_t mfl_spectrum_bytes_per_channel(int log2L) {
  return log2L == 15 ? (size_t)mfl::Plan<4>::SPEC_WORDS * 4 : (size_t)mfl::Plan<8>::SPEC_WORDS * 4;
}

hipError_t launch_conv_mfl(int log2L, int order, int B, int D, const void* v, const void* const* x,
                           const void* const* spectra, void* y, void* ws, int chunk_pairs, const void* mats,
                           const Twiddles& tw, hipStream_t s, const SideStream* side) {
  if (!mfl_supported(log2L, B) || order < 1 || chunk_pairs < 1) return hipErrorInvalidValue;
  if (log2L == 15)
    return mfl_conv_launch<4>(order, B, D, v, x, spectra, y, (uint32_t*)ws, chunk_pairs, mats, tw, s, side);
  return mfl_conv_launch<8>(order, B, D, v, x, spectra, y, (uint32_t*)ws, chunk_pairs, mats, tw, s, side);
}

hipError_t launch_mfl_spectrum(int log2L, const float2* Hnat, void* Hc, int D, hipStream_t s) {
  if (log2L == 15)
    hipLaunchKernelGGL(k_mfl_spectrum<4>, dim3(D), dim3(256), 0, s, Hnat, (uint32_t*)Hc);
  else if (log2L == 16)
    hipLaunchKernelGGL(k_mfl_spectrum<8>, dim3(D), dim3(256), 0, s, Hnat, (uint32_t*)Hc);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hyena
