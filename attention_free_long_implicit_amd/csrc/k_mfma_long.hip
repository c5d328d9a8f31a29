// Matrix-core causal long convolution for bf16 storage and long rows (L = 2^15, 2^16, 2^17), one row at a time.
//
// Operation: Hyena study note, steps 2-3 (long convolution with the implicit filter, gate); EulerStack
// "4. Hyena 상세", how it works 2 (FFT, elementwise product, inverse FFT); HyenaND summary, boundary handling
// (zero-pad to twice the size).  The real row u of L samples, zero-padded to 2L, is packed into M = L complex
// points z[n] = u[2n] + i u[2n+1] (zero for n >= M/2).  With Z = DFT_M(z) and H the 2L-point DFT of the filter,
// the packed spectrum of the padded product is
//
//   Z'[k] = A[k] Z[k] + B[k] conj(Z[M - k]),   A = Hs - Hd sin(pi k / M),  B = i Hd cos(pi k / M),
//   Hs = (H[k] + H[k + M]) / 2,  Hd = (H[k] - H[k + M]) / 2,
//
// (the usual split of a real transform into the transforms of its even and odd samples, the product, and the
// re-packing, folded into two coefficients per bin), and the inverse transform of Z' gives (h * u)[2n] +
// i (h * u)[2n+1].  A row is too long for one workgroup, so the transform is split four-step style,
// M = N1 x N2 with N2 = 16384 the matrix-core transform of the 8192-sample kernel:
//
//   n = m + N2 n0 (only n0 < N1/2 non-zero), k = k0 + N1 kappa,  W_M^{nk} = W_N1^{n0 k0} W_M^{m k0} W_N2^{m kappa}.
//
//   column pass (k_mfl_cols): for every column m, the N1-point DFT over n0 and the twiddle W_M^{m k0} -> plane
//       k0; in fp32, one thread per four consecutive columns.
//   plane pass (k_mfl_planes): every plane k0 is an N2-point sequence, transformed on the matrix cores with the
//       slab decomposition of the 8192-sample kernel (16 x 32 x 32; all 16 inputs of the first radix-16
//       product non-zero, all 16 outputs of the last one kept); the split above needs bin M - k, which lies in
//       plane N1 - k0 (mod N1), so a workgroup takes the planes k0 and N1 - k0 (0 and N1/2 together) and
//       exchanges the bins through LDS.
//   column pass again: conjugate twiddle, inverse N1-point DFT, keep n0 < N1/2 (the causal half), gate; for
//       every order but the last the same workgroup then runs the next order's forward column pass on the
//       gated values, so u_i never goes to memory.
//
// A row's planes live in the workspace as fp16 (11-bit significand), real and imaginary parts in separate
// planes, each block of values written by one workgroup scaled by a power of two (its exponent stored beside
// the planes; the reader scales back exactly), so every row keeps its own scale.
#include "engine.h"
#include "launch.h"
#include "mfma_core.h"

namespace hyena {

namespace mfl {
constexpr int N2 = 16384;                 // plane length
constexpr int TILE_C = 64;                // column pass: columns c .. c + 63 (mod 1024) for all 16 n1
constexpr int NTILE = 1024 / TILE_C;      // column tiles per row
constexpr int TC = 256;                   // column-pass threads: four consecutive columns each
constexpr int TP = 512;                   // plane-pass threads: two planes of four waves
// Per row: N1 planes of N2 fp16 real parts then N2 fp16 imaginary parts (M 32-bit words), then a header of
// HDR words: the column pass's tile exponents (H_EA + tile), the plane pass's plane exponents (H_EB + k0).
enum { H_EA = 0, H_EB = 32, HDR = 64 };
// tile exponent of an all-zero tile: below any real one (2^kNoExponent is 0 in fp32)
constexpr int kNoExponent = -4096;
template <int N1>
struct Plan {
  static_assert(N1 == 2 || N1 == 4 || N1 == 8, "L = 2^15, 2^16 or 2^17");
  static constexpr int M = N1 * N2;       // packed points per row = samples per row
  static constexpr int LOG2M = N1 == 2 ? 15 : (N1 == 4 ? 16 : 17);
  static constexpr size_t ROW_WORDS = (size_t)M + HDR;
  // split coefficients per channel: [plane][slab][32 words][64 lanes] (words 0..15: A, 16..31: B; in each,
  // 8 real-part pairs then 8 imaginary-part pairs), then a 64-word tail (word 0: log2 of the scale back)
  static constexpr int COEF_WORDS = N1 * 16 * 32 * 64;
  static constexpr int SPEC_WORDS = COEF_WORDS + 64;
};
}  // namespace mfl

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ----------------------------------------------------------------------------------------------
// Column pass.  MODE 0: forward from the bf16 input u (first order).  MODE 1: inverse of the planes, gate
// (GATE), then store y, or (CHAIN) the forward column pass of the next order on the gated values.
// grid.x = NTILE * nq (row fastest); thread t: n1 = t / 16, columns m = 64 tile + 4 (t % 16) + i + 1024 n1,
// i < 4: 8 consecutive samples of a row (16 bytes) and 4 consecutive values of a plane (8 bytes) per access.
template <int N1, int MODE, bool GATE, bool CHAIN>
__global__ void __launch_bounds__(mfl::TC)
k_mfl_cols(const uint16_t* u, const uint16_t* gate, uint16_t* y, uint32_t* W, int q0, int nq, int B, int D,
           Twiddles tw) {
  using namespace mfl;
  using P = Plan<N1>;
  constexpr int M = P::M, H = N1 / 2;
  __shared__ float red[TC / 64];
  const int t = threadIdx.x;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int rl = lb % nq, tile = lb / nq;
  const int q = q0 + rl;                     // rows visited channel-major: q = d B + b
  const size_t row = (size_t)(q % B) * D + q / B;
  uint32_t* const Wp = W + (size_t)rl * P::ROW_WORDS;
  uint16_t* const planes = reinterpret_cast<uint16_t*>(Wp);
  uint32_t* const hdr = Wp + M;
  const int m0 = TILE_C * tile + 4 * (t & 15) + 1024 * (t >> 4);

  float2 z[4][H];   // [column][n0]: samples 2n and 2n + 1 of the row
  if constexpr (MODE == 0) {
#pragma unroll
    for (int n0 = 0; n0 < H; ++n0) {
      const uint4 a = *reinterpret_cast<const uint4*>(u + row * M + 2 * (m0 + N2 * n0));
      z[0][n0] = make_float2(bf16_lo(a.x), bf16_hi(a.x));
      z[1][n0] = make_float2(bf16_lo(a.y), bf16_hi(a.y));
      z[2][n0] = make_float2(bf16_lo(a.z), bf16_hi(a.z));
      z[3][n0] = make_float2(bf16_lo(a.w), bf16_hi(a.w));
    }
  } else {
    uint2 re[N1], im[N1];
#pragma unroll
    for (int k0 = 0; k0 < N1; ++k0) {
      re[k0] = *reinterpret_cast<const uint2*>(planes + (size_t)k0 * 2 * N2 + m0);
      im[k0] = *reinterpret_cast<const uint2*>(planes + (size_t)k0 * 2 * N2 + N2 + m0);
    }
    uint4 g[H];
    if constexpr (GATE) {
#pragma unroll
      for (int n0 = 0; n0 < H; ++n0) g[n0] = *reinterpret_cast<const uint4*>(gate + row * M + 2 * (m0 + N2 * n0));
    }
    float eb[N1];   // the plane pass's scales back
#pragma unroll
    for (int k0 = 0; k0 < N1; ++k0) eb[k0] = __builtin_ldexpf(1.0f, (int)hdr[H_EB + k0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2 w = twiddle<P::LOG2M>(tw, uint32_t(m0 + i));
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
        float a = x[n0].x, b = x[n0].y;
        if constexpr (GATE) {
          const uint32_t gw = i == 0 ? g[n0].x : (i == 1 ? g[n0].y : (i == 2 ? g[n0].z : g[n0].w));
          a *= bf16_lo(gw);
          b *= bf16_hi(gw);
        }
        z[i][n0] = make_float2(a, b);
      }
    }
    if constexpr (!CHAIN) {
#pragma unroll
      for (int n0 = 0; n0 < H; ++n0) {
        uint4 o;
        o.x = f32x2_to_bf16x2_rne(z[0][n0].x, z[0][n0].y);
        o.y = f32x2_to_bf16x2_rne(z[1][n0].x, z[1][n0].y);
        o.z = f32x2_to_bf16x2_rne(z[2][n0].x, z[2][n0].y);
        o.w = f32x2_to_bf16x2_rne(z[3][n0].x, z[3][n0].y);
        *reinterpret_cast<uint4*>(y + row * M + 2 * (m0 + N2 * n0)) = o;
      }
      return;
    }
  }

  // forward column pass; the tile's scale from a bound: each output component is at most N1 times the largest
  // input component (N1 / 2 inputs, each component of a product with a unit twiddle at most twice as large)
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n0 = 0; n0 < H; ++n0) a = fmaxf(a, fmaxf(fabsf(z[i][n0].x), fabsf(z[i][n0].y)));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
  if ((t & 63) == 0) red[t >> 6] = a;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < TC / 64; ++k) a = fmaxf(a, red[k]);
  const int ex = h16_exponent((float)N1 * a);
  const float sc = __builtin_ldexpf(1.0f, -ex);
  // an all-zero tile records kNoExponent, so that it cannot set the row's common scale in the plane pass
  if (t == 0) hdr[H_EA + tile] = (uint32_t)(a > 0.0f ? ex : kNoExponent);
  uint32_t rw[N1][2], iw[N1][2];   // fp16 pairs of columns (0, 1) and (2, 3)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2 w = twiddle<P::LOG2M>(tw, uint32_t(m0 + i));
    float2 p[N1];
    twiddle_powers<N1>(w, p);
    float2 x[N1];
#pragma unroll
    for (int n0 = 0; n0 < H; ++n0) x[n0] = z[i][n0];
    dft<N1, false, true, false>(x);
#pragma unroll
    for (int k0 = 0; k0 < N1; ++k0) {
      const float2 v = cmul(x[k0], p[k0]);
      const uint32_t br = __builtin_bit_cast(uint16_t, (_Float16)(v.x * sc));
      const uint32_t bi = __builtin_bit_cast(uint16_t, (_Float16)(v.y * sc));
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
// Plane pass: workgroup = planes k0 = g and N1 - g of one row (g = 0: planes 0 and N1/2), 8 waves, one LDS
// plane each.  Waves 4q..4q+3 run pass 1 and pass 1' of plane q; in the slab passes wave w owns slabs w and
// w + 8 of both planes, with one set of matrix loads.  Steps (as in k_conv_mfma, the 8192-sample kernel):
//   pass 1   radix 16 over n1 (all 16 inputs) -> slab k1                                    | barrier
//   forward  pass 2 (radix 32, the slab's matrix), twiddle W_1024, pass 3 -> bins
//            kappa = k1 + 16 k2 + 512 k3, written back over the slab (k3 row, k2 column)  | barrier
//   split    Z' = A Z + B conj(Z[M - k]) for the wave's four slab units, the mirrored bins read from LDS
//            (plane N1 - k0, slab 15 - k1, k2 -> 31 - k2, k3 -> 31 - k3; in plane 0, slab 16 - k1, and
//            for its slab 0, k2 -> 32 - k2 and, where k2 = 0, k3 -> 32 - k3, all mod 32); kept in registers
//                                                                                         | barrier
//   inverse  pass 3', conjugate twiddle, pass 2' -> slab                                   | barrier
//   pass 1'  radix 16 over k1, all 16 outputs, stored as fp16.
//
// Scaling (all exact powers of two): the column pass's tiles have exponents e_A (kNoExponent for an all-zero
// tile); the plane's input is read as fp16 and its first product's accumulators are scaled by
// 2^(e_A - E - 17), E = max e_A, which keeps every
// input component below 1/4, the bins' magnitudes below 2^12.5 and the split's below 2^14 (fp16 holds 65504); the
// coefficient table holds c A / M and c B / M; the output block is stored as fp16 scaled by 2^-e', e' chosen
// from a bound (each output component is at most 32 times the largest value pass 2' leaves), with
// e_B = e' + 10 + log2(1/c) + E + 17 recorded for the column pass (the 10: the inverse matrices' 1/32 each).
template <int N1>
__global__ void __launch_bounds__(mfl::TP, 1)
k_mfl_planes(uint32_t* W, const uint32_t* __restrict__ spec, const u32x4* __restrict__ mats, int q0, int nq, int B) {
  using namespace mf;
  using P = mfl::Plan<N1>;
  constexpr int N2 = mfl::N2, NW = 8, G = N1 / 2;
  __shared__ uint32_t S[2 * PLANE];
  __shared__ float red[2 * NW];
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int rl = lb / G, g = lb % G;
  const int d = (q0 + rl) / B;
  uint32_t* const Wp = W + (size_t)rl * P::ROW_WORDS;
  uint16_t* const planes = reinterpret_cast<uint16_t*>(Wp);
  uint32_t* const hdr = Wp + P::M;
  const int mine = (int)(threadIdx.x >> 8);
  auto plane_of = [&](int qq) { return qq == 0 ? g : (g == 0 ? N1 / 2 : N1 - g); };

  const int t = threadIdx.x, w = t >> 6, wq = w & 3, l = t & 63, j = l & 31, h = l >> 5;
  const int c0 = 256 * wq + 8 * j;
  const int n2c = 8 * wq + (j >> 2), n3c = 8 * (j & 3);
  uint32_t* const Sm = S + mine * PLANE;
  uint16_t* const Pm = planes + (size_t)plane_of(mine) * 2 * N2;   // this group's plane (real parts first)

  // pass 1 input: lanes h = 0 / 1 carry the real / imaginary parts, n1 = e and 8 + e, 8 consecutive columns
  u32x4 VA[8], VB[8];
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
  int E = mfl::kNoExponent;
#pragma unroll
  for (int k = 0; k < mfl::NTILE; ++k) E = max(E, (int)hdr[mfl::H_EA + k]);
  const float f_in = __builtin_ldexpf(1.0f, (int)hdr[mfl::H_EA + (c0 >> 6)] - E - 17);
  const uint32_t* __restrict__ Hc = spec + (size_t)d * P::SPEC_WORDS;
  const int eH = (int)Hc[P::COEF_WORDS];

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
  const __amdgpu_buffer_rsrc_t crs =
      __builtin_amdgcn_make_buffer_rsrc((void*)Hc, (short)0, P::COEF_WORDS * 4, kRawBufferWord3);
  // the 32 coefficient words of plane qq's slab k1 (scalar) for this lane
  auto load_coef = [&](int qq, int k1s_, uint32_t (&c)[32]) {
    const int base = (plane_of(qq) * 16 + k1s_) * 32;
#pragma unroll
    for (int k = 0; k < 32; ++k) c[k] = __builtin_amdgcn_raw_buffer_load_b32(crs, l * 4, (base + k) * 256, 0);
  };
  const int ws = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  load_mat(ws, MF2, Ma);
  load_mat(ws, MF3, Mb);
  // pass 1: both halves of the radix-16 input, accumulators scaled into range
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

  // ---------------- forward: passes 2 and 3 of the wave's slabs, bins written back over each slab
  uint32_t cf[32];   // coefficients of the next split unit
  static_for<2>([&](auto itc) {
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
    if (it == 0) load_mat(k1s + NW, MF2, Ma);
    else load_mat(ws, MI3, Ma);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      f16x2 ar[8], ai[8];
      to_pairs(dr[q], ar);
      to_pairs(di[q], ai);
      cmul_pairs<false>(ar, ai, pc, ps, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q]);
      dft32<false, false>(Mb, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q], dr[q], di[q]);
    }
    if (it == 0) {
      load_mat(k1s + NW, MF3, Mb);
    } else {
      load_mat(ws, MI2, Mb);
      load_coef(0, ws, cf);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t* sl = S + q * PLANE + k1 * SLAB;
#pragma unroll
      for (int v = 0; v < 16; ++v) sl[acc_row(v, h) * ROW + j] = pack2h(dr[q][v], di[q][v]);
    }
  });
  __syncthreads();

  // ---------------- split: units (it, q) = plane q, slab w + 8 it; results kept as pass 3' operands
  f16x8 zr_lo[2][2], zr_hi[2][2], zi_lo[2][2], zi_hi[2][2];
  static_for<4>([&](auto uc) {
    constexpr int U = uc.value, it = U >> 1, q = U & 1;
    const int k1 = w + NW * it;
    const int qm = g == 0 ? q : 1 - q;                  // the plane holding the mirrored bins
    const bool p0 = plane_of(q) == 0, s0 = p0 && k1 == 0;   // (wave-uniform)
    const int k1m = p0 ? (16 - k1) & 15 : 15 - k1;
    const int k2m = s0 ? (32 - j) & 31 : 31 - j;
    const uint32_t* own = S + q * PLANE + k1 * SLAB + j;
    const uint32_t* mir = S + qm * PLANE + k1m * SLAB + k2m;
    uint32_t zw[16], mw[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int k3 = acc_row(v, h);
      const int k3m = (s0 && j == 0) ? (32 - k3) & 31 : 31 - k3;
      zw[v] = own[k3 * ROW];
      mw[v] = mir[k3m * ROW];
    }
    uint32_t c[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) c[k] = cf[k];
    if constexpr (U + 1 < 4) load_coef((U + 1) & 1, ws + NW * ((U + 1) >> 1), cf);
    // pairs of registers (2p, 2p + 1): real parts, imaginary parts
    u32x4 rl_, rh_, il_, ih_;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const f16x2 zr = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(zw[2 * p + 1], zw[2 * p], 0x05040100u));
      const f16x2 zi = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(zw[2 * p + 1], zw[2 * p], 0x07060302u));
      const f16x2 mr = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(mw[2 * p + 1], mw[2 * p], 0x05040100u));
      const f16x2 mi = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(mw[2 * p + 1], mw[2 * p], 0x07060302u));
      const uint32_t c0_ = c[p], c1_ = c[8 + p], c2_ = c[16 + p], c3_ = c[24 + p];
      const f16x2 ar = __builtin_bit_cast(f16x2, c0_), ai = __builtin_bit_cast(f16x2, c1_);
      const f16x2 br = __builtin_bit_cast(f16x2, c2_), bi = __builtin_bit_cast(f16x2, c3_);
      // A Z + B conj(Zm)
      const f16x2 re = __builtin_elementwise_fma(ar, zr, __builtin_elementwise_fma(-ai, zi,
                           __builtin_elementwise_fma(br, mr, bi * mi)));
      const f16x2 im = __builtin_elementwise_fma(ar, zi, __builtin_elementwise_fma(ai, zr,
                           __builtin_elementwise_fma(bi, mr, -(br * mi))));
      const uint32_t rb = __builtin_bit_cast(uint32_t, re), ib = __builtin_bit_cast(uint32_t, im);
      if (p < 4) {
        rl_[p] = rb;
        il_[p] = ib;
      } else {
        rh_[p - 4] = rb;
        ih_[p - 4] = ib;
      }
    }
    zr_lo[it][q] = as_h(rl_);
    zr_hi[it][q] = as_h(rh_);
    zi_lo[it][q] = as_h(il_);
    zi_hi[it][q] = as_h(ih_);
  });
  __syncthreads();

  // ---------------- inverse: passes 3' and 2' of the wave's slabs
  float vm[2] = {0.0f, 0.0f};   // largest |value| pass 2' leaves, per plane
  static_for<2>([&](auto itc) {
    constexpr int it = decltype(itc)::value;
    const int k1 = w + NW * it;
    const int k1s = ws + NW * it;
    f16x8 xr_lo[2], xr_hi[2], xi_lo[2], xi_hi[2];
    f32x16 dr[2], di[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
      dft32<true, true>(Ma, zr_lo[it][q], zr_hi[it][q], zi_lo[it][q], zi_hi[it][q], dr[q], di[q]);
    if (it == 0) load_mat(k1s + NW, MI3, Ma);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      f16x2 ar[8], ai[8];
      to_pairs(dr[q], ar);
      to_pairs(di[q], ai);
      cmul_pairs<true>(ar, ai, pc, ps, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q]);
      dft32<true, false>(Mb, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q], dr[q], di[q]);
    }
    if (it == 0) load_mat(k1s + NW, MI2, Mb);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t* sl = S + q * PLANE + k1 * SLAB;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        vm[q] = fmaxf(vm[q], fmaxf(fabsf(dr[q][v]), fabsf(di[q][v])));
        sl[acc_row(v, h) * ROW + j] = pack2h(dr[q][v], di[q][v]);
      }
    }
  });
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
  if ((threadIdx.x & 255) == 0) hdr[mfl::H_EB + plane_of(mine)] = (uint32_t)(eo + 10 + eH + E + 17);
}

// Split coefficients of the natural-order bins 0..L of the 2L-point filter spectrum: for plane k0, slab k1,
// word wd, lane l: words 0..15 hold A, 16..31 B; word 8 r + p of either holds the real (r = 0) or imaginary
// (r = 1) parts of c X[k(2p)] / M and c X[k(2p + 1)] / M as fp16 (register 2p low), k(v) = k0 + N1 (k1 + 16
// (l % 32) + 512 k3(v, l / 32)); then the tail, word 0 = log2(1/c).  c is the power of two that brings the
// largest component of A / M and B / M into [0.5, 1).
// A[k], B[k] from H[k] and H[k + M] = conj(H[M - k]) (k >= 1; H[M] itself for k = 0).
template <int N1>
__device__ __forceinline__ void mfl_coef(const float2* hn, const Twiddles& tw, int k, float2& A, float2& Bc) {
  constexpr int M = mfl::Plan<N1>::M;
  const float2 h0 = hn[k];
  const float2 h1 = k == 0 ? hn[M] : cconj(hn[M - k]);
  const float2 hs = make_float2(0.5f * (h0.x + h1.x), 0.5f * (h0.y + h1.y));
  const float2 hd = make_float2(0.5f * (h0.x - h1.x), 0.5f * (h0.y - h1.y));
  const float2 wk = twiddle<mfl::Plan<N1>::LOG2M + 1>(tw, uint32_t(k));   // cos(pi k / M) - i sin(pi k / M)
  const float cs = wk.x, sn = -wk.y;
  A = make_float2(hs.x - hd.x * sn, hs.y - hd.y * sn);
  Bc = make_float2(-hd.y * cs, hd.x * cs);
}

// The scale c of one channel per workgroup: the largest component over every bin's A and B (bins read in
// order); writes the tail.
template <int N1>
__global__ void __launch_bounds__(256) k_mfl_spec_scale(const float2* __restrict__ Hnat, uint32_t* __restrict__ Hc,
                                                        Twiddles tw) {
  using namespace mf;
  using P = mfl::Plan<N1>;
  constexpr int M = P::M;
  __shared__ float red[4];
  const int d = blockIdx.x;
  const float2* hn = Hnat + (size_t)d * (M + 1);
  float m = 0.0f;
  for (int k = threadIdx.x; k < M; k += 256) {
    float2 A, Bc;
    mfl_coef<N1>(hn, tw, k, A, Bc);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(A.x), fabsf(A.y)), fmaxf(fabsf(Bc.x), fabsf(Bc.y))));
  }
  const float c = range_scale(block_max4(m * (1.0f / M), red));
  uint32_t* out = Hc + (size_t)d * P::SPEC_WORDS;
  if (threadIdx.x < 64)
    out[P::COEF_WORDS + threadIdx.x] = threadIdx.x == 0 ? (uint32_t)(__builtin_amdgcn_frexp_expf(1.0f / c) - 1) : 0u;
}

// The coefficient words of one channel and one pair of accumulator rows (r, r + 1) per workgroup (sixteen per
// channel: rows 0..31).  Their bins k0 + N1 (k1 + 16 l' + 512 r'), r' = r, r + 1, fill one window of 1024 N1 consecutive
// bins, whose A and B go to LDS first (bins, their mirrors and twiddles read in order); the words then gather
// from LDS, the window padded by one element per 16 N1 so that the lanes, 16 N1 bins apart, hit distinct banks.
// Rows r, r + 1 are registers 2p, 2p + 1 of lane half h (r = 8 (p >> 1) + 4 h + 2 (p & 1)): words p, 8 + p,
// 16 + p and 24 + p of lanes 32 h .. 32 h + 31, every plane and slab.  Runs after k_mfl_spec_scale (reads c
// from the tail).
template <int N1>
__global__ void __launch_bounds__(256) k_mfl_spec_coef(const float2* __restrict__ Hnat, uint32_t* __restrict__ Hc,
                                                       Twiddles tw) {
  using namespace mf;
  using P = mfl::Plan<N1>;
  constexpr int M = P::M, NW = 1024 * N1, S = 16 * N1, NWP = NW + NW / S + 1;
  __shared__ float2 cA[NWP], cB[NWP];
  const int d = blockIdx.x >> 4, r = 2 * (blockIdx.x & 15);
  const int p = 2 * (r >> 3) + ((r >> 1) & 1), h = (r >> 2) & 1;
  const int W0 = 512 * N1 * r;
  const float2* hn = Hnat + (size_t)d * (M + 1);
  uint32_t* out = Hc + (size_t)d * P::SPEC_WORDS;
  for (int i = threadIdx.x; i < NW; i += 256) {
    float2 A, Bc;
    mfl_coef<N1>(hn, tw, W0 + i, A, Bc);
    cA[i + i / S] = A;
    cB[i + i / S] = Bc;
  }
  const int e = (int)out[P::COEF_WORDS];                  // log2(1/c), from k_mfl_spec_scale
  const float sc = ldexpf(1.0f, -e) * (1.0f / M);
  __syncthreads();
  for (int it = threadIdx.x; it < N1 * 16 * 32; it += 256) {
    const int lq = it & 31, unit = it >> 5;
    const int k0 = unit >> 4, k1 = unit & 15;
    const int i0 = k0 + N1 * (k1 + 16 * lq), i1 = i0 + 512 * N1;
    const float2 a0 = cA[i0 + i0 / S], b0 = cB[i0 + i0 / S], a1 = cA[i1 + i1 / S], b1 = cB[i1 + i1 / S];
    uint32_t* o = out + (size_t)unit * 2048 + 32 * h + lq;
    o[p * 64] = pack2h(a0.x * sc, a1.x * sc);
    o[(8 + p) * 64] = pack2h(a0.y * sc, a1.y * sc);
    o[(16 + p) * 64] = pack2h(b0.x * sc, b1.x * sc);
    o[(24 + p) * 64] = pack2h(b0.y * sc, b1.y * sc);
  }
}

// ------------------------------------------------------------------ host side
namespace {

template <int N1>
hipError_t mfl_conv_launch(int order, int B, int D, const void* v, const void* const* x, const void* const* spectra,
                           void* y, uint32_t* W0, int chunk, const void* mats, const Twiddles& tw, hipStream_t s0,
                           const SideStream* side) {
  using P = mfl::Plan<N1>;
  const int rows = B * D;
  const int ways = (side != nullptr && rows > chunk) ? side->ways : 1;
  if (ways > 1) {
    const hipError_t e = side_fork(side, s0);
    if (e != hipSuccess) return e;
  }
  const u32x4* mt = (const u32x4*)mats;
  const uint16_t* vv = (const uint16_t*)v;
  uint16_t* yy = (uint16_t*)y;
  int k = 0;
  for (int q0 = 0; q0 < rows; q0 += chunk, ++k) {
    const int nq = (rows - q0 < chunk) ? rows - q0 : chunk;
    const int j = k % ways;
    const hipStream_t s = j ? side->s[j - 1] : s0;
    uint32_t* W = W0 + (size_t)j * chunk * P::ROW_WORDS;
    const dim3 gc(mfl::NTILE * nq), gp((N1 / 2) * nq);
    hipLaunchKernelGGL((k_mfl_cols<N1, 0, false, false>), gc, dim3(mfl::TC), 0, s, vv, (const uint16_t*)nullptr,
                       (uint16_t*)nullptr, W, q0, nq, B, D, tw);
    for (int i = 0; i < order; ++i) {
      hipLaunchKernelGGL((k_mfl_planes<N1>), gp, dim3(mfl::TP), 0, s, W, (const uint32_t*)spectra[i], mt, q0, nq, B);
      const uint16_t* g = (const uint16_t*)x[i];
      if (i + 1 < order)
        hipLaunchKernelGGL((k_mfl_cols<N1, 1, true, true>), gc, dim3(mfl::TC), 0, s, (const uint16_t*)nullptr, g,
                           (uint16_t*)nullptr, W, q0, nq, B, D, tw);
      else if (g)
        hipLaunchKernelGGL((k_mfl_cols<N1, 1, true, false>), gc, dim3(mfl::TC), 0, s, (const uint16_t*)nullptr, g,
                           yy, W, q0, nq, B, D, tw);
      else
        hipLaunchKernelGGL((k_mfl_cols<N1, 1, false, false>), gc, dim3(mfl::TC), 0, s, (const uint16_t*)nullptr,
                           (const uint16_t*)nullptr, yy, W, q0, nq, B, D, tw);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return ways > 1 ? side_join(side, s0) : hipSuccess;
}

}  // namespace

bool mfl_supported(int log2L) { return log2L >= 15 && log2L <= 17; }

size_t mfl_row_bytes(int log2L) { return (((size_t)1 << log2L) + mfl::HDR) * 4; }

size_t mfl_spectrum_bytes_per_channel(int log2L) {
  switch (log2L) {
    case 15: return (size_t)mfl::Plan<2>::SPEC_WORDS * 4;
    case 16: return (size_t)mfl::Plan<4>::SPEC_WORDS * 4;
    case 17: return (size_t)mfl::Plan<8>::SPEC_WORDS * 4;
  }
  return 0;
}

hipError_t launch_conv_mfl(int log2L, int order, int B, int D, const void* v, const void* const* x,
                           const void* const* spectra, void* y, void* ws, int chunk_rows, const void* mats,
                           const Twiddles& tw, hipStream_t s, const SideStream* side) {
  if (!mfl_supported(log2L) || order < 1 || chunk_rows < 1) return hipErrorInvalidValue;
  uint32_t* W = (uint32_t*)ws;
  switch (log2L) {
    case 15: return mfl_conv_launch<2>(order, B, D, v, x, spectra, y, W, chunk_rows, mats, tw, s, side);
    case 16: return mfl_conv_launch<4>(order, B, D, v, x, spectra, y, W, chunk_rows, mats, tw, s, side);
    default: return mfl_conv_launch<8>(order, B, D, v, x, spectra, y, W, chunk_rows, mats, tw, s, side);
  }
}

hipError_t launch_mfl_spectrum(int log2L, const float2* Hnat, void* Hc, int D, const Twiddles& tw, hipStream_t s) {
  auto go = [&](auto scale, auto coef) {
    hipLaunchKernelGGL(scale, dim3(D), dim3(256), 0, s, Hnat, (uint32_t*)Hc, tw);
    hipLaunchKernelGGL(coef, dim3(16 * D), dim3(256), 0, s, Hnat, (uint32_t*)Hc, tw);
  };
  switch (log2L) {
    case 15: go(k_mfl_spec_scale<2>, k_mfl_spec_coef<2>); break;
    case 16: go(k_mfl_spec_scale<4>, k_mfl_spec_coef<4>); break;
    case 17: go(k_mfl_spec_scale<8>, k_mfl_spec_coef<8>); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hyena
