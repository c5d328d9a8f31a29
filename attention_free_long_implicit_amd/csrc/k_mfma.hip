// Matrix-core (MFMA) causal long convolution for bf16 storage, L = 8192, rows taken in pairs.
//
// Operation: Hyena study note, steps 2-3 (long convolution with the implicit filter, gate);
// EulerStack "4. Hyena 상세", how it works 2 (FFT, elementwise product, inverse FFT); HyenaND summary,
// boundary handling (zero-pad to twice the size) and nSubQ implementation (forward transform,
// spectral product, inverse transform and output cut in one kernel, intermediates on chip).  The
// transform steps are small dense DFT matrices, evaluated as 16-bit matrix products with fp32
// accumulation (a DFT as a dense matrix product is the remark in the SPECTRE digest's comments).
//
// Precision: every operand after the first product is fp16 (11-bit significand), not bf16 (8 bits):
// the products cost the same on the matrix cores, and eight times finer rounding keeps the order-2
// result well inside the bf16-storage tolerance even without a decay window (bf16 operands measured
// up to 1.96e-2 of the 2e-2 allowed).  fp16's range is kept by exact power-of-two scaling: each row of each
// order's input is scaled so that its largest magnitude lies in [0.5, 1) (one scale per row, not per pair:
// the transform mixes the two rows, and a row far smaller than its partner would otherwise be resolved only
// to the partner's rounding level), the filter spectrum so that its largest bin does, and the inverse
// radix-32 matrices carry a factor 1/32 each, so no intermediate exceeds 2^13; the output is scaled back in
// fp32 before the gate, and a row that is all zeros gives exact zeros.  The first product of the first order
// reads the bf16 inputs exactly, against a matrix split into two bf16 parts (hi + lo) times the row scales.
// The two elementwise steps between products (the twiddle W_1024 and the spectral product) take the
// accumulators rounded to fp16 and multiply them in packed fp16 arithmetic, two complex values per
// instruction, with twiddles and spectrum already stored as fp16 pairs; the result is the next product's
// operand as it stands (two more roundings per step than an fp32 product, which moved the order-2 error on
// the 8192-sample workload from 2.4e-3 to 2.8e-3, for a third fewer vector instructions).
//
// Two rows b0, b1 of one channel (same filter) are transformed together as z = u_b0 + i u_b1:
// since h is real, IDFT(DFT(z) H) = (h * u_b0) + i (h * u_b1), so no real-input split is needed.
// N = 2L = 16384 = 16 x 32 x 32, n = n3 + 32 n2 + 1024 n1 (n1 < 8 nonzero), k = k1 + 16 k2 + 512 k3, and
//   W_N^{nk} = W_16^{n1 k1} . W_512^{n2 (16 k2 + k1)} . W_1024^{n3 k2} . W_N^{n3 (512 k3 + k1)}.
//   pass 1  DFT over n1 (radix 16, half the inputs zero) -> slab k1
//   pass 2  over n2 with the slab's matrix W_512^{n2 (16 k2 + k1)}, then twiddle W_1024^{n3 k2}
//   pass 3  over n3 with the slab's matrix W_N^{n3 (512 k3 + k1)} -> Z[k]; times H[k]/N
//   pass 3' inverse of pass 3 straight from the accumulators (the matrix's input order is the
//           accumulator row order), conj twiddle W_1024^{n3 k2}
//   pass 2' inverse of pass 2
//   pass 1' inverse DFT over k1, keep n1 < 8 (the causal half); gate; store
// Every factor that depends on the slab k1 and on one of a pass's own indices lives in that pass's
// matrix (16 slabs x 4 matrices, a 256 KB table that stays in L2), so the only elementwise twiddle
// left is W_1024^{n3 k2}, whose two indices are the row and the column of one product.  The filter
// spectrum is stored for slabs 0..8 only (36 KB per channel, plus its scale); conjugate symmetry gives the
// rest.
// A complex radix-R DFT is a real 2R x 2R matrix on (Re, Im); each MFMA (32x32x16) multiplies a 32-row
// block of it by 32 columns (independent sub-transforms).  LDS holds one plane of complex fp16 words
// (re low, im high); rows hold 32 words plus one pad, so lanes reading one word each from 32
// consecutive rows, or 32 consecutive words of one row, hit distinct banks.  Passes 2, 3, 3' and 2'
// of slab k1 touch only that slab, which one wave owns, so only two barriers are needed.  Global
// memory is touched in 16-byte accesses only: pass 1 and pass 1' give each lane 8 tiles whose columns
// are 8 consecutive samples.
#include <math.h>
#include <string.h>

#include <type_traits>

#include "engine.h"
#include "launch.h"
#include "mfma_core.h"

namespace hyena {

// Orders run back to back in one launch: gate and matrix-core spectrum copy of each order.
struct MfmaChain {
  const __bf16* gate[kMfmaMaxChain];
  const uint32_t* spectrum[kMfmaMaxChain];
  int order;
};

// Workgroups of NP x 4 waves take NP row pairs of one channel (NP = 2 when a channel has an even number of
// row pairs): each wave's passes 1 and 1' serve its own pair, and in passes 2..2' a wave transforms its
// slabs for every pair of the workgroup with one set of matrix and spectrum loads.
// Pass 1 / pass 1' column mapping: wave w (of its pair's four), lane j (= lane % 32), tile t handle column
// c = 256 w + 8 j + t (n3 = c % 32, n2 = c / 32), so each lane's 8 tiles cover 8 consecutive samples: one
// 16-byte access per (row, n1) in global memory.
template <bool GATE, int NP>
__global__ void __launch_bounds__(mf::T * NP, 2 / NP)
k_conv_mfma(const __bf16* u, __bf16* y, MfmaChain ch, const u32x4* __restrict__ mats, int B, int D) {
  using namespace mf;
  static_assert(NP == 1 || NP == 2, "one or two row pairs per workgroup");
  constexpr int NW = 4 * NP;        // waves; wave w owns slabs k1 = w + NW it, it < NIT
  constexpr int NIT = 16 / NW;
  __shared__ uint32_t S[NP * PLANE];
  __shared__ float red[2 * NW];
  const int ngrp = (B >> 1) / NP;   // workgroups per channel
  const int r = xcd_logical_block(blockIdx.x, D * ngrp);
  const int d = r / ngrp;
  const int mine = (int)(threadIdx.x >> 8);   // this wave's pair (passes 1 and 1')
  const int p = (r % ngrp) * NP + mine;
  const size_t row0 = (size_t)(2 * p) * D + d, row1 = (size_t)(2 * p + 1) * D + d;

  // pass 1 input of the first order: lanes h = 0 / 1 carry row b0 / b1 (real / imaginary input), n1 = e
  u32x4 V[8];
  {
    const int l = threadIdx.x & 63, c0 = 256 * ((threadIdx.x >> 6) & 3) + 8 * (l & 31);
    const __bf16* src = ((l >> 5) == 0 ? u + row0 * L : u + row1 * L) + c0;
#pragma unroll
    for (int e = 0; e < 8; ++e) V[e] = *reinterpret_cast<const u32x4*>(src + 1024 * e);
  }
  // Order-independent operands, loaded once right behind the first input (inside the order loop they
  // would queue behind that order's spectrum loads): the fixed radix-16 matrices and the per-lane
  // twiddles W_1024^{j k(v)}, k(v) = row of accumulator v.
  const int l0 = threadIdx.x & 63;
  // m1a, m1b: the forward radix-16 matrix of the next pass 1 (first order: its two bf16 parts; later
  // orders: m1a in fp16, loaded at the end of the previous order)
  u32x4 m1a = mats[M1F_HI * 64 + l0], m1b = mats[M1F_LO * 64 + l0];
  const u32x4 m1r = mats[M1I_R * 64 + l0], m1i = mats[M1I_I * 64 + l0];
  // as fp16 pairs (real parts, imaginary parts) in accumulator order
  f16x2 pc[8], ps[8];
  {
    const u32x4 c0 = mats[TW_C0 * 64 + l0], c1 = mats[TW_C1 * 64 + l0];
    const u32x4 s0 = mats[TW_S0 * 64 + l0], s1 = mats[TW_S1 * 64 + l0];
    // (each element goes through a scalar: this compiler's __builtin_bit_cast of a subscripted vector
    // element reads element 0 whatever the subscript)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = c0[q], b = c1[q], e = s0[q], f = s1[q];
      pc[q] = __builtin_bit_cast(f16x2, a);
      pc[4 + q] = __builtin_bit_cast(f16x2, b);
      ps[q] = __builtin_bit_cast(f16x2, e);
      ps[4 + q] = __builtin_bit_cast(f16x2, f);
    }
  }
  // Scales of the first order's input, one per row: each row's largest |u| (bf16 magnitudes compare as
  // integers) brought into [0.5, 1), so that each row of the pair keeps its own range (the transform mixes
  // the two rows: with one scale for both, a row much smaller than its partner would be resolved only to
  // the partner's rounding level).  The row scale of lane half h goes into the first product's matrix: its
  // lanes h carry the inputs K = 8h .. 8h + 7 of row h, and the bf16 parts times a power of two stay exact.
  // A row that is all zeros gives exact zeros (its scale back is 0).
  float s0, s1, k0, k1;   // row scales; 1, or 0 for a row that is all zeros
  {
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = V[e][q] & 0x7fff7fffu;
        m = max(m, max(w & 0xffffu, w >> 16));
      }
    float m0, m1;
    block_max4_rows(__uint_as_float(m << 16), red, m0, m1);
    s0 = range_scale(m0);
    s1 = range_scale(m1);
    k0 = m0 != 0.0f ? 1.0f : 0.0f;
    k1 = m1 != 0.0f ? 1.0f : 0.0f;
    const float sl = (l0 >> 5) ? s1 : s0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m1a[q] = pack2(lo_f32(m1a[q]) * sl, hi_f32(m1a[q]) * sl);
      m1b[q] = pack2(lo_f32(m1b[q]) * sl, hi_f32(m1b[q]) * sl);
    }
  }

  for (int ord = 0; ord < ch.order; ++ord) {
  // lane constants derived from an opaque copy of the thread id, so nothing is hoisted across orders
  int tq = threadIdx.x;
  asm volatile("" : "+v"(tq));
  const int t = tq, w = t >> 6, wq = w & 3, l = t & 63, j = l & 31, h = l >> 5;
  const int c0 = 256 * wq + 8 * j;
  const int n2c = 8 * wq + (j >> 2), n3c = 8 * (j & 3);   // tile t: n2 = n2c, n3 = n3c + t
  uint32_t* const Sm = S + (w >> 2) * PLANE;                // this wave's pair's plane
  const uint32_t* __restrict__ Hc = ch.spectrum[ord] + (size_t)d * PAIR_STRIDE;
  const __bf16* gate = ch.gate[ord];
  // scales back: the inverse matrices' 1/1024, the spectrum's normalisation, the input's scale
  const float f_h = INV_SCALE * __builtin_bit_cast(float, Hc[PAIR_WORDS]);
  const float f_out0 = f_h * k0 / s0, f_out1 = f_h * k1 / s1;

  // Slab matrices rotate through two buffers, each load issued one pass before its use:
  // Ma = pass 2, Mb = pass 3, then Ma = pass 3', Mb = pass 2', then the next slab's pass 2 and 3.
  // The first slab's matrices and filter spectrum are in flight during pass 1.
  f16x8 Ma[NBLK], Mb[NBLK];
  // The matrix table and the spectrum are read through buffer descriptors: the per-lane part of the
  // offset is fixed, the block / register part (and the mirror choice, uniform per wave) stays in
  // scalar registers, so a slab's 32 loads cost no vector instructions for their addresses.
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(mats + NFIX * 64), (short)0, 16 * SLAB_TABLE * 64 * 16, kRawBufferWord3);
  const int mvo = l * 16;
  // blocks of matrix `which` of slab k1s (scalar) into M
  auto load_mat = [&](int k1s_, int which, f16x8 (&M)[NBLK]) {
#pragma unroll
    for (int b = 0; b < NBLK; ++b)
      M[b] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                           mrs, mvo, ((k1s_ * SLAB_TABLE + which * NBLK + b) * 64) * 16, 0));
  };
  // Filter spectrum: only slabs 0..8 are stored, as fp16 pairs in accumulator order (word q < 8: the real
  // parts of registers 2q, 2q + 1; word 8 + q: their imaginary parts).  h is real, so H[N - k] = conj(H[k]);
  // bin N - k of slab k1 > 8 is register 15 - v of lane 63 - l in slab 16 - k1: pair q of a mirrored slab
  // is pair 7 - q of lane 63 - l with its halves swapped and the imaginary parts negated; the swap and
  // the sign are applied where the value is used, so the load stays in flight until then.
  uint32_t hw[16];
  const __amdgpu_buffer_rsrc_t hrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)Hc, (short)0, PAIR_WORDS * 4, kRawBufferWord3);
  const int ws = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto load_spectrum = [&](int k1) {
    const bool mirror = k1 > 8;
    const int slab = (mirror ? 16 - k1 : k1) * (16 * 64 * 4);
    const int vo = (mirror ? 63 - l : l) * 4;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      hw[k] = __builtin_amdgcn_raw_buffer_load_b32(hrs, vo, slab + (mirror ? (k < 8 ? 7 - k : 23 - k) : k) * 256, 0);
  };
  load_mat(ws, MF2, Ma);
  load_mat(ws, MF3, Mb);
  load_spectrum(ws);
  // pass 1.  First order: the bf16 inputs exactly, against the forward matrix in two bf16 parts (scaled by
  // the row scales).  Later orders: the scaled fp16 input against the fp16 matrix.
  auto pass1 = [&](auto first) {
    static_for<8>([&](auto tt) {
      constexpr int TT = tt.value;
      const f32x16 z = {};
      f32x16 D1;
      if constexpr (decltype(first)::value) {
        const bf16x8 col = as_b(column8<TT>(V));
        D1 = mfma(as_b(m1a), col, z);
        D1 = mfma(as_b(m1b), col, D1);
      } else {
        D1 = mfma(as_h(m1a), as_h(column8<TT>(V)), z);
      }
      // rows k1 = acc_row(e, h): real part in D1[e], imaginary part in D1[8 + e]
#pragma unroll
      for (int e = 0; e < 8; ++e)
        Sm[acc_row(e, h) * SLAB + n2c * ROW + n3c + TT] = pack2h(D1[e], D1[8 + e]);
    });
  };
  if (ord == 0) pass1(std::true_type{});
  else pass1(std::false_type{});
  __syncthreads();

  // ---------------- passes 2, 3, 3', 2' per slab k1, for each pair of the workgroup
  u32x4 G[2][4];
  auto load_gate = [&]() {
    if (GATE) {
      const __bf16* g0 = gate + row0 * L + c0;
      const __bf16* g1p = gate + row1 * L + c0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        G[0][e] = *reinterpret_cast<const u32x4*>(g0 + 1024 * (4 * h + e));
        G[1][e] = *reinterpret_cast<const u32x4*>(g1p + 1024 * (4 * h + e));
      }
    }
  };
  auto slab_step = [&](auto itc) {
    constexpr int it = decltype(itc)::value;
    const int k1 = w + NW * it;
    const int k1s = ws + NW * it;   // the same slab index, in a scalar register
    f16x8 xr_lo[NP], xr_hi[NP], xi_lo[NP], xi_hi[NP];
    f32x16 dr[NP], di[NP];
    // pass 2: data on A (rows n3 = j, K = n2 from LDS: element (n2, n3) at n2 * ROW + n3), matrix on B
    //   -> lane = k2, registers = n3 (row of v)
#pragma unroll
    for (int q = 0; q < NP; ++q) {
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
    // twiddle W_1024^{n3 k2} (k2 = j, n3 = row of v); pass 3: matrix on A (rows k3, input n3 in accumulator
    // order), data on B -> lane = k2, registers = k3
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      f16x2 ar[8], ai[8];
      to_pairs(dr[q], ar);
      to_pairs(di[q], ai);
      cmul_pairs<false>(ar, ai, pc, ps, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q]);
      dft32<false, false>(Mb, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q], dr[q], di[q]);
    }
    load_mat(k1s, MI2, Mb);
    // spectral product: bin k1 + 16 j + 512 k3(v); Hc holds H/N (normalised) in this exact order.
    {
      f16x2 hr[8], hi[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        hr[q] = __builtin_bit_cast(f16x2, hw[q]);
        hi[q] = __builtin_bit_cast(f16x2, hw[8 + q]);
      }
      auto product = [&](auto conj) {
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          f16x2 ar[8], ai[8];
          to_pairs(dr[q], ar);
          to_pairs(di[q], ai);
          cmul_pairs<decltype(conj)::value>(ar, ai, hr, hi, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q]);
        }
      };
      if (k1s > 8) {   // wave-uniform: mirrored slab, conj(H) with the pair halves swapped
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          hr[q] = hr[q].yx;
          hi[q] = hi[q].yx;
        }
        product(std::true_type{});
      } else {
        product(std::false_type{});
      }
    }
    if (it + 1 < NIT) load_spectrum(k1s + NW);
    else if (NP == 2) load_gate();   // (two pairs leave no registers for it before the spectrum is used)
    // pass 3': data on A (rows k2 = j, input k3 in accumulator order), matrix on B -> lane = n3,
    // registers = k2
#pragma unroll
    for (int q = 0; q < NP; ++q) dft32<true, true>(Ma, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q], dr[q], di[q]);
    if (it + 1 < NIT) load_mat(k1s + NW, MF2, Ma);
    // conj twiddle W_1024^{n3 k2} (n3 = j, k2 = row of v); pass 2': matrix on A (rows n2, input k2 in
    // accumulator order), data on B -> lane = n3, registers = n2; store (n2, n3) at n2 * ROW + n3
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      f16x2 ar[8], ai[8];
      to_pairs(dr[q], ar);
      to_pairs(di[q], ai);
      cmul_pairs<true>(ar, ai, pc, ps, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q]);
      dft32<true, false>(Mb, xr_lo[q], xr_hi[q], xi_lo[q], xi_hi[q], dr[q], di[q]);
    }
    if (it + 1 < NIT) load_mat(k1s + NW, MF3, Mb);
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      uint32_t* sl = S + q * PLANE + k1 * SLAB;
#pragma unroll
      for (int v = 0; v < 16; ++v) sl[acc_row(v, h) * ROW + j] = pack2h(dr[q][v], di[q][v]);
    }
  };
  // The gate for pass 1' is issued before the last slab, behind that slab's matrix and spectrum loads
  // (the vector-memory counter retires in order, so no earlier slab waits on it): lane keeps rows
  // b0 / b1 at n1 = 4h + e (e < 4), 8 consecutive samples each.
  static_for<NIT>([&](auto itc) {
    if constexpr (decltype(itc)::value == NIT - 1 && NP == 1) load_gate();
    slab_step(itc);
  });

  __syncthreads();

  // ---------------- pass 1': tiles t, column c = c0 + t, K = k1 (slab index), outputs n1 = 4h + e
  {
    const bool last = ord + 1 == ch.order;
    float yv[2][4][8];   // [row][e][tile], fp32: the output, or the next order's input
    float vmax0 = 0.0f, vmax1 = 0.0f;
    // the tiles, and (when another order follows) the largest |value| for its input scale
    auto tiles = [&](auto chain) {
    static_for<8>([&](auto tt) {
      constexpr int TT = tt.value;
      uint32_t cw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cw[e] = Sm[(8 * h + e) * SLAB + n2c * ROW + n3c + TT];
      f16x8 xr, xi;
      split8(cw, xr, xi);
      const f32x16 z = {};
      f32x16 o = mfma(as_h(m1r), xr, z);
      o = mfma(as_h(m1i), xi, o);
      // rows 4h + e (e < 4): real part (row b0) in o[e], imaginary part (row b1) in o[8 + e]
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a = o[e], b = o[8 + e];   // times f_out0 / f_out1 (powers of two, or 0) is the result
        if (GATE) {
          a *= elem_f32<TT>(G[0][e]);
          b *= elem_f32<TT>(G[1][e]);
        }
        yv[0][e][TT] = a;
        yv[1][e][TT] = b;
        if constexpr (decltype(chain)::value) {
          vmax0 = fmaxf(vmax0, fabsf(a));
          vmax1 = fmaxf(vmax1, fabsf(b));
        }
      }
    });
    };
    __bf16* y0 = y + row0 * L + c0;
    __bf16* y1 = y + row1 * L + c0;
    if (last) {
      tiles(std::false_type{});
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32x4 Y0, Y1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          Y0[q] = pack2(yv[0][e][2 * q] * f_out0, yv[0][e][2 * q + 1] * f_out0);
          Y1[q] = pack2(yv[1][e][2 * q] * f_out1, yv[1][e][2 * q + 1] * f_out1);
        }
        *reinterpret_cast<u32x4*>(y0 + 1024 * (4 * h + e)) = Y0;
        *reinterpret_cast<u32x4*>(y1 + 1024 * (4 * h + e)) = Y1;
      }
    } else {
      tiles(std::true_type{});
      // u_i stays on chip: the next order's input, each row scaled into fp16's range by its own maximum
      // (the barrier inside block_max4x2 also keeps the next pass 1 from writing LDS this pass still reads).
      // Pass 1' left lane (j, h) with rows b0, b1 at n1 = 4h + e; the next pass 1 wants row b_h at
      // n1 = 0..7 in lane (j, h).  One cross-half swap per register does it: swapping the upper half of the
      // row-b0 register with the lower half of the row-b1 register leaves [b0 from lanes 0..31, b1 from
      // lanes 0..31] (n1 = e) in the first and [b0 from lanes 32..63, b1 from lanes 32..63] (n1 = 4 + e) in
      // the second.
      m1a = mats[M1F_H * 64 + l0];
      float m0, m1;
      block_max4x2(vmax0 * f_out0, vmax1 * f_out1, red, m0, m1);
      s0 = range_scale(m0);
      s1 = range_scale(m1);
      k0 = m0 != 0.0f ? 1.0f : 0.0f;
      k1 = m1 != 0.0f ? 1.0f : 0.0f;
      // powers of two: each row of u_i scaled into [0.5, 1) in one exact product
      const float c0 = f_out0 * s0, c1 = f_out1 * s1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t a = pack2h(yv[0][e][2 * q] * c0, yv[0][e][2 * q + 1] * c0);
          const uint32_t b = pack2h(yv[1][e][2 * q] * c1, yv[1][e][2 * q + 1] * c1);
          const auto rr = __builtin_amdgcn_permlane32_swap(a, b, false, false);
          V[e][q] = rr[0];
          V[4 + e][q] = rr[1];
        }
      }
    }
  }
  }
}


// Pair-order spectrum of one channel per workgroup: for k1 = 0..8 (the convolution kernel mirrors slabs
// 9..15 from slabs 7..1), Hc[d][k1][q][lane] = the real parts of c_d H[k(2q)]/N and c_d H[k(2q + 1)]/N as fp16
// (register 2q low), Hc[d][k1][8 + q][lane] their imaginary parts, k(v) = k1 + 16 (lane%32) + 512 k3(v, lane/32);
// then the float 1/c_d.  c_d is the power of two that brings the channel's largest |H[k]|/N into [0.5, 1).
// H from the natural-order bins 0..L (upper bins by conjugate symmetry).
__global__ void __launch_bounds__(256) k_pair_spectrum(const float2* __restrict__ Hnat, uint32_t* __restrict__ Hc) {
  using namespace mf;
  __shared__ float red[4];
  // the channel's bins, read once, coalesced; the copy below gathers them from LDS.  Bin k sits at
  // k + k / 16: the gather's lanes step 16 bins apart, which the padding spreads over distinct banks.
  __shared__ float2 hb[L + 1 + (L >> 4) + 1];
  const int d = blockIdx.x;
  const float2* hn = Hnat + (size_t)d * (L + 1);
  float m = 0.0f;
  for (int k = threadIdx.x; k <= L; k += 256) {
    const float2 v = hn[k];
    hb[k + (k >> 4)] = v;
    m = fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y)));
  }
  const float c = range_scale(block_max4(m * (1.0f / N), red));   // (its barrier also publishes hb)
  const float sc = c * (1.0f / N);
  uint32_t* out = Hc + (size_t)d * PAIR_STRIDE;
  auto bin = [&](int k) {
    const int j = k <= L ? k : N - k;
    const float2 v = hb[j + (j >> 4)];
    return k <= L ? v : cconj(v);
  };
  for (int idx = threadIdx.x; idx < PAIR_WORDS; idx += 256) {   // (k1, word, lane)
    const int k1 = idx / (16 * 64), wd = (idx / 64) % 16, l = idx % 64;
    const int q = wd & 7;
    const float2 a = bin(k1 + 16 * (l & 31) + 512 * acc_row(2 * q, l >> 5));
    const float2 b = bin(k1 + 16 * (l & 31) + 512 * acc_row(2 * q + 1, l >> 5));
    out[idx] = wd < 8 ? pack2h(a.x * sc, b.x * sc) : pack2h(a.y * sc, b.y * sc);
  }
  if (threadIdx.x < 64) out[PAIR_WORDS + threadIdx.x] = threadIdx.x == 0 ? __float_as_uint(1.0f / c) : 0u;
}

// ------------------------------------------------------------------ host side
namespace {
constexpr double kTwoPi = 2.0 * 3.14159265358979323846;

// input order of the matrices that read accumulators (passes 3, 3', 2'): K' (register order of the
// previous product's output rows) -> index
int perm_k3(int Kp) {
  const int hh = (Kp >> 3) & 1, e = Kp & 7, hi = Kp >> 4;
  return 16 * hi + (e < 4 ? 4 * hh + e : 8 + 4 * hh + e - 4);
}

// Radix-16 matrices, entry (row i, input K): q = 0 the forward one (inputs 0..7), q = 1 / 2 the inverse's
// blocks, q = 3 the forward one for inputs 8..15.
double fixed_entry(int q, int i, int K) {
  auto c = [](int a, int b) { return cos(kTwoPi * (double)((a * b) % 16) / 16); };
  auto s = [](int a, int b) { return sin(kTwoPi * (double)((a * b) % 16) / 16); };
  switch (q) {
    case 0: {   // forward, inputs m < 8: rows (Yr k | Yi k), cols (Xr m | Xi m)
      const int k = i & 15, m = K & 7;
      const bool yi = i >= 16, xi = K >= 8;
      if (!yi) return xi ? s(k, m) : c(k, m);
      return xi ? c(k, m) : -s(k, m);
    }
    case 1: {   // inverse, Xr block: Yr = c, Yi = s
      const int n = i & 15;
      return i < 16 ? c(n, K) : s(n, K);
    }
    case 2: {   // inverse, Xi block: Yr = -s, Yi = c
      const int n = i & 15;
      return i < 16 ? -s(n, K) : c(n, K);
    }
    case 3: {   // forward, inputs 8 <= m < 16 (same layout as q = 0)
      const int k = i & 15, m = 8 + (K & 7);
      const bool yi = i >= 16, xi = K >= 8;
      if (!yi) return xi ? s(k, m) : c(k, m);
      return xi ? c(k, m) : -s(k, m);
    }
  }
  return 0.0;
}

// Angle (in turns) of the radix-32 entry (row i, input k) of slab matrix m for slab k1.
double slab_angle(int m, int k1, int i, int k) {
  switch (m) {
    case mf::MF2: return (double)((k * (16 * i + k1)) % 512) / 512;                 // row k2, input n2
    case mf::MF3: return (double)((perm_k3(k) * (512 * i + k1)) % mf::N) / mf::N;   // row k3, input n3
    case mf::MI3: return (double)((i * (512 * perm_k3(k) + k1)) % mf::N) / mf::N;   // row n3, input k3
    case mf::MI2: return (double)((i * (16 * perm_k3(k) + k1)) % 512) / 512;        // row n2, input k2
  }
  return 0.0;
}

uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
double bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
// fp16 bits of v, rounded to nearest even directly from double
uint16_t f16_rne(double v) {
  const _Float16 h = (_Float16)v;
  uint16_t b;
  memcpy(&b, &h, 2);
  return b;
}
}  // namespace

static_assert(kMfmaMatrixCount == ((size_t)mf::M1F_H2 + 1) * 64 * 8, "matrix table size");

// [NFIX][64][8], [16 slabs][4 mats][4 blocks][64][8], [1][64][8] (16-bit values; see the table layout in
// mfma_core.h)
void mfma_matrices_host(uint16_t* out) {
  for (int l = 0; l < 64; ++l)
    for (int e = 0; e < 8; ++e) {
      const int i = l % 32, K = 8 * (l / 32) + e;
      const double f = fixed_entry(0, i, K);
      const uint16_t hi = bf16_rne((float)f);
      out[(mf::M1F_HI * 64 + l) * 8 + e] = hi;
      out[(mf::M1F_LO * 64 + l) * 8 + e] = bf16_rne((float)(f - bf16_value(hi)));
      out[(mf::M1F_H * 64 + l) * 8 + e] = f16_rne(f);
      out[(mf::M1I_R * 64 + l) * 8 + e] = f16_rne(fixed_entry(1, i, K));
      out[(mf::M1I_I * 64 + l) * 8 + e] = f16_rne(fixed_entry(2, i, K));
      // twiddle pairs: dword m of block TW_C0 / TW_C1 holds registers 2m, 2m + 1 (resp. 8 + 2m, 9 + 2m)
      const int h = l / 32, j = l % 32;
      for (int blk = 0; blk < 2; ++blk) {
        const int v = 8 * blk + e;
        const int rowk = 8 * (v >> 2) + 4 * h + (v & 3);   // accumulator row of register v
        const double a = kTwoPi * (double)((j * rowk) % 1024) / 1024;
        out[((mf::TW_C0 + blk) * 64 + l) * 8 + e] = f16_rne(cos(a));
        out[((mf::TW_S0 + blk) * 64 + l) * 8 + e] = f16_rne(-sin(a));
      }
    }
  uint16_t* o = out + (size_t)mf::NFIX * 64 * 8;
  for (int k1 = 0; k1 < 16; ++k1)
    for (int m = 0; m < mf::NSLABMAT; ++m) {
      const double scale = (m == mf::MI3 || m == mf::MI2) ? 1.0 / 32 : 1.0;
      for (int b = 0; b < mf::NBLK; ++b)
        for (int l = 0; l < 64; ++l)
          for (int e = 0; e < 8; ++e) {
            const int i = l % 32, k = 8 * (l / 32) + e + ((b == mf::B_CHI || b == mf::B_SHI) ? 16 : 0);
            const double a = kTwoPi * slab_angle(m, k1, i, k);
            const double val = (b == mf::B_CLO || b == mf::B_CHI) ? cos(a) : sin(a);
            o[((((size_t)k1 * mf::NSLABMAT + m) * mf::NBLK + b) * 64 + l) * 8 + e] = f16_rne(val * scale);
          }
    }
  for (int l = 0; l < 64; ++l)
    for (int e = 0; e < 8; ++e)
      out[((size_t)mf::M1F_H2 * 64 + l) * 8 + e] = f16_rne(fixed_entry(3, l % 32, 8 * (l / 32) + e));
}

bool mfma_pair_supported(int log2L, int B) { return log2L == 13 && B % 2 == 0; }
size_t mfma_pair_spectrum_bytes_per_channel() { return (size_t)mf::PAIR_STRIDE * 4; }

hipError_t launch_conv_mfma(const void* u, const void* const* gates, const void* const* spectra, int order,
                            void* y, const void* mats, int B, int D, hipStream_t s) {
  if (order < 1 || order > kMfmaMaxChain) return hipErrorInvalidValue;
  MfmaChain ch{};
  bool gated = true;
  for (int i = 0; i < order; ++i) {
    ch.gate[i] = (const __bf16*)gates[i];
    ch.spectrum[i] = (const uint32_t*)spectra[i];
    gated = gated && gates[i] != nullptr;
  }
  if (!gated && (order != 1 || gates[0])) return hipErrorInvalidValue;   // only a single order may go ungated
  ch.order = order;
  // two row pairs per workgroup when a channel has an even number of them
  const int np = (B / 2) % 2 == 0 ? 2 : 1;
  const dim3 grid(D * (B / 2) / np), block(mf::T * np);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, (const __bf16*)u, (__bf16*)y, ch, (const u32x4*)mats, B, D);
  };
  if (gated) np == 2 ? go(k_conv_mfma<true, 2>) : go(k_conv_mfma<true, 1>);
  else np == 2 ? go(k_conv_mfma<false, 2>) : go(k_conv_mfma<false, 1>);
  return hipGetLastError();
}

hipError_t launch_pair_spectrum(const float2* Hnat, void* Hc, int D, hipStream_t s) {
  hipLaunchKernelGGL(k_pair_spectrum, dim3(D), dim3(256), 0, s, Hnat, (uint32_t*)Hc);
  return hipGetLastError();
}

}  // namespace hyena
