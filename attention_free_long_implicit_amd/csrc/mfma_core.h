// Matrix-core building blocks shared by the kernels that evaluate 16384-point transforms as products of
// small DFT matrices on the matrix cores (32x32x16 MFMA, fp16 / bf16 operands, fp32 accumulation): operand
// types, the layout of the constant matrix table, the complex radix-32 product, packed fp16 complex
// products, and the conversions between accumulators, fp16 pairs and MFMA operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hyena {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

namespace mf {
constexpr int L = 8192, N = 2 * L;
constexpr int ROW = 33;                     // 32 values + 1 pad
constexpr int SLAB = 32 * ROW;              // one k1 (or n1-free) slab
constexpr int PLANE = 16 * SLAB;            // 16 slabs
constexpr int T = 256;                      // 4 waves
// Matrix table, per lane 8 16-bit values in the A-operand layout (row i = lane % 32, K = 8 (lane / 32) + e).
// Fixed radix-16 matrices first -- the forward one as two bf16 parts (hi, and lo = the rest) and in fp16,
// the two inverse blocks in fp16 -- and the lane's twiddles W_1024^{j k(v)} as fp16 pairs (cos parts of
// registers 0..7, 8..15, then the -sin parts) -- then per slab k1 four fp16 radix-32 matrices of four blocks each (cos
// and sin, each for K < 16 and K >= 16; the inverse ones, passes 3' and 2', scaled by 1/32).
// After the slab matrices, one more fixed block: the forward radix-16 matrix for inputs 8..15 in fp16
// (M1F_H2, for transforms whose inputs are all non-zero).
enum { M1F_HI = 0, M1F_LO, M1F_H, M1I_R, M1I_I, TW_C0, TW_C1, TW_S0, TW_S1, NFIX };
enum { MF2 = 0, MF3, MI3, MI2, NSLABMAT };       // pass 2, pass 3, pass 3', pass 2'
enum { B_CLO = 0, B_CHI, B_SLO, B_SHI, NBLK };   // cos / sin, K < 16 / K >= 16
constexpr int SLAB_TABLE = NSLABMAT * NBLK;       // 16-byte entries per lane per slab
constexpr int PAIR_SLABS = 9;                     // filter-spectrum slabs stored per channel (k1 = 0..8)
constexpr int PAIR_WORDS = PAIR_SLABS * 16 * 64;  // fp16 complex words of one channel's spectrum copy
constexpr int PAIR_STRIDE = PAIR_WORDS + 64;      // + one 256-byte tail: word 0 = the spectrum's scale back
constexpr float INV_SCALE = 1024.0f;              // undoes the two 1/32 factors of the inverse matrices
constexpr int M1F_H2 = NFIX + 16 * SLAB_TABLE;    // index of the block after the slab matrices
}  // namespace mf

// Word 3 of a raw buffer descriptor on this architecture family: DATA_FORMAT = 32-bit (bits 15..18 = 4),
// no swizzle, no index stride; offsets beyond the record count read zero.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 neg8(f16x8 v) {     // flip the 8 sign bits, one XOR per dword
  u32x4 r = __builtin_bit_cast(u32x4, v);
  r ^= 0x80008000u;
  return __builtin_bit_cast(f16x8, r);
}
__device__ __forceinline__ f16x8 as_h(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ bf16x8 as_b(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 2^-e with e the binary exponent of m (m = f 2^e, f in [0.5, 1)): the power of two that brings the
// largest magnitude m into [0.5, 1); 1 for a zero or non-finite m.  The exponent is clamped to what an
// fp32 power of two can hold.
__device__ __forceinline__ float range_scale(float m) {
  if (!(m > 0.0f) || !(m <= 3.0e38f)) return 1.0f;
  int e = __builtin_amdgcn_frexp_expf(m);
  e = e < -125 ? -125 : (e > 125 ? 125 : e);
  return __builtin_ldexpf(1.0f, -e);
}
// largest value of v over this thread's group of four waves (waves 4g..4g+3); red: one float of LDS per
// wave of the workgroup; every thread returns its group's result.  The caller's next barrier must not be
// this one's: the slots are rewritten only after later barriers.
__device__ __forceinline__ float block_max4(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float* g = red + 4 * (threadIdx.x >> 8);
  return fmaxf(fmaxf(g[0], g[1]), fmaxf(g[2], g[3]));
}

// Largest values per row over this thread's group of four waves (waves 4g..4g+3), for data whose lanes
// carry row h = lane / 32 (v) or both rows (v0, v1); red: two floats of LDS per wave of the workgroup.
// Every thread receives both rows' results.  The caller's next barrier must not be this one's.
__device__ __forceinline__ void block_max4_rows(float v, float* red, float& m0, float& m1) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 31) == 0) red[2 * (threadIdx.x >> 6) + ((threadIdx.x >> 5) & 1)] = v;
  __syncthreads();
  const float* g = red + 8 * (threadIdx.x >> 8);
  m0 = fmaxf(fmaxf(g[0], g[2]), fmaxf(g[4], g[6]));
  m1 = fmaxf(fmaxf(g[1], g[3]), fmaxf(g[5], g[7]));
}
__device__ __forceinline__ void block_max4x2(float v0, float v1, float* red, float& m0, float& m1) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    v0 = fmaxf(v0, __shfl_xor(v0, o));
    v1 = fmaxf(v1, __shfl_xor(v1, o));
  }
  if ((threadIdx.x & 63) == 0) {
    red[2 * (threadIdx.x >> 6)] = v0;
    red[2 * (threadIdx.x >> 6) + 1] = v1;
  }
  __syncthreads();
  const float* g = red + 8 * (threadIdx.x >> 8);
  m0 = fmaxf(fmaxf(g[0], g[2]), fmaxf(g[4], g[6]));
  m1 = fmaxf(fmaxf(g[1], g[3]), fmaxf(g[5], g[7]));
}

// output row of accumulator register v for lane half h (32x32 MFMA layout)
__device__ __forceinline__ int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// Complex radix-32 product of matrix blocks M (cos lo/hi, sin lo/hi) and data blocks (xr_lo, xr_hi, xi_lo,
// xi_hi).  Forward (W = cos - i sin): Yr = C Xr + S Xi, Yi = C Xi - S Xr;
// inverse (W = cos + i sin):           Yr = C Xr - S Xi, Yi = C Xi + S Xr.
// (Storing -sin blocks instead of negating data costs more in matrix loads than the sign flips cost.)
// A and B operands share one register layout (lane % 32 = row or column, K = 8 (lane / 32) + e), so the
// same registers serve either side.  DATA_A = false: matrix on A, data columns on B -> output row = the
// matrix row, lane = the data column.  DATA_A = true: data on A -> the transpose (lane = the matrix row,
// registers = the data column), which puts the next contraction index in registers.
template <bool INV, bool DATA_A>
__device__ __forceinline__ void dft32(const f16x8 (&M)[mf::NBLK], f16x8 xr_lo, f16x8 xr_hi, f16x8 xi_lo,
                                      f16x8 xi_hi, f32x16& dr, f32x16& di) {
  using namespace mf;
  auto mm = [](f16x8 m, f16x8 x, f32x16 c) { return DATA_A ? mfma(x, m, c) : mfma(m, x, c); };
  const f32x16 z = {};
  const f16x8 sxi_lo = INV ? neg8(xi_lo) : xi_lo, sxi_hi = INV ? neg8(xi_hi) : xi_hi;
  const f16x8 sxr_lo = INV ? xr_lo : neg8(xr_lo), sxr_hi = INV ? xr_hi : neg8(xr_hi);
  dr = mm(M[B_CLO], xr_lo, z);
  dr = mm(M[B_CHI], xr_hi, dr);
  dr = mm(M[B_SLO], sxi_lo, dr);
  dr = mm(M[B_SHI], sxi_hi, dr);
  di = mm(M[B_CLO], xi_lo, z);
  di = mm(M[B_CHI], xi_hi, di);
  di = mm(M[B_SLO], sxr_lo, di);
  di = mm(M[B_SHI], sxr_hi, di);
}

// two floats -> one dword of bf16 (round to nearest even), a in the low half
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// two floats -> one dword of fp16 (round to nearest even), a in the low half
__device__ __forceinline__ uint32_t pack2h(float a, float b) {
  const f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// fp32 accumulators -> fp16 pairs in accumulator order: pair q holds registers 2q (low half) and 2q + 1
__device__ __forceinline__ void to_pairs(const f32x16& x, f16x2 (&p)[8]) {
#pragma unroll
  for (int q = 0; q < 8; ++q) p[q] = f16x2{(_Float16)x[2 * q], (_Float16)x[2 * q + 1]};
}
// Complex product of fp16 pairs (a + i b) and (c + i s), or (c - i s) with CONJ, in packed fp16 arithmetic
// (two complex values per instruction), written as MFMA operands (block lo = pairs 0..3, hi = pairs 4..7).
template <bool CONJ>
__device__ __forceinline__ void cmul_pairs(const f16x2 (&a)[8], const f16x2 (&b)[8], const f16x2 (&c)[8],
                                           const f16x2 (&sn)[8], f16x8& r_lo, f16x8& r_hi, f16x8& i_lo,
                                           f16x8& i_hi) {
  u32x4 rl, rh, il, ih;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    f16x2 re, im;
    if (CONJ) {
      re = __builtin_elementwise_fma(a[q], c[q], b[q] * sn[q]);
      im = __builtin_elementwise_fma(b[q], c[q], -(a[q] * sn[q]));
    } else {
      re = __builtin_elementwise_fma(a[q], c[q], -(b[q] * sn[q]));
      im = __builtin_elementwise_fma(a[q], sn[q], b[q] * c[q]);
    }
    if (q < 4) {
      rl[q] = __builtin_bit_cast(uint32_t, re);
      il[q] = __builtin_bit_cast(uint32_t, im);
    } else {
      rh[q - 4] = __builtin_bit_cast(uint32_t, re);
      ih[q - 4] = __builtin_bit_cast(uint32_t, im);
    }
  }
  r_lo = as_h(rl);
  r_hi = as_h(rh);
  i_lo = as_h(il);
  i_hi = as_h(ih);
}

// 8 complex fp16 words (re low, im high) -> the 8 real parts and the 8 imaginary parts as MFMA operands
__device__ __forceinline__ void split8(const uint32_t (&c)[8], f16x8& re, f16x8& im) {
  u32x4 r, i;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    r[m] = __builtin_amdgcn_perm(c[2 * m + 1], c[2 * m], 0x05040100u);
    i[m] = __builtin_amdgcn_perm(c[2 * m + 1], c[2 * m], 0x07060302u);
  }
  re = as_h(r);
  im = as_h(i);
}
// element t (compile-time) of each of 8 vectors of 8 16-bit values -> one operand (its bits)
template <int TT>
__device__ __forceinline__ u32x4 column8(const u32x4 (&V)[8]) {
  constexpr uint32_t sel = (TT & 1) ? 0x07060302u : 0x05040100u;
  u32x4 r;
#pragma unroll
  for (int m = 0; m < 4; ++m) r[m] = __builtin_amdgcn_perm(V[2 * m + 1][TT >> 1], V[2 * m][TT >> 1], sel);
  return r;
}
template <int TT>
__device__ __forceinline__ float elem_f32(const u32x4& g) {
  return (TT & 1) ? hi_f32(g[TT >> 1]) : lo_f32(g[TT >> 1]);
}

}  // namespace hyena
