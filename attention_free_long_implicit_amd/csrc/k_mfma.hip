// Matrix-core (MFMA) causal long convolution for bf16 storage, L = 8192, rows taken in pairs.
//
// Operation: Hyena study note, steps 2-3 (long convolution with the implicit filter, gate);
// EulerStack "4. Hyena 상세", how it works 2 (FFT, elementwise product, inverse FFT); HyenaND summary,
// boundary handling (zero-pad to twice the size) and nSubQ implementation (forward transform,
// spectral product, inverse transform and output cut in one kernel, intermediates on chip).  The
// transform steps are small dense DFT matrices, evaluated as bf16 matrix products with fp32
// accumulation (a DFT as a dense matrix product is the remark in the SPECTRE digest's comments).
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
// spectrum is stored for slabs 0..8 only (36 KB per channel); conjugate symmetry gives the rest.
// A complex radix-R DFT is a real 2R x 2R matrix on (Re, Im); each MFMA (32x32x16) multiplies a 32-row
// block of it by 32 columns (independent sub-transforms).  LDS holds one plane of complex bf16 words
// (re low, im high); rows hold 32 words plus one pad, so lanes reading one word each from 32
// consecutive rows, or 32 consecutive words of one row, hit distinct banks.  Passes 2, 3, 3' and 2'
// of slab k1 touch only that slab, which one wave owns, so only two barriers are needed.  Global
// memory is touched in 16-byte accesses only: pass 1 and pass 1' give each lane 8 tiles whose columns
// are 8 consecutive samples.
#include <math.h>
#include <string.h>

#include "engine.h"
#include "launch.h"

namespace hyena {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

namespace mf {
constexpr int L = 8192, N = 2 * L;
constexpr int ROW = 33;                     // 32 values + 1 pad
constexpr int SLAB = 32 * ROW;              // one k1 (or n1-free) slab
constexpr int PLANE = 16 * SLAB;            // 16 slabs
constexpr int T = 256;                      // 4 waves
// Matrix table, per lane 8 bf16 in the A-operand layout (row i = lane % 32, K = 8 (lane / 32) + e).
// Fixed radix-16 matrices first, then per slab k1 four radix-32 matrices of four blocks each.
enum { M1F = 0, M1I_R, M1I_I, NFIX };
enum { MF2 = 0, MF3, MI3, MI2, NSLABMAT };       // pass 2, pass 3, pass 3', pass 2'
enum { B_CLO = 0, B_CHI, B_SLO, B_SHI, NBLK };   // cos / sin, K < 16 / K >= 16
constexpr int SLAB_TABLE = NSLABMAT * NBLK;       // bf16x8 per lane per slab
constexpr int PAIR_SLABS = 9;                     // filter-spectrum slabs stored per channel (k1 = 0..8)
}  // namespace mf

// Orders run back to back in one launch: gate and matrix-core spectrum copy of each order.
struct MfmaChain {
  const __bf16* gate[kMfmaMaxChain];
  const uint32_t* spectrum[kMfmaMaxChain];
  int order;
};

// Word 3 of a raw buffer descriptor on this architecture family: DATA_FORMAT = 32-bit (bits 15..18 = 4),
// no swizzle, no index stride; offsets beyond the record count read zero.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 neg8(bf16x8 v) {   // flip the 8 sign bits, one XOR per dword
  u32x4 r = __builtin_bit_cast(u32x4, v);
  r ^= 0x80008000u;
  return __builtin_bit_cast(bf16x8, r);
}

// output row of accumulator register v for lane half h (32x32 MFMA layout)
__device__ __forceinline__ int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// Complex radix-32 product of matrix blocks M (cos lo/hi, sin lo/hi) and data blocks (xr_lo, xr_hi, xi_lo,
// xi_hi).  Forward (W = cos - i sin): Yr = C Xr + S Xi, Yi = C Xi - S Xr;
// inverse (W = cos + i sin):           Yr = C Xr - S Xi, Yi = C Xi + S Xr.
// A and B operands share one register layout (lane % 32 = row or column, K = 8 (lane / 32) + e), so the
// same registers serve either side.  DATA_A = false: matrix on A, data columns on B -> output row = the
// matrix row, lane = the data column.  DATA_A = true: data on A -> the transpose (lane = the matrix row,
// registers = the data column), which puts the next contraction index in registers.
template <bool INV, bool DATA_A>
__device__ __forceinline__ void dft32(const bf16x8 (&M)[mf::NBLK], bf16x8 xr_lo, bf16x8 xr_hi, bf16x8 xi_lo,
                                      bf16x8 xi_hi, f32x16& dr, f32x16& di) {
  using namespace mf;
  auto mm = [](bf16x8 m, bf16x8 x, f32x16 c) { return DATA_A ? mfma(x, m, c) : mfma(m, x, c); };
  const f32x16 z = {};
  const bf16x8 sxi_lo = INV ? neg8(xi_lo) : xi_lo, sxi_hi = INV ? neg8(xi_hi) : xi_hi;
  const bf16x8 sxr_lo = INV ? xr_lo : neg8(xr_lo), sxr_hi = INV ? xr_hi : neg8(xr_hi);
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
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float2 unpack_c(uint32_t w) { return make_float2(lo_f32(w), hi_f32(w)); }

// fp32 accumulators, each multiplied by a complex factor, -> bf16 operands in accumulator order
// (block lo = registers 0..7, block hi = registers 8..15)
template <class F>
__device__ __forceinline__ void pack_operands(const f32x16& xr, const f32x16& xi, F&& factor, bf16x8& r_lo,
                                              bf16x8& r_hi, bf16x8& i_lo, bf16x8& i_hi) {
  u32x4 rl, rh, il, ih;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float2 a0 = factor(2 * m, make_float2(xr[2 * m], xi[2 * m]));
    const float2 a1 = factor(2 * m + 1, make_float2(xr[2 * m + 1], xi[2 * m + 1]));
    const float2 b0 = factor(8 + 2 * m, make_float2(xr[8 + 2 * m], xi[8 + 2 * m]));
    const float2 b1 = factor(9 + 2 * m, make_float2(xr[9 + 2 * m], xi[9 + 2 * m]));
    rl[m] = pack2(a0.x, a1.x);
    il[m] = pack2(a0.y, a1.y);
    rh[m] = pack2(b0.x, b1.x);
    ih[m] = pack2(b0.y, b1.y);
  }
  r_lo = __builtin_bit_cast(bf16x8, rl);
  r_hi = __builtin_bit_cast(bf16x8, rh);
  i_lo = __builtin_bit_cast(bf16x8, il);
  i_hi = __builtin_bit_cast(bf16x8, ih);
}

// 8 complex bf16 words (re low, im high) -> the 8 real parts and the 8 imaginary parts as MFMA operands
__device__ __forceinline__ void split8(const uint32_t (&c)[8], bf16x8& re, bf16x8& im) {
  u32x4 r, i;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    r[m] = __builtin_amdgcn_perm(c[2 * m + 1], c[2 * m], 0x05040100u);
    i[m] = __builtin_amdgcn_perm(c[2 * m + 1], c[2 * m], 0x07060302u);
  }
  re = __builtin_bit_cast(bf16x8, r);
  im = __builtin_bit_cast(bf16x8, i);
}
// element t (compile-time) of each of 8 vectors of 8 bf16 -> one operand
template <int TT>
__device__ __forceinline__ bf16x8 column8(const u32x4 (&V)[8]) {
  constexpr uint32_t sel = (TT & 1) ? 0x07060302u : 0x05040100u;
  u32x4 r;
#pragma unroll
  for (int m = 0; m < 4; ++m) r[m] = __builtin_amdgcn_perm(V[2 * m + 1][TT >> 1], V[2 * m][TT >> 1], sel);
  return __builtin_bit_cast(bf16x8, r);
}
template <int TT>
__device__ __forceinline__ float elem_f32(const u32x4& g) {
  return (TT & 1) ? hi_f32(g[TT >> 1]) : lo_f32(g[TT >> 1]);
}

// Pass 1 / pass 1' column mapping: wave w, lane j (= lane % 32), tile t handle column c = 256 w + 8 j + t
// (n3 = c % 32, n2 = c / 32), so each lane's 8 tiles cover 8 consecutive samples: one 16-byte access per
// (row, n1) in global memory.
template <bool GATE>
__global__ void __launch_bounds__(mf::T, 2)
k_conv_mfma(const __bf16* u, __bf16* y, MfmaChain ch, const bf16x8* __restrict__ mats, int B, int D,
            Twiddles tw) {
  using namespace mf;
  __shared__ uint32_t S[PLANE];
  const int npair = B >> 1;
  const int r = xcd_logical_block(blockIdx.x, D * npair);
  const int d = r / npair, p = r % npair;
  const size_t row0 = (size_t)(2 * p) * D + d, row1 = (size_t)(2 * p + 1) * D + d;

  // pass 1 input of the first order: lanes h = 0 / 1 carry row b0 / b1 (real / imaginary input), n1 = e
  u32x4 V[8];
  {
    const int l = threadIdx.x & 63, c0 = 256 * (threadIdx.x >> 6) + 8 * (l & 31);
    const __bf16* src = ((l >> 5) == 0 ? u + row0 * L : u + row1 * L) + c0;
#pragma unroll
    for (int e = 0; e < 8; ++e) V[e] = *reinterpret_cast<const u32x4*>(src + 1024 * e);
  }
  // Order-independent operands, loaded once right behind the first input (inside the order loop they
  // would queue behind that order's spectrum loads): the fixed radix-16 matrices and the per-lane
  // twiddles W_1024^{j k(v)}, k(v) = row of accumulator v.
  const int l0 = threadIdx.x & 63;
  const bf16x8 m1f = mats[M1F * 64 + l0], m1r = mats[M1I_R * 64 + l0], m1i = mats[M1I_I * 64 + l0];
  float2 p2[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) p2[v] = twiddle<10>(tw, uint32_t((l0 & 31) * acc_row(v, l0 >> 5)));

  for (int ord = 0; ord < ch.order; ++ord) {
  // lane constants derived from an opaque copy of the thread id, so nothing is hoisted across orders
  int tq = threadIdx.x;
  asm volatile("" : "+v"(tq));
  const int t = tq, w = t >> 6, l = t & 63, j = l & 31, h = l >> 5;
  const int c0 = 256 * w + 8 * j;
  const int n2c = 8 * w + (j >> 2), n3c = 8 * (j & 3);   // tile t: n2 = n2c, n3 = n3c + t
  const uint32_t* __restrict__ Hc = ch.spectrum[ord];
  const __bf16* gate = ch.gate[ord];

  // Slab matrices rotate through two buffers, each load issued one pass before its use:
  // Ma = pass 2, Mb = pass 3, then Ma = pass 3', Mb = pass 2', then the next slab's pass 2 and 3.
  // The first slab's matrices and filter spectrum are in flight during pass 1.
  bf16x8 Ma[NBLK], Mb[NBLK];
  // The matrix table and the spectrum are read through buffer descriptors: the per-lane part of the
  // offset is fixed, the block / register part (and the mirror choice, uniform per wave) stays in
  // scalar registers, so a slab's 32 loads cost no vector instructions for their addresses.
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(mats + NFIX * 64), (short)0, 16 * SLAB_TABLE * 64 * 16, kRawBufferWord3);
  const int mvo = l * 16;
  // blocks of matrix `which` of slab k1s (scalar) into M
  auto load_mat = [&](int k1s_, int which, bf16x8 (&M)[NBLK]) {
#pragma unroll
    for (int b = 0; b < NBLK; ++b)
      M[b] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                            mrs, mvo, ((k1s_ * SLAB_TABLE + which * NBLK + b) * 64) * 16, 0));
  };
  // Filter spectrum: only slabs 0..8 are stored.  h is real, so H[N - k] = conj(H[k]); bin N - k of
  // slab k1 > 8 is register 15 - v of lane 63 - l in slab 16 - k1, read mirrored; the conjugation (sign
  // of the imaginary half) is applied where the value is used, so the load stays in flight until then.
  uint32_t hw[16];
  const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Hc + (size_t)d * PAIR_SLABS * 16 * 64), (short)0, PAIR_SLABS * 16 * 64 * 4, kRawBufferWord3);
  const int ws = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto load_spectrum = [&](int k1) {
    const bool mirror = k1 > 8;
    const int slab = (mirror ? 16 - k1 : k1) * (16 * 64 * 4);
    const int vo = (mirror ? 63 - l : l) * 4;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      hw[v] = __builtin_amdgcn_raw_buffer_load_b32(hrs, vo, slab + (mirror ? 15 - v : v) * 256, 0);
  };
  load_mat(ws, MF2, Ma);
  load_mat(ws, MF3, Mb);
  load_spectrum(ws);
  {
    static_for<8>([&](auto tt) {
      constexpr int TT = tt.value;
      const f32x16 z = {};
      const f32x16 D1 = mfma(m1f, column8<TT>(V), z);
      // rows k1 = acc_row(e, h): real part in D1[e], imaginary part in D1[8 + e]
#pragma unroll
      for (int e = 0; e < 8; ++e) S[acc_row(e, h) * SLAB + n2c * ROW + n3c + TT] = pack2(D1[e], D1[8 + e]);
    });
  }
  __syncthreads();

  // ---------------- passes 2, 3, 3', 2' per slab k1 (wave w owns k1 = w, w+4, w+8, w+12)
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
  auto slab_step = [&](int it) {
    const int k1 = w + 4 * it;
    const int k1s = ws + 4 * it;   // the same slab index, in a scalar register
    uint32_t* sl = S + k1 * SLAB;
    bf16x8 xr_lo, xr_hi, xi_lo, xi_hi;
    f32x16 dr, di;
    // pass 2: data on A (rows n3 = j, K = n2 from LDS: element (n2, n3) at n2 * ROW + n3), matrix on B
    //   -> lane = k2, registers = n3 (row of v)
    {
      uint32_t clo[8], chi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        clo[e] = sl[(8 * h + e) * ROW + j];
        chi[e] = sl[(16 + 8 * h + e) * ROW + j];
      }
      split8(clo, xr_lo, xi_lo);
      split8(chi, xr_hi, xi_hi);
      dft32<false, true>(Ma, xr_lo, xr_hi, xi_lo, xi_hi, dr, di);
      load_mat(k1s, MI3, Ma);
    }
    // twiddle W_1024^{n3 k2} (k2 = j, n3 = row of v); pass 3: matrix on A (rows k3, input n3 in accumulator
    // order), data on B -> lane = k2, registers = k3
    pack_operands(dr, di, [&](int v, float2 x) { return cmul(x, p2[v]); }, xr_lo, xr_hi, xi_lo, xi_hi);
    dft32<false, false>(Mb, xr_lo, xr_hi, xi_lo, xi_hi, dr, di);
    load_mat(k1s, MI2, Mb);
    // spectral product: bin k1 + 16 j + 512 k3(v); Hc holds H/N in this exact order.
    // pass 3': data on A (rows k2 = j, input k3 in accumulator order), matrix on B -> lane = n3,
    // registers = k2
    const uint32_t flip = k1s > 8 ? 0x80000000u : 0u;
    pack_operands(dr, di, [&](int v, float2 x) { return cmul(x, unpack_c(hw[v] ^ flip)); }, xr_lo, xr_hi, xi_lo,
                  xi_hi);
    if (it < 3) load_spectrum(k1s + 4);
    f32x16 er, ei;
    dft32<true, true>(Ma, xr_lo, xr_hi, xi_lo, xi_hi, er, ei);
    if (it < 3) load_mat(k1s + 4, MF2, Ma);
    // conj twiddle W_1024^{n3 k2} (n3 = j, k2 = row of v); pass 2': matrix on A (rows n2, input k2 in
    // accumulator order), data on B -> lane = n3, registers = n2; store (n2, n3) at n2 * ROW + n3
    pack_operands(er, ei, [&](int v, float2 x) { return cmulc(x, p2[v]); }, xr_lo, xr_hi, xi_lo, xi_hi);
    dft32<true, false>(Mb, xr_lo, xr_hi, xi_lo, xi_hi, er, ei);
    if (it < 3) load_mat(k1s + 4, MF3, Mb);
#pragma unroll
    for (int v = 0; v < 16; ++v) sl[acc_row(v, h) * ROW + j] = pack2(er[v], ei[v]);
  };
  // The gate for pass 1' is issued before the last slab, behind that slab's matrix and spectrum loads
  // (the vector-memory counter retires in order, so no earlier slab waits on it): lane keeps rows
  // b0 / b1 at n1 = 4h + e (e < 4), 8 consecutive samples each.
  for (int it = 0; it < 3; ++it) slab_step(it);
  load_gate();
  slab_step(3);

  __syncthreads();

  // ---------------- pass 1': tiles t, column c = c0 + t, K = k1 (slab index), outputs n1 = 4h + e
  {
    u32x4 Y[2][4];
    float pa[4], pb[4];
    static_for<8>([&](auto tt) {
      constexpr int TT = tt.value;
      uint32_t cw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cw[e] = S[(8 * h + e) * SLAB + n2c * ROW + n3c + TT];
      bf16x8 xr, xi;
      split8(cw, xr, xi);
      const f32x16 z = {};
      f32x16 o = mfma(m1r, xr, z);
      o = mfma(m1i, xi, o);
      // rows 4h + e (e < 4): real part (row b0) in o[e], imaginary part (row b1) in o[8 + e]
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a = o[e], b = o[8 + e];
        if (GATE) {
          a *= elem_f32<TT>(G[0][e]);
          b *= elem_f32<TT>(G[1][e]);
        }
        if constexpr (TT % 2 == 0) {
          pa[e] = a;
          pb[e] = b;
        } else {
          Y[0][e][TT >> 1] = pack2(pa[e], a);
          Y[1][e][TT >> 1] = pack2(pb[e], b);
        }
      }
    });
    __bf16* y0 = y + row0 * L + c0;
    __bf16* y1 = y + row1 * L + c0;
    if (ord + 1 == ch.order) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<u32x4*>(y0 + 1024 * (4 * h + e)) = Y[0][e];
        *reinterpret_cast<u32x4*>(y1 + 1024 * (4 * h + e)) = Y[1][e];
      }
    } else {
      // u_i stays on chip, rounded to bf16 exactly as its store would be.  Pass 1' left lane (j, h) with
      // rows b0, b1 at n1 = 4h + e; the next pass 1 wants row b_h at n1 = 0..7 in lane (j, h).  One
      // cross-half swap per register does it: swapping the upper half of the row-b0 register with the
      // lower half of the row-b1 register leaves [b0 from lanes 0..31, b1 from lanes 0..31] (n1 = e) in
      // the first and [b0 from lanes 32..63, b1 from lanes 32..63] (n1 = 4 + e) in the second.
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const auto r = __builtin_amdgcn_permlane32_swap(Y[0][e][q], Y[1][e][q], false, false);
          V[e][q] = r[0];
          V[4 + e][q] = r[1];
        }
      }
      __syncthreads();   // every wave is done reading LDS before the next order's pass 1 writes it
    }
  }
  }
}


// Pair-order spectrum: Hc[d][k1][v][lane] = H[k]/N as bf16 (re low, im high), k = k1 + 16 (lane%32)
// + 512 k3(v, lane/32), for k1 = 0..8 (the convolution kernel mirrors slabs 9..15 from slabs 7..1);
// H from the natural-order bins 0..L (upper bins by conjugate symmetry).
__global__ void k_pair_spectrum(const float2* __restrict__ Hnat, uint32_t* __restrict__ Hc) {
  using namespace mf;
  const int d = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;    // (k1, v, lane)
  if (idx >= PAIR_SLABS * 16 * 64) return;
  const int k1 = idx / (16 * 64), v = (idx / 64) % 16, l = idx % 64;
  const int jj = l & 31, h = l >> 5;
  const int k = k1 + 16 * jj + 512 * acc_row(v, h);
  const float2* hn = Hnat + (size_t)d * (L + 1);
  float2 hv = k <= L ? hn[k] : cconj(hn[N - k]);
  hv = cscale(hv, 1.0f / N);
  const uint32_t lo = (uint32_t)f32_to_bf16_rne(hv.x), hi = (uint32_t)f32_to_bf16_rne(hv.y);
  Hc[(size_t)d * PAIR_SLABS * 16 * 64 + idx] = lo | (hi << 16);
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

// Radix-16 matrices, entry (row i, input K).
float fixed_entry(int q, int i, int K) {
  auto c = [](int a, int b) { return cos(kTwoPi * (double)((a * b) % 16) / 16); };
  auto s = [](int a, int b) { return sin(kTwoPi * (double)((a * b) % 16) / 16); };
  switch (q) {
    case mf::M1F: {   // forward, inputs m < 8: rows (Yr k | Yi k), cols (Xr m | Xi m)
      const int k = i & 15, m = K & 7;
      const bool yi = i >= 16, xi = K >= 8;
      if (!yi) return (float)(xi ? s(k, m) : c(k, m));
      return (float)(xi ? c(k, m) : -s(k, m));
    }
    case mf::M1I_R: {  // inverse, Xr block: Yr = c, Yi = s
      const int n = i & 15;
      return (float)(i < 16 ? c(n, K) : s(n, K));
    }
    case mf::M1I_I: {  // inverse, Xi block: Yr = -s, Yi = c
      const int n = i & 15;
      return (float)(i < 16 ? -s(n, K) : c(n, K));
    }
  }
  return 0.f;
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
}  // namespace

static_assert(kMfmaMatrixCount == ((size_t)mf::NFIX + 16 * mf::SLAB_TABLE) * 64 * 8, "matrix table size");

// [NFIX][64][8], [16 slabs][4 mats][4 blocks][64][8] (bf16)
void mfma_matrices_host(uint16_t* out) {
  for (int q = 0; q < mf::NFIX; ++q)
    for (int l = 0; l < 64; ++l)
      for (int e = 0; e < 8; ++e) out[(q * 64 + l) * 8 + e] = bf16_rne(fixed_entry(q, l % 32, 8 * (l / 32) + e));
  uint16_t* o = out + (size_t)mf::NFIX * 64 * 8;
  for (int k1 = 0; k1 < 16; ++k1)
    for (int m = 0; m < mf::NSLABMAT; ++m)
      for (int b = 0; b < mf::NBLK; ++b)
        for (int l = 0; l < 64; ++l)
          for (int e = 0; e < 8; ++e) {
            const int i = l % 32, k = 8 * (l / 32) + e + ((b == mf::B_CHI || b == mf::B_SHI) ? 16 : 0);
            const double a = kTwoPi * slab_angle(m, k1, i, k);
            const double val = (b == mf::B_CLO || b == mf::B_CHI) ? cos(a) : sin(a);
            o[((((size_t)k1 * mf::NSLABMAT + m) * mf::NBLK + b) * 64 + l) * 8 + e] = bf16_rne((float)val);
          }
}

bool mfma_pair_supported(int log2L, int B) { return log2L == 13 && B % 2 == 0; }
size_t mfma_pair_spectrum_bytes_per_channel() { return (size_t)mf::PAIR_SLABS * 16 * 64 * 4; }

hipError_t launch_conv_mfma(const void* u, const void* const* gates, const void* const* spectra, int order,
                            void* y, const void* mats, int B, int D, const Twiddles& tw, hipStream_t s) {
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
  const dim3 grid(D * (B / 2)), block(mf::T);
  if (gated)
    hipLaunchKernelGGL((k_conv_mfma<true>), grid, block, 0, s, (const __bf16*)u, (__bf16*)y, ch, (const bf16x8*)mats,
                       B, D, tw);
  else
    hipLaunchKernelGGL((k_conv_mfma<false>), grid, block, 0, s, (const __bf16*)u, (__bf16*)y, ch,
                       (const bf16x8*)mats, B, D, tw);
  return hipGetLastError();
}

hipError_t launch_pair_spectrum(const float2* Hnat, void* Hc, int D, hipStream_t s) {
  hipLaunchKernelGGL(k_pair_spectrum, dim3((mf::PAIR_SLABS * 16 * 64 + 255) / 256, D), dim3(256), 0, s, Hnat,
                     (uint32_t*)Hc);
  return hipGetLastError();
}

}  // namespace hyena
