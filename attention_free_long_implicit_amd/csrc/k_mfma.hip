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
// N = 2L = 16384 = 16 x 32 x 32, n = n3 + 32 n2 + 1024 n1 (n1 < 8 nonzero), k = k1 + 16 k2 + 512 k3.
//   pass 1  DFT over n1 (radix 16, half the inputs zero), twiddle W_N^{(n3 + 32 n2) k1}
//   pass 2  DFT over n2 (radix 32), twiddle W_1024^{n3 k2}
//   pass 3  DFT over n3 (radix 32) -> Z[k]; times H[k]/N (bf16 spectrum in consumption order)
//   pass 3' inverse DFT over k3 straight from the accumulators (the matrix's input order is the
//           accumulator row order), conj twiddle W_1024^{n3 k2}
//   pass 2' inverse DFT over k2, conj twiddle W_N^{(n3 + 32 n2) k1}
//   pass 1' inverse DFT over k1, keep n1 < 8 (the causal half); gate; store
// A complex radix-R DFT is a real 2R x 2R matrix on (Re, Im); each MFMA (32x32x16) multiplies a 32-row
// block of it by 32 columns (independent sub-transforms).  Every lane keeps the DFT matrices it needs
// (44 VGPRs).  LDS rows hold 32 values plus one pad, so lanes reading one element each from 32
// consecutive rows, or 32 consecutive elements of one row, hit distinct banks.  Passes 2, 3, 3' and
// 2' of tile k1 touch only slab k1, which one wave owns, so only two barriers are needed.
#include <math.h>
#include <string.h>

#include "engine.h"
#include "launch.h"

namespace hyena {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

namespace mf {
constexpr int L = 8192, N = 2 * L;
constexpr int ROW = 33;                     // 32 values + 1 pad
constexpr int SLAB = 32 * ROW;              // one k1 (or n1-free) slab
constexpr int PLANE = 16 * SLAB;            // 16 slabs
constexpr int T = 256;                      // 4 waves
// DFT matrices, each stored per lane as 8 bf16 (A operand layout): index into the table
enum { M1F = 0, C_LO, C_HI, S_LO, S_HI, CP_LO, CP_HI, SP_LO, SP_HI, M1I_R, M1I_I, NMAT };
}  // namespace mf

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 neg8(bf16x8 v) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = -v[e];
  return r;
}
__device__ __forceinline__ __bf16 tobf(float f) { return (__bf16)f; }

// output row of accumulator register v for lane half h (32x32 MFMA layout)
__device__ __forceinline__ int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// radix-32 forward / inverse on B blocks (xr_lo, xr_hi, xi_lo, xi_hi); out dr, di
template <bool INV>
__device__ __forceinline__ void dft32(const bf16x8 (&A)[mf::NMAT], int c_lo, int c_hi, int s_lo, int s_hi,
                                      bf16x8 xr_lo, bf16x8 xr_hi, bf16x8 xi_lo, bf16x8 xi_hi, f32x16& dr,
                                      f32x16& di) {
  f32x16 z = {};
  // forward: Yr = C Xr + S Xi, Yi = C Xi - S Xr;  inverse: Yr = C Xr - S Xi, Yi = C Xi + S Xr
  const bf16x8 sxi_lo = INV ? neg8(xi_lo) : xi_lo, sxi_hi = INV ? neg8(xi_hi) : xi_hi;
  const bf16x8 sxr_lo = INV ? xr_lo : neg8(xr_lo), sxr_hi = INV ? xr_hi : neg8(xr_hi);
  dr = mfma(A[c_lo], xr_lo, z);
  dr = mfma(A[c_hi], xr_hi, dr);
  dr = mfma(A[s_lo], sxi_lo, dr);
  dr = mfma(A[s_hi], sxi_hi, dr);
  di = mfma(A[c_lo], xi_lo, z);
  di = mfma(A[c_hi], xi_hi, di);
  di = mfma(A[s_lo], sxr_lo, di);
  di = mfma(A[s_hi], sxr_hi, di);
}

// Gather 8 bf16 of one plane: base + e * stride, e < 8
template <int STRIDE>
__device__ __forceinline__ bf16x8 lds8(const __bf16* p) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = p[e * STRIDE];
  return r;
}

template <bool GATE>
__global__ void __launch_bounds__(mf::T, 2)
k_conv_mfma(const __bf16* u, const __bf16* gate, __bf16* y, const uint32_t* __restrict__ Hc,
            const bf16x8* __restrict__ mats, int B, int D, Twiddles tw) {
  using namespace mf;
  __shared__ __bf16 lre[PLANE];
  __shared__ __bf16 lim[PLANE];
  const int t = threadIdx.x, w = t >> 6, l = t & 63, j = l & 31, h = l >> 5;
  const int npair = B >> 1;
  const int r = xcd_logical_block(blockIdx.x, D * npair);
  const int d = r / npair, p = r % npair;
  const size_t row0 = (size_t)(2 * p) * D + d, row1 = (size_t)(2 * p + 1) * D + d;

  bf16x8 A[NMAT];
#pragma unroll
  for (int q = 0; q < NMAT; ++q) A[q] = mats[q * 64 + l];

  // per-lane twiddles: p1[e] = W_N^{j k1(e)}, k1(e) = row of accumulator e (e < 8);
  //                    p2[v] = W_1024^{j k(v)},  k(v) = row of accumulator v
  float2 p1[8], p2[16];
#pragma unroll
  for (int e = 0; e < 8; ++e) p1[e] = twiddle<14>(tw, uint32_t(j * acc_row(e, h)));
#pragma unroll
  for (int v = 0; v < 16; ++v) p2[v] = twiddle<10>(tw, uint32_t(j * acc_row(v, h)));

  // ---------------- pass 1: tiles n2 (8 per wave), columns n3 = j; lanes h = 0 / 1 carry row b0 / b1
  {
    const __bf16* src = (h == 0 ? u + row0 * L : u + row1 * L) + j;
    for (int it = 0; it < 8; ++it) {
      const int n2 = w * 8 + it;
      bf16x8 b;
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = src[32 * n2 + 1024 * e];
      f32x16 z = {};
      const f32x16 D1 = mfma(A[M1F], b, z);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k1 = acc_row(e, h);
        const float2 q = twiddle<9>(tw, uint32_t(n2 * k1));     // W_512^{n2 k1}, same across the half-wave
        const float2 tw1 = cmul(p1[e], q);
        const float2 v = cmul(make_float2(D1[e], D1[8 + e]), tw1);
        const int a = (k1 * 32 + n2) * ROW + j;
        lre[a] = tobf(v.x);
        lim[a] = tobf(v.y);
      }
    }
  }
  __syncthreads();

  // ---------------- passes 2, 3, 3', 2' per slab k1 (wave w owns k1 = w, w+4, w+8, w+12)
  for (int it = 0; it < 4; ++it) {
    const int k1 = w + 4 * it;
    __bf16* sre = lre + k1 * SLAB;
    __bf16* sim = lim + k1 * SLAB;
    // pass 2: columns n3 = j, K = n2: element (n2, n3) at n2 * ROW + n3
    {
      const bf16x8 xr_lo = lds8<ROW>(sre + (8 * h) * ROW + j), xr_hi = lds8<ROW>(sre + (16 + 8 * h) * ROW + j);
      const bf16x8 xi_lo = lds8<ROW>(sim + (8 * h) * ROW + j), xi_hi = lds8<ROW>(sim + (16 + 8 * h) * ROW + j);
      f32x16 dr, di;
      dft32<false>(A, C_LO, C_HI, S_LO, S_HI, xr_lo, xr_hi, xi_lo, xi_hi, dr, di);
      // twiddle W_1024^{n3 k2} (n3 = j, k2 = row of v), store (k2, n3) at k2 * ROW + n3
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float2 o = cmul(make_float2(dr[v], di[v]), p2[v]);
        const int a = acc_row(v, h) * ROW + j;
        sre[a] = tobf(o.x);
        sim[a] = tobf(o.y);
      }
    }
    // pass 3: columns k2 = j, K = n3: element (k2, n3) at k2 * ROW + n3
    f32x16 dr, di;
    {
      const bf16x8 xr_lo = lds8<1>(sre + j * ROW + 8 * h), xr_hi = lds8<1>(sre + j * ROW + 16 + 8 * h);
      const bf16x8 xi_lo = lds8<1>(sim + j * ROW + 8 * h), xi_hi = lds8<1>(sim + j * ROW + 16 + 8 * h);
      dft32<false>(A, C_LO, C_HI, S_LO, S_HI, xr_lo, xr_hi, xi_lo, xi_hi, dr, di);
    }
    // spectral product: bin k1 + 16 j + 512 k3(v); Hc holds H/N in this exact order
    {
      const uint32_t* hp = Hc + ((size_t)d * 16 + k1) * 16 * 64 + l;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t hw = hp[v * 64];
        const float2 hv = make_float2(__uint_as_float(hw << 16), __uint_as_float(hw & 0xffff0000u));
        const float2 o = cmul(make_float2(dr[v], di[v]), hv);
        dr[v] = o.x;
        di[v] = o.y;
      }
    }
    // pass 3': inverse over k3 from the accumulators (register v is input K' = v of the permuted matrix)
    {
      bf16x8 yr_lo, yr_hi, yi_lo, yi_hi;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        yr_lo[e] = tobf(dr[e]); yr_hi[e] = tobf(dr[8 + e]);
        yi_lo[e] = tobf(di[e]); yi_hi[e] = tobf(di[8 + e]);
      }
      f32x16 er, ei;
      dft32<true>(A, CP_LO, CP_HI, SP_LO, SP_HI, yr_lo, yr_hi, yi_lo, yi_hi, er, ei);
      // conj twiddle W_1024^{n3 k2} (k2 = j, n3 = row of v), store (n3, k2) at n3 * ROW + k2
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float2 o = cmulc(make_float2(er[v], ei[v]), p2[v]);
        const int a = acc_row(v, h) * ROW + j;
        sre[a] = tobf(o.x);
        sim[a] = tobf(o.y);
      }
    }
    // pass 2': inverse over k2, columns n3 = j: element (n3, k2) at n3 * ROW + k2
    {
      const bf16x8 xr_lo = lds8<1>(sre + j * ROW + 8 * h), xr_hi = lds8<1>(sre + j * ROW + 16 + 8 * h);
      const bf16x8 xi_lo = lds8<1>(sim + j * ROW + 8 * h), xi_hi = lds8<1>(sim + j * ROW + 16 + 8 * h);
      f32x16 er, ei;
      dft32<true>(A, C_LO, C_HI, S_LO, S_HI, xr_lo, xr_hi, xi_lo, xi_hi, er, ei);
      // conj twiddle W_N^{(n3 + 32 n2) k1} = conj(W_N^{n3 k1} W_512^{n2 k1}); store (n2, n3) at n2 * ROW + n3
      const float2 a1 = twiddle<14>(tw, uint32_t(j * k1));
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int n2 = acc_row(v, h);
        const float2 b1 = twiddle<9>(tw, uint32_t(n2 * k1));
        const float2 o = cmulc(make_float2(er[v], ei[v]), cmul(a1, b1));
        const int a = n2 * ROW + j;
        sre[a] = tobf(o.x);
        sim[a] = tobf(o.y);
      }
    }
  }
  __syncthreads();

  // ---------------- pass 1': tiles n2 (8 per wave), columns n3 = j, K = k1 (slab index)
  {
    const size_t base0 = row0 * L, base1 = row1 * L;
    for (int it = 0; it < 8; ++it) {
      const int n2 = w * 8 + it;
      const bf16x8 xr = lds8<SLAB>(lre + (8 * h) * SLAB + n2 * ROW + j);
      const bf16x8 xi = lds8<SLAB>(lim + (8 * h) * SLAB + n2 * ROW + j);
      f32x16 z = {};
      f32x16 o = mfma(A[M1I_R], xr, z);
      o = mfma(A[M1I_I], xi, o);
      // rows 4h + e (e < 4) are n1 = 4h + e (< 8): real part in o[e], imaginary part in o[8 + e]
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = j + 32 * n2 + 1024 * (4 * h + e);
        float a = o[e], b = o[8 + e];
        if (GATE) {
          a *= (float)gate[base0 + n];
          b *= (float)gate[base1 + n];
        }
        y[base0 + n] = tobf(a);
        y[base1 + n] = tobf(b);
      }
    }
  }
}

// Pair-order spectrum: Hc[d][k1][v][lane] = H[k]/N as bf16 (re low, im high), k = k1 + 16 (lane%32)
// + 512 k3(v, lane/32); H from the natural-order bins 0..L (upper bins by conjugate symmetry).
__global__ void k_pair_spectrum(const float2* __restrict__ Hnat, uint32_t* __restrict__ Hc) {
  using namespace mf;
  const int d = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;    // (k1, v, lane)
  if (idx >= 16 * 16 * 64) return;
  const int k1 = idx / (16 * 64), v = (idx / 64) % 16, l = idx % 64;
  const int jj = l & 31, h = l >> 5;
  const int k = k1 + 16 * jj + 512 * acc_row(v, h);
  const float2* hn = Hnat + (size_t)d * (L + 1);
  float2 hv = k <= L ? hn[k] : cconj(hn[N - k]);
  hv = cscale(hv, 1.0f / N);
  const uint32_t lo = (uint32_t)f32_to_bf16_rne(hv.x), hi = (uint32_t)f32_to_bf16_rne(hv.y);
  Hc[(size_t)d * 16 * 16 * 64 + idx] = lo | (hi << 16);
}

// ------------------------------------------------------------------ host side
// DFT matrices per lane in the MFMA A-operand layout (row i = lane % 32, K = 8 (lane / 32) + e).
static float host_mat(int q, int i, int K) {
  const double tp = 2.0 * 3.14159265358979323846;
  auto c = [&](int a, int b, int n) { return cos(tp * (double)((a * b) % n) / n); };
  auto s = [&](int a, int b, int n) { return sin(tp * (double)((a * b) % n) / n); };
  auto perm = [](int Kp) {   // permuted input order of the pass-3' matrix: K' -> k3
    const int hh = (Kp >> 3) & 1, e = Kp & 7, hi = Kp >> 4;
    return 16 * hi + (e < 4 ? 4 * hh + e : 8 + 4 * hh + e - 4);
  };
  switch (q) {
    case mf::M1F: {   // radix 16, inputs m < 8: rows (Yr k | Yi k), cols (Xr m | Xi m)
      const int k = i & 15, m = K & 7;
      const bool yi = i >= 16, xi = K >= 8;
      if (!yi) return (float)(xi ? s(k, m, 16) : c(k, m, 16));
      return (float)(xi ? c(k, m, 16) : -s(k, m, 16));
    }
    case mf::C_LO: return (float)c(i, K, 32);
    case mf::C_HI: return (float)c(i, K + 16, 32);
    case mf::S_LO: return (float)s(i, K, 32);
    case mf::S_HI: return (float)s(i, K + 16, 32);
    case mf::CP_LO: return (float)c(i, perm(K), 32);
    case mf::CP_HI: return (float)c(i, perm(K + 16), 32);
    case mf::SP_LO: return (float)s(i, perm(K), 32);
    case mf::SP_HI: return (float)s(i, perm(K + 16), 32);
    case mf::M1I_R: {  // inverse radix 16, Xr block: Yr = c, Yi = s
      const int n = i & 15;
      return (float)(i < 16 ? c(n, K, 16) : s(n, K, 16));
    }
    case mf::M1I_I: {  // Xi block: Yr = -s, Yi = c
      const int n = i & 15;
      return (float)(i < 16 ? -s(n, K, 16) : c(n, K, 16));
    }
  }
  return 0.f;
}

void mfma_matrices_host(uint16_t* out) {   // [NMAT][64 lanes][8]
  for (int q = 0; q < mf::NMAT; ++q)
    for (int l = 0; l < 64; ++l)
      for (int e = 0; e < 8; ++e) {
        const float f = host_mat(q, l % 32, 8 * (l / 32) + e);
        uint32_t u;
        memcpy(&u, &f, 4);
        u += 0x7fffu + ((u >> 16) & 1u);
        out[(q * 64 + l) * 8 + e] = (uint16_t)(u >> 16);
      }
}
size_t mfma_matrices_count() { return (size_t)mf::NMAT * 64 * 8; }

bool mfma_pair_supported(int log2L, int B) { return log2L == 13 && B % 2 == 0; }
size_t mfma_pair_spectrum_bytes_per_channel() { return (size_t)16 * 16 * 64 * 4; }

hipError_t launch_conv_mfma(const void* u, const void* gate, void* y, const void* Hc, const void* mats, int B, int D,
                            const Twiddles& tw, hipStream_t s) {
  const dim3 grid(D * (B / 2)), block(mf::T);
  if (gate)
    hipLaunchKernelGGL((k_conv_mfma<true>), grid, block, 0, s, (const __bf16*)u, (const __bf16*)gate, (__bf16*)y,
                       (const uint32_t*)Hc, (const bf16x8*)mats, B, D, tw);
  else
    hipLaunchKernelGGL((k_conv_mfma<false>), grid, block, 0, s, (const __bf16*)u, (const __bf16*)nullptr,
                       (__bf16*)y, (const uint32_t*)Hc, (const bf16x8*)mats, B, D, tw);
  return hipGetLastError();
}

hipError_t launch_pair_spectrum(const float2* Hnat, void* Hc, int D, hipStream_t s) {
  hipLaunchKernelGGL(k_pair_spectrum, dim3((16 * 16 * 64 + 255) / 256, D), dim3(256), 0, s, Hnat, (uint32_t*)Hc);
  return hipGetLastError();
}

}  // namespace hyena
