// Multi-pass ("four-step") causal long convolution for 2^15 <= L <= 2^20, where one row's transform
// does not fit in LDS.  Same operation as the single-pass kernels (Hyena study note, steps 2-3;
// EulerStack "4. Hyena 상세", how it works 2; HyenaND summary, boundary handling and nSubQ fusion):
// the packed row z[n] = u[2n] + i u[2n+1] (zero for n >= M/2, M = L) is transformed as an
// M1 x M2 matrix, n = n2 + M2 n1, bin k = k1 + M1 k2:
//
//   pass A  (k_fs_cols)  columns n2: M1-point DFT over n1 (upper half of the input is zero)
//   pass B  (k_fs_rows)  rows k1 and M1-k1 together: twiddle W_M^{n2 k1}, M2-point DFT over n2,
//                        mirrored-bin split, product with the filter spectrum, re-pack, inverse
//                        M2-point DFT, conjugate twiddle
//   pass C  (k_fs_cols)  columns: inverse M1-point DFT, keep n1 < M1/2 (the causal half), gate;
//                        for every order but the last the same workgroup then runs the next
//                        order's pass A on the gated tile, so u_i never goes to HBM
//
// Periodic boundary (FULL; HyenaND summary, boundary handling: circular convolution, no padding): a
// row of L = 2M samples fills all M packed values, pass A loads every n1 and pass C keeps every n1,
// so the same passes compute the L-point circular convolution (the row pass is unchanged).
//
// The intermediate is one complex M-vector per row.  fp32 storage keeps it in fp32.  With bf16 storage (only v,
// the gates and y are bf16) it is held in fp16 with block scaling: every block of values written by one
// workgroup is scaled by a power of two that brings its largest component into [2^14, 2^15) and rounded to
// fp16 (11-bit significand, half the bytes of fp32), its exponent stored beside the row; the reader scales
// back in fp32.  Rounding to bf16 instead (8 bits) compounds across passes and orders into errors beyond what
// bf16 storage is allowed; u_i itself stays fp32 from one order to the next (it lives in LDS between pass C
// and the next pass A).  Rows are processed in chunks whose intermediates stay resident in L2 / the
// memory-side cache.  Rows are visited channel-major (q = d*B + b) so the B rows of a channel read its filter
// spectrum back to back.
//
// Spectrum layout per channel: Hs[g][slot][t'] for row-pair group g < M1/2, slot < 2 RP, thread t'
// of the pair (see k_fs_rows); g = 0 holds rows k1 = 0 and k1 = M1/2.  Hs = H / (4M).
#include "engine.h"
#include "launch.h"

namespace hyena {

template <int LOG2M> struct FourStepPlan;
// M1 (columns) x M2 (rows); column radices, row radices (last radix 8, 16 elements per thread)
template <> struct FourStepPlan<15> { using Col = Radices<16, 8>;    using Row = Radices<4, 8, 8>;   static constexpr int G = 4; };
template <> struct FourStepPlan<16> { using Col = Radices<16, 8>;    using Row = Radices<8, 8, 8>;   static constexpr int G = 2; };
template <> struct FourStepPlan<17> { using Col = Radices<16, 16>;   using Row = Radices<8, 8, 8>;   static constexpr int G = 2; };
template <> struct FourStepPlan<18> { using Col = Radices<16, 16>;   using Row = Radices<16, 8, 8>;  static constexpr int G = 1; };
template <> struct FourStepPlan<19> { using Col = Radices<8, 8, 8>;  using Row = Radices<16, 8, 8>;  static constexpr int G = 1; };
template <> struct FourStepPlan<20> { using Col = Radices<8, 8, 8>;  using Row = Radices<16, 16, 8>; static constexpr int G = 1; };

// Block-scaled fp16 intermediate: a row's region of M + 1024 32-bit words holds the M values as fp16 pairs
// (real low, imaginary high) in [0, M), the exponents of pass A's column tiles (M / 8192 <= 128 of them) from
// word M + EA, and the exponents of pass B's workgroups, one per bin-row position (M1 <= 512), from M + EB.
struct H16Row {
  static constexpr int EA = 0, EB = 128;   // offsets from word M
  static constexpr int EXTRA = 1024;       // words after the values
};
__device__ __forceinline__ uint32_t h16_pack(float2 v, float s) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 r = {(_Float16)(v.x * s), (_Float16)(v.y * s)};
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float2 h16_unpack(uint32_t w, float s) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 r = __builtin_bit_cast(h2, w);
  return make_float2((float)r.x * s, (float)r.y * s);
}
// largest value of v over the NT threads of the workgroup (red: NT / 64 floats of LDS); every thread returns it.
// The caller's next barrier must not be this one's.
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int k = 1; k < NT / 64; ++k) m = fmaxf(m, red[k]);
  return m;
}

template <int LOG2M>
struct FS {
  using Plan = FourStepPlan<LOG2M>;
  using ColRL = typename Plan::Col;
  using RowRL = typename Plan::Row;
  static constexpr int M = 1 << LOG2M;
  static constexpr int M1 = ColRL::S, M2 = RowRL::S;
  static_assert(M1 * M2 == M, "plan");
  // column tiles: C columns x M1 positions = 8192 complex in LDS
  static constexpr int TILE = 8192;
  static constexpr int C = TILE / M1;
  static constexpr int TC = 512;
  // 16-column tiles take the swizzled unpadded layout (conflict-free 64-bit accesses), wider ones padding
  using Col = ColEngine<C, C, 1, TC, ColRL, C != 16, C == 16>;
  // row pairs
  static constexpr int G = Plan::G;
  using Row = RowEngine<2 * G, RowRL>;
  static constexpr int RP = RowRL::RP;
  static constexpr int TP = M2 / RP;              // threads per row pair
  static constexpr int TR = Row::T;               // = G * TP
  static_assert(TR == G * TP, "row engine threads");
};

// ----------------------------------------------------------------------------------------------
// pass A / pass C (+A of the next order).  MODE: 0 = A from u (load u, forward columns, store I)
//                                                1 = C (+A): inverse columns, gate, [forward, store I] or store y
// grid.x = tiles * rows_in_chunk (row fastest); one workgroup = one column tile of one row.
template <int LOG2M, bool BF16, int MODE, bool GATE, bool CHAIN, bool FULL>
__global__ void __launch_bounds__(FS<LOG2M>::TC)
k_fs_cols(const typename Store<BF16>::elem* u, const typename Store<BF16>::elem* gate,
          typename Store<BF16>::elem* y, float2* I, int q0, int nq, int B, int D, Twiddles tw) {
  using F = FS<LOG2M>;
  using St = Store<BF16>;
  constexpr int M = F::M, M1 = F::M1, M2 = F::M2, C = F::C, TC = F::TC;
  constexpr int PER_T = C * M1 / TC;              // tile elements per thread
  constexpr int PER_IO = FULL ? PER_T : PER_T / 2;  // of them loaded from u / stored to y
  constexpr int RS = FULL ? 2 * M : M;            // samples per row
  __shared__ float2 lds[lds_padded_size(C * M1)];
  const int t = threadIdx.x;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ql = lb % nq, tile = lb / nq;
  const int q = q0 + ql;
  const int d = q / B, b = q % B;
  const size_t row = (size_t)b * D + d;
  const int c0 = tile * C;
  constexpr bool H16 = BF16;
  float2* Irow = I + (size_t)ql * M;
  // the fp16 form (bf16 storage): rows of M + EXTRA words
  uint32_t* const Wrow = reinterpret_cast<uint32_t*>(I) + (size_t)ql * (M + H16Row::EXTRA);
  static_assert(!H16 || M / 8192 <= 128, "tile exponents");
  auto tile_addr = [&](int p, int c) { return F::Col::addr(p, c); };

  if constexpr (MODE == 0) {
    // load the packed row: positions n1 < M1/2 (the rest is the zero padding), or all of them (FULL)
    const auto* urow = u + row * RS;
    static_for<PER_IO>([&](auto ii) {
      const int e = t + TC * ii.value;
      const int p = e / C, c = e % C;
      lds[tile_addr(p, c)] = St::load2(urow + 2 * ((size_t)(c0 + c) + (size_t)M2 * p));
    });
    __syncthreads();
  } else {
    if constexpr (H16) {
      __shared__ float rsc[M1];   // 2^e of pass B's block that wrote bin-row position p
      for (int p = t; p < M1; p += TC) rsc[p] = __builtin_ldexpf(1.0f, (int)Wrow[M + H16Row::EB + p]);
      __syncthreads();
      static_for<PER_T>([&](auto ii) {
        const int e = t + TC * ii.value;
        const int p = e / C, c = e % C;
        lds[tile_addr(p, c)] = h16_unpack(Wrow[(size_t)p * M2 + c0 + c], rsc[p]);
      });
    } else {
      static_for<PER_T>([&](auto ii) {
        const int e = t + TC * ii.value;
        const int p = e / C, c = e % C;
        lds[tile_addr(p, c)] = Irow[(size_t)p * M2 + c0 + c];
      });
    }
    __syncthreads();
    F::Col::template inverse<!FULL>(lds, tw, t);
    // gate the causal half (positions n1 < M1/2 are z'[n2 + M2 n1]), or every position (FULL)
    const auto* grow = GATE ? gate + row * RS : nullptr;
    auto* yrow = CHAIN ? nullptr : y + row * RS;
    static_for<PER_IO>([&](auto ii) {
      const int e = t + TC * ii.value;
      const int p = e / C, c = e % C;
      const size_t j = (size_t)(c0 + c) + (size_t)M2 * p;
      float2 v = lds[tile_addr(p, c)];
      if constexpr (GATE) {
        const float2 g = St::load2(grow + 2 * j);
        v = make_float2(v.x * g.x, v.y * g.y);
      }
      if constexpr (CHAIN) {
        lds[tile_addr(p, c)] = v;             // the next order's input, kept in fp32
      } else {
        St::store2(yrow + 2 * j, v);
      }
    });
    if constexpr (!CHAIN) return;
    __syncthreads();
  }
  F::Col::template forward<!FULL>(lds, tw, t);
  if constexpr (H16) {
    // the tile's values, their largest component over the workgroup, then the scaled fp16 store
    __shared__ float red[TC / 64];
    float2 vals[PER_T];
    float m = 0.0f;
    static_for<PER_T>([&](auto ii) {
      const int e = t + TC * ii.value;
      vals[ii.value] = lds[tile_addr(e / C, e % C)];
      m = fmaxf(m, fmaxf(fabsf(vals[ii.value].x), fabsf(vals[ii.value].y)));
    });
    const int ex = h16_exponent(block_max<TC>(m, red));
    const float sc = __builtin_ldexpf(1.0f, -ex);
    static_for<PER_T>([&](auto ii) {
      const int e = t + TC * ii.value;
      const int p = e / C, c = e % C;
      Wrow[(size_t)p * M2 + c0 + c] = h16_pack(vals[ii.value], sc);
    });
    if (t == 0) Wrow[M + H16Row::EA + tile] = (uint32_t)ex;
  } else {
    static_for<PER_T>([&](auto ii) {
      const int e = t + TC * ii.value;
      const int p = e / C, c = e % C;
      Irow[(size_t)p * M2 + c0 + c] = lds[tile_addr(p, c)];
    });
  }
}

// Spectrum pass A: fp32 taps h[d, 0:M) zero-padded, or h[d, 0:2M) (FULL; one "row" per channel, B = 1).
template <int LOG2M, bool FULL>
__global__ void __launch_bounds__(FS<LOG2M>::TC)
k_fs_cols_taps(const float* h, float2* I, int q0, int nq, Twiddles tw) {
  using F = FS<LOG2M>;
  constexpr int M = F::M, M1 = F::M1, M2 = F::M2, C = F::C, TC = F::TC;
  constexpr int PER_T = C * M1 / TC;
  __shared__ float2 lds[lds_padded_size(C * M1)];
  const int t = threadIdx.x;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ql = lb % nq, tile = lb / nq;
  const int d = q0 + ql;
  const int c0 = tile * C;
  const float* hrow = h + (size_t)d * (FULL ? 2 * M : M);
  static_for<FULL ? PER_T : PER_T / 2>([&](auto ii) {
    const int e = t + TC * ii.value;
    const int p = e / C, c = e % C;
    lds[F::Col::addr(p, c)] = Store<false>::load2(hrow + 2 * ((size_t)(c0 + c) + (size_t)M2 * p));
  });
  __syncthreads();
  F::Col::template forward<!FULL>(lds, tw, t);
  float2* Irow = I + (size_t)ql * M;
  static_for<PER_T>([&](auto ii) {
    const int e = t + TC * ii.value;
    const int p = e / C, c = e % C;
    Irow[(size_t)p * M2 + c0 + c] = lds[F::Col::addr(p, c)];
  });
}

// ----------------------------------------------------------------------------------------------
// pass B.  MODE 0: convolution (spectral product with Hs); MODE 1: write the filter spectrum.
// Workgroup = G row pairs of one row; pair g_glob = group*G + j covers bin rows k1 = g_glob and
// M1 - g_glob (g_glob = 0: rows 0 and M1/2).  In the last pass, thread t' < TP of a pair holds block
// beta_A = t' of the first row and beta_B = NBLK-1-t' of the second (their bins mirror each other:
// k <-> M-k pairs k1 with M1-k1 and complements every k2 digit); the g_glob = 0 pair instead uses
// whole-row negation pairing on row 0 (threads < TP/2) and in-row complement pairing on row M1/2.
// H16: the intermediate is block-scaled fp16 (bf16 storage, MODE 0 only).
template <int LOG2M, int MODE, bool H16>
__global__ void __launch_bounds__(FS<LOG2M>::TR)
k_fs_rows(float2* I, const float2* __restrict__ Hs, float2* __restrict__ Hs_out, int q0, int nq, int B, int hsb,
          Twiddles tw) {
  using F = FS<LOG2M>;
  using Row = typename F::Row;
  using RL = typename F::RowRL;
  constexpr int M = F::M, M1 = F::M1, M2 = F::M2, G = F::G, TP = F::TP, TR = F::TR, RP = F::RP;
  constexpr int E = Row::E, R0 = RL::R[0], PER0 = M2 / R0, NBLK = Row::NBLK;
  __shared__ float2 lds[Row::LDS_ELEMS];
  const int t = threadIdx.x;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ql = lb % nq, grp = lb / nq;
  const int q = q0 + ql;
  // spectrum channel: d (one filter per channel, hsb = 0) or b * D + d (one per (b, d), hsb = D)
  const int d = (MODE == 0) ? q / B + (q % B) * hsb : q;
  float2* Irow = I + (size_t)ql * M;
  uint32_t* const Wrow = reinterpret_cast<uint32_t*>(I) + (size_t)ql * (M + H16Row::EXTRA);
  static_assert(!H16 || MODE == 0, "fp16 intermediate in the convolution only");
  constexpr int NTILE = M / 8192, TCOL = M2 / NTILE;   // pass A's column tiles: TCOL columns each
  __shared__ float tsc[H16 ? NTILE : 1];               // 2^e of pass A's tiles
  if constexpr (H16) {
    for (int k = t; k < NTILE; k += TR) tsc[k] = __builtin_ldexpf(1.0f, (int)Wrow[M + H16Row::EA + k]);
    __syncthreads();
  }

  // bin row k1 of sub-row s (s = 2j: first of pair j, 2j+1: second)
  auto k1_of = [&](int s) {
    const int gg = grp * G + s / 2;
    if (gg == 0) return (s & 1) ? M1 / 2 : 0;
    return (s & 1) ? M1 - gg : gg;
  };

  // load + forward twiddle W_M^{n2 k1}: element m of butterfly i is column n + m * PER0
  float2 x[E];
  static_for<E / R0>([&](auto ii) {
    constexpr int i = ii.value;
    int s, n;
    Row::first_input(t, i, s, n);
    const int k1 = k1_of(s);
    const size_t roff = (size_t)F::ColRL::position_of_bin(k1) * M2;
    // W_M^{(n + m PER0) k1} for m = 0..R0-1 as a running product from W_M^{n k1} by W_M^{PER0 k1}
    const float2 ws = twiddle<LOG2M>(tw, uint32_t(PER0) * uint32_t(k1));
    float2 w = twiddle<LOG2M>(tw, uint32_t(n) * uint32_t(k1));
    static_for<R0>([&](auto m) {
      const int col = n + m.value * PER0;
      const float2 v = H16 ? h16_unpack(Wrow[roff + col], tsc[col / TCOL]) : Irow[roff + col];
      x[i * R0 + m.value] = cmul(v, w);
      if constexpr (m.value + 1 < R0) w = cmul(w, ws);
    });
  });
  Row::template forward_to_last<false>(x, lds, tw, t);

  // last-pass assignment
  const int j = t / TP, tp = t % TP;                 // pair within the workgroup, thread within pair
  const int gg = grp * G + j;
  int bA, bB, kapA, kapB, k1A;
  bool selfmirror = false;
  if (gg != 0) {
    bA = (2 * j) * NBLK + tp;
    bB = (2 * j + 1) * NBLK + (NBLK - 1 - tp);
    kapA = RL::kappa_of_block(tp);
    kapB = 0;
    k1A = gg;
  } else if (tp < TP / 2) {                          // row k1 = 0, negation pairing
    const auto np = NegPairs<RL>::of(tp);
    bA = (2 * j) * NBLK + np.betaA;
    bB = (2 * j) * NBLK + np.betaB;
    kapA = np.kapA; kapB = np.kapB;
    selfmirror = np.special;
    k1A = 0;
  } else {                                           // row k1 = M1/2, in-row complement pairing
    const int tq = tp - TP / 2;
    bA = (2 * j + 1) * NBLK + tq;
    bB = (2 * j + 1) * NBLK + (NBLK - 1 - tq);
    kapA = RL::kappa_of_block(tq);
    kapB = 0;
    k1A = M1 / 2;
  }
  Row::fwd_last(x, lds, bA, bB);

  const size_t hoff = (size_t)d * M + (size_t)gg * (2 * RP * TP) + tp;
  if (!selfmirror) {
    const float2 wA = twiddle<LOG2M + 1>(tw, uint32_t(k1A) + uint32_t(M1) * uint32_t(kapA));
    if constexpr (MODE == 0) spectral_complement<RP, 0>(x, wA, Hs + hoff, TP, nullptr, 0.f);
    else spectral_complement<RP, 1, float2>(x, wA, nullptr, TP, Hs_out + hoff, 1.0f / (8.0f * M));
  } else {
    const float2 wB = twiddle<LOG2M + 1>(tw, uint32_t(M1) * uint32_t(kapB));
    if constexpr (MODE == 0) spectral_selfmirror<RP, 0>(x, wB, Hs + hoff, TP, nullptr, 0.f);
    else spectral_selfmirror<RP, 1, float2>(x, wB, nullptr, TP, Hs_out + hoff, 1.0f / (8.0f * M));
  }
  if constexpr (MODE == 1) return;

  Row::inv_last(x, lds, bA, bB);
  Row::template inverse_from_last<false>(x, lds, tw, t);
  // fp16 form: one power of two for the workgroup's rows (the twiddle below keeps magnitudes), recorded at
  // each of its bin-row positions
  float sc = 1.0f;
  if constexpr (H16) {
    __shared__ float red[TR / 64 > 0 ? TR / 64 : 1];
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < E; ++k) m = fmaxf(m, fmaxf(fabsf(x[k].x), fabsf(x[k].y)));
    const int ex = h16_exponent(block_max<TR>(m, red));
    sc = __builtin_ldexpf(1.0f, -ex);
    if (t < 2 * G) Wrow[M + H16Row::EB + F::ColRL::position_of_bin(k1_of(t))] = (uint32_t)ex;
  }
  // conjugate twiddle and store back
  static_for<E / R0>([&](auto ii) {
    constexpr int i = ii.value;
    int s, n;
    Row::first_input(t, i, s, n);
    const int k1 = k1_of(s);
    const size_t roff = (size_t)F::ColRL::position_of_bin(k1) * M2;
    const float2 ws = twiddle<LOG2M>(tw, uint32_t(PER0) * uint32_t(k1));
    float2 w = twiddle<LOG2M>(tw, uint32_t(n) * uint32_t(k1));
    static_for<R0>([&](auto m) {
      const float2 r = cmulc(x[i * R0 + m.value], w);
      if constexpr (H16) Wrow[roff + n + m.value * PER0] = h16_pack(r, sc);
      else Irow[roff + n + m.value * PER0] = r;
      if constexpr (m.value + 1 < R0) w = cmul(w, ws);
    });
  });
}

// Engine-order spectrum -> H[d, k], k = 0..L (unscaled 2L-point DFT bins); mirrors k_fs_rows' slots.
template <int LOG2M>
__global__ void k_export1d_fs(const float2* __restrict__ Hs, float2* __restrict__ H) {
  using F = FS<LOG2M>;
  using RL = typename F::RowRL;
  constexpr int M = F::M, M1 = F::M1, M2 = F::M2, TP = F::TP, RP = F::RP, NBLK = F::Row::NBLK;
  const int d = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= M) return;
  const int gg = idx / (2 * RP * TP), rem = idx % (2 * RP * TP);
  const int slot = rem / TP, tp = rem % TP;
  const float sc = 4.0f * M;
  const float2 v = Hs[(size_t)d * M + idx];
  float2* out = H + (size_t)d * (M + 1);
  const int m = slot % RP;
  const bool second = slot >= RP;
  int k1, kap;
  if (gg != 0) {
    k1 = second ? M1 - gg : gg;
    kap = RL::kappa_of_block(second ? NBLK - 1 - tp : tp);
  } else if (tp < TP / 2) {
    const auto np = NegPairs<RL>::of(tp);
    if (np.special && slot == 0) {
      out[0] = make_float2(v.x * sc, 0.f);
      out[M] = make_float2(v.y * sc, 0.f);
      return;
    }
    k1 = 0;
    kap = second ? np.kapB : np.kapA;
  } else {
    const int tq = tp - TP / 2;
    k1 = M1 / 2;
    kap = RL::kappa_of_block(second ? NBLK - 1 - tq : tq);
  }
  out[k1 + M1 * (kap + (M2 / RP) * m)] = cscale(v, sc);
}

// ------------------------------------------------------------------ host side
namespace {

template <int LOG2M>
size_t fs_row_bytes() { return (size_t)(1 << LOG2M) * sizeof(float2); }

// Chunks of rows run every pass of every order before the next chunk starts, so a chunk's intermediate is
// reread while the memory-side cache may still hold it; with side streams several chunks run at once, which
// keeps the compute units busy while each chunk stays small (two streams of 64 MB of intermediate measured
// best at L = 2^20: 4.77 ms per step against 5.37 ms for one stream of 160 MB chunks).
template <int LOG2M, bool BF16, bool FULL>
hipError_t fs_conv_launch(int order, int B, int D, const void* v, const void* const* x, const void* const* spectra,
                          void* y, float2* I0, int chunk, const Twiddles& tw, hipStream_t s0, int hsb,
                          const SideStream* side) {
  using F = FS<LOG2M>;
  using E = typename Store<BF16>::elem;
  const int rows = B * D;
  const int tiles = F::M2 / F::C;
  const int groups = (F::M1 / 2) / F::G;
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
    // rows of M float2 (fp32 intermediate) or of M + EXTRA words (fp16, bf16 storage)
    float2* I = I0 + (size_t)j * chunk * (BF16 ? (F::M + H16Row::EXTRA) / 2 : F::M);
    hipLaunchKernelGGL((k_fs_cols<LOG2M, BF16, 0, false, false, FULL>), dim3(tiles * nq), dim3(F::TC), 0, s,
                       (const E*)v, (const E*)nullptr, (E*)nullptr, I, q0, nq, B, D, tw);
    for (int i = 0; i < order; ++i) {
      hipLaunchKernelGGL((k_fs_rows<LOG2M, 0, BF16>), dim3(groups * nq), dim3(F::TR), 0, s, I,
                         (const float2*)spectra[i], (float2*)nullptr, q0, nq, B, hsb, tw);
      if (i + 1 < order)
        hipLaunchKernelGGL((k_fs_cols<LOG2M, BF16, 1, true, true, FULL>), dim3(tiles * nq), dim3(F::TC), 0, s,
                           (const E*)nullptr, (const E*)x[i], (E*)nullptr, I, q0, nq, B, D, tw);
      else if (x[i])
        hipLaunchKernelGGL((k_fs_cols<LOG2M, BF16, 1, true, false, FULL>), dim3(tiles * nq), dim3(F::TC), 0, s,
                           (const E*)nullptr, (const E*)x[i], (E*)y, I, q0, nq, B, D, tw);
      else
        hipLaunchKernelGGL((k_fs_cols<LOG2M, BF16, 1, false, false, FULL>), dim3(tiles * nq), dim3(F::TC), 0, s,
                           (const E*)nullptr, (const E*)nullptr, (E*)y, I, q0, nq, B, D, tw);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return ways > 1 ? side_join(side, s0) : hipSuccess;
}

template <int LOG2M, bool FULL>
hipError_t fs_spectrum_launch(const float* h, float2* Hs, int D, float2* I, int chunk, const Twiddles& tw,
                              hipStream_t s) {
  using F = FS<LOG2M>;
  const int tiles = F::M2 / F::C;
  const int groups = (F::M1 / 2) / F::G;
  for (int q0 = 0; q0 < D; q0 += chunk) {
    const int nq = (D - q0 < chunk) ? D - q0 : chunk;
    hipLaunchKernelGGL((k_fs_cols_taps<LOG2M, FULL>), dim3(tiles * nq), dim3(F::TC), 0, s, h, I, q0, nq, tw);
    hipLaunchKernelGGL((k_fs_rows<LOG2M, 1, false>), dim3(groups * nq), dim3(F::TR), 0, s, I, (const float2*)nullptr,
                       Hs, q0, nq, 1, 0, tw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool fourstep_supported(int log2L) { return log2L >= 15 && log2L <= 20; }

size_t fourstep_row_bytes(int log2L, int bf16) {
  return bf16 ? (((size_t)1 << log2L) + H16Row::EXTRA) * 4 : (size_t)1 << log2L << 3;
}

#define HYENA_FS_CASES(X) X(15) X(16) X(17) X(18) X(19) X(20)

hipError_t launch_export1d_fourstep(int log2L, const float2* Hs, float2* H, int D, hipStream_t s) {
  switch (log2L) {
#define X(n)                                                                                              \
  case n:                                                                                                 \
    hipLaunchKernelGGL((k_export1d_fs<n>), dim3(((1 << n) + 255) / 256, D), dim3(256), 0, s, Hs, H);    \
    return hipGetLastError();
    HYENA_FS_CASES(X)
#undef X
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv1d_fourstep(int log2L, int bf16, int order, int B, int D, const void* v,
                                  const void* const* x, const void* const* spectra, void* y, float2* I, int chunk,
                                  const Twiddles& tw, hipStream_t s, int full, int hsb, const SideStream* side) {
  switch (log2L) {
#define X(n)                                                                                                   \
  case n:                                                                                                      \
    if (full)                                                                                                  \
      return bf16 ? fs_conv_launch<n, true, true>(order, B, D, v, x, spectra, y, I, chunk, tw, s, hsb, side)   \
                  : fs_conv_launch<n, false, true>(order, B, D, v, x, spectra, y, I, chunk, tw, s, hsb, side); \
    return bf16 ? fs_conv_launch<n, true, false>(order, B, D, v, x, spectra, y, I, chunk, tw, s, hsb, side)    \
                : fs_conv_launch<n, false, false>(order, B, D, v, x, spectra, y, I, chunk, tw, s, hsb, side);
    HYENA_FS_CASES(X)
#undef X
  }
  return hipErrorInvalidValue;
}

hipError_t launch_spectrum1d_fourstep(int log2L, const float* h, float2* Hs, int D, float2* I, int chunk,
                                      const Twiddles& tw, hipStream_t s, int full) {
  switch (log2L) {
#define X(n)                                                                           \
  case n:                                                                              \
    return full ? fs_spectrum_launch<n, true>(h, Hs, D, I, chunk, tw, s)               \
                : fs_spectrum_launch<n, false>(h, Hs, D, I, chunk, tw, s);
    HYENA_FS_CASES(X)
#undef X
  }
  return hipErrorInvalidValue;
}

}  // namespace hyena
