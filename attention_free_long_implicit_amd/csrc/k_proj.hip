// Input projection (Hyena study note, step 1: v, x_1, ..., x_N = split(W_proj x), a learned linear map
// of the token-major input; the listing chunks the projected channels into N + 1 equal parts, v first).
//
// For x [B, L, K] (token-major) and W [M, K] (M = (N+1) D, one row per output channel) the product
// C[c, t] = sum_k W[c, k] x[b, t, k] (+ bias[c]) is formed directly in channel-major orientation (rows
// c, columns t), so row c lands in out_{c / D}[b, c mod D, t]: the channel-last -> channel-major change
// of layout that the convolution needs costs no pass of its own.  Both operands are contiguous in k,
// which is the order the matrix-core operands want (lane l holds 8 consecutive k of row l mod 32).
//
// A workgroup owns 128 channels x 128 tokens of one sample; its 4 waves own 64 x 64 each (2 x 2 blocks
// of 32 x 32 accumulators).  k advances in tiles of 32, staged through LDS and double-buffered through
// registers (the next tile's global loads are in flight while the current one is multiplied).  Global
// loads go through raw buffer descriptors: rows past the last channel or token read zero.
#include "launch.h"

namespace hyena {

namespace {
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 pj_bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float pj_f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t pj_u32x4;
// raw buffer descriptor word 3: 32-bit data format, offsets beyond the record count read zero
constexpr int kProjRsrcWord3 = 0x00020000;

namespace pj {
constexpr int BM = 128, BN = 128, BK = 32, T = 256;
}

template <bool BF16> struct ProjT;
template <> struct ProjT<true> {
  using E = uint16_t;                         // bf16 storage
  static constexpr int ES = 2;
  static constexpr int LDK = pj::BK + 8;      // LDS row stride (80 bytes: 16-byte rows, no read conflicts)
};
template <> struct ProjT<false> {
  using E = float;
  static constexpr int ES = 4;
  static constexpr int LDK = pj::BK + 4;      // 144 bytes
};

struct ProjOut {
  void* p[kProjMaxOut];
};

template <bool BF16>
__global__ void __launch_bounds__(pj::T, 2)
k_proj(const void* __restrict__ x, const void* __restrict__ W, const float* __restrict__ bias, ProjOut out,
       int L, int K, int M, int D, int tiles_c, int tiles_t) {
  using namespace pj;
  using P = ProjT<BF16>;
  using E = typename P::E;
  constexpr int ES = P::ES, LDK = P::LDK;
  constexpr int CPR = BK * ES / 16;           // 16-byte chunks per tile row
  constexpr int CH = BM * CPR / T;            // chunks per thread per operand
  static_assert(BM == BN && (BM * CPR) % T == 0, "tile");
  __shared__ __align__(16) E As[2][BM * LDK];
  __shared__ __align__(16) E Bs[2][BN * LDK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ct = lb % tiles_c, rest = lb / tiles_c;
  const int tt = rest % tiles_t, b = rest / tiles_t;
  const int c0 = ct * BM, t0 = tt * BN;

  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(W), (short)0, M * K * ES, kProjRsrcWord3);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)x + (size_t)b * L * K * ES), (short)0, L * K * ES, kProjRsrcWord3);
  int voa[CH], vob[CH], lofs[CH];
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    const int i = tid + T * r, row = i / CPR, cc = i % CPR;
    voa[r] = (c0 + row) * K * ES + cc * 16;
    vob[r] = (t0 + row) * K * ES + cc * 16;
    lofs[r] = row * LDK + cc * (16 / ES);
  }
  pj_u32x4 ra[CH], rb[CH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      ra[r] = __builtin_bit_cast(pj_u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, voa[r], k0 * ES, 0));
      rb[r] = __builtin_bit_cast(pj_u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, vob[r], k0 * ES, 0));
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      *reinterpret_cast<pj_u32x4*>(&As[buf][lofs[r]]) = ra[r];
      *reinterpret_cast<pj_u32x4*>(&Bs[buf][lofs[r]]) = rb[r];
    }
  };

  pj_f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int ra_row = wm * 64 + (lane & 31), rb_row = wn * 64 + (lane & 31), hk = lane >> 5;
  auto compute = [&](int buf) {
    if constexpr (BF16) {
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        pj_bf16x8 a[2], bb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          a[i] = *reinterpret_cast<const pj_bf16x8*>(&As[buf][(ra_row + 32 * i) * LDK + 16 * s + 8 * hk]);
          bb[i] = *reinterpret_cast<const pj_bf16x8*>(&Bs[buf][(rb_row + 32 * i) * LDK + 16 * s + 8 * hk]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < BK / 2; ++s) {
        float a[2], bb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          a[i] = As[buf][(ra_row + 32 * i) * LDK + 2 * s + hk];
          bb[i] = Bs[buf][(rb_row + 32 * i) * LDK + 2 * s + hk];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], bb[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  const int nk = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    compute(cur);
    // buffer cur ^ 1 was last read in the previous iteration, before the barrier that ended it
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: accumulator register v of lane (col, h) holds row 8 (v / 4) + 4 h + (v mod 4), column col
  const int h = lane >> 5, col = lane & 31;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int c = c0 + wm * 64 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
      if (c >= M) continue;
      const int j = c / D, d = c - j * D;
      const float bc = bias ? bias[c] : 0.0f;
      E* orow = static_cast<E*>(out.p[j]) + ((size_t)b * D + d) * L;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int t = t0 + wn * 64 + 32 * jj + col;
        if (t >= L) continue;
        const float val = acc[i][jj][v] + bc;
        if constexpr (BF16) orow[t] = f32_to_bf16_rne(val);
        else orow[t] = val;
      }
    }
  }
}
}  // namespace

bool projection_supported(int64_t B, int64_t L, int64_t K, int64_t M, int es) {
  if (K % pj::BK) return false;
  if ((M + pj::BM) * K * es >= ((int64_t)1 << 31) || (L + pj::BN) * K * es >= ((int64_t)1 << 31)) return false;
  const int64_t tiles = ((M + pj::BM - 1) / pj::BM) * ((L + pj::BN - 1) / pj::BN) * B;
  return tiles < ((int64_t)1 << 31);
}

hipError_t launch_projection(int bf16, const void* x, const void* W, const float* bias, void* const* outs, int nout,
                             int B, int L, int K, int D, hipStream_t s) {
  if (nout < 1 || nout > kProjMaxOut) return hipErrorInvalidValue;
  ProjOut o{};
  for (int j = 0; j < nout; ++j) o.p[j] = outs[j];
  const int M = nout * D;
  const int tiles_c = (M + pj::BM - 1) / pj::BM, tiles_t = (L + pj::BN - 1) / pj::BN;
  const dim3 grid((unsigned)(tiles_c * tiles_t * B));
  if (bf16)
    hipLaunchKernelGGL(k_proj<true>, grid, dim3(pj::T), 0, s, x, W, bias, o, L, K, M, D, tiles_c, tiles_t);
  else
    hipLaunchKernelGGL(k_proj<false>, grid, dim3(pj::T), 0, s, x, W, bias, o, L, K, M, D, tiles_c, tiles_t);
  return hipGetLastError();
}

}  // namespace hyena
