// Input projection (Hyena study note, step 1: v, x_1, ..., x_N = split(W_proj x), a learned linear map
// of the token-major input; the listing chunks the projected channels into N + 1 equal parts, v first).
//
// For x [B, L, K] (token-major) and W [M, K] (M = (N+1) D, one row per output channel) the product
// C[c, t] = sum_k W[c, k] x[b, t, k] (+ bias[c]) is formed directly in channel-major orientation (rows
// c, columns t), so row c lands in out_{c / D}[b, c mod D, t]: the channel-last -> channel-major change
// of layout that the convolution needs costs no pass of its own.  Both operands are contiguous in k,
// which is the order the matrix-core operands want (lane l holds 8 consecutive k of row l mod 32).
//
// A workgroup owns a tile of channels x tokens of one sample, split among its waves in blocks of 32 x 32
// accumulators.  k advances in tiles, staged through LDS and double-buffered through registers (the
// next tile's global loads are in flight while the current one is multiplied).  Global loads go through
// raw buffer descriptors: rows past the last channel or token read zero.
#include "launch.h"

namespace hyena {

namespace {
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 pj_bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float pj_f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t pj_u32x4;
// raw buffer descriptor word 3: 32-bit data format, offsets beyond the record count read zero
constexpr int kProjRsrcWord3 = 0x00020000;

template <bool BF16> struct ProjT;
template <> struct ProjT<true> {
  using E = uint16_t;                         // bf16 storage
  static constexpr int ES = 2, PAD = 8;       // LDS rows padded by 16 bytes: conflict-free 16-byte reads
};
template <> struct ProjT<false> {
  using E = float;
  static constexpr int ES = 4, PAD = 4;
};

// Tile shape: WM x WN waves, each owning FM x FN blocks of 32 x 32 accumulators; k tiles of BK.
template <int WM_, int WN_, int FM_, int FN_, int BK_>
struct ProjCfg {
  static constexpr int WM = WM_, WN = WN_, FM = FM_, FN = FN_, BK = BK_;
  static constexpr int T = WM * WN * 64, BM = WM * FM * 32, BN = WN * FN * 32;
};
// 256 channels x 256 tokens per workgroup, 8 waves of 64 x 128 (measured against 128 x 128 and 256 x 128
// tiles, 4 to 16 waves, 1 or 2 waves per SIMD: this shape ran fastest on the layer's shapes)
using PCB = ProjCfg<4, 2, 2, 4, 64>;          // bf16 operands
using PCF = ProjCfg<4, 2, 2, 4, 32>;          // fp32 operands (k tile halved: LDS)

struct ProjOut {
  void* p[kProjMaxOut];
};

template <bool BF16, class C>
__global__ void __launch_bounds__(C::T)
k_proj(const void* __restrict__ x, const void* __restrict__ W, const float* __restrict__ bias, ProjOut out,
       int L, int K, int M, int D, int tiles_c, int tiles_t, int vec_store) {
  using P = ProjT<BF16>;
  using E = typename P::E;
  constexpr int T = C::T, BM = C::BM, BN = C::BN, BK = C::BK, FM = C::FM, FN = C::FN, WM = C::WM;
  constexpr int ES = P::ES, LDK = BK + P::PAD;
  constexpr int CPR = BK * ES / 16;           // 16-byte chunks per tile row
  constexpr int CHA = BM * CPR / T, CHB = BN * CPR / T;
  static_assert((BM * CPR) % T == 0 && (BN * CPR) % T == 0, "tile");
  // one LDS array: two k-tile buffers of each operand, reused by the epilogue's staging
  __shared__ __align__(16) E lds[2 * (BM + BN) * LDK];
  E* const As = lds;                          // buffer q at As + q * BM * LDK
  E* const Bs = lds + 2 * BM * LDK;           // buffer q at Bs + q * BN * LDK
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ct = lb % tiles_c, rest = lb / tiles_c;
  const int tt = rest % tiles_t, b = rest / tiles_t;
  const int c0 = ct * BM, t0 = tt * BN;

  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(W), (short)0, M * K * ES, kProjRsrcWord3);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)x + (size_t)b * L * K * ES), (short)0, L * K * ES, kProjRsrcWord3);
  // chunk r of this thread: tile row, k offset within the tile (elements), LDS offset
  int voa[CHA], loa[CHA], koa[CHA], vob[CHB], lob[CHB], kob[CHB];
#pragma unroll
  for (int r = 0; r < CHA; ++r) {
    const int i = tid + T * r, row = i / CPR, cc = i % CPR;
    voa[r] = (c0 + row) * K * ES + cc * 16;
    koa[r] = cc * (16 / ES);
    loa[r] = row * LDK + koa[r];
  }
#pragma unroll
  for (int r = 0; r < CHB; ++r) {
    const int i = tid + T * r, row = i / CPR, cc = i % CPR;
    vob[r] = (t0 + row) * K * ES + cc * 16;
    kob[r] = cc * (16 / ES);
    lob[r] = row * LDK + kob[r];
  }
  pj_u32x4 ra[CHA], rb[CHB];
  // in the last, partial k tile a chunk past the last k of a row would read the next row: it is zero
  auto gload = [&](int k0, bool tail) {
#pragma unroll
    for (int r = 0; r < CHA; ++r)
      ra[r] = !tail || k0 + koa[r] < K
                  ? __builtin_bit_cast(pj_u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, voa[r], k0 * ES, 0))
                  : pj_u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < CHB; ++r)
      rb[r] = !tail || k0 + kob[r] < K
                  ? __builtin_bit_cast(pj_u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, vob[r], k0 * ES, 0))
                  : pj_u32x4{0u, 0u, 0u, 0u};
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < CHA; ++r) *reinterpret_cast<pj_u32x4*>(As + buf * BM * LDK + loa[r]) = ra[r];
#pragma unroll
    for (int r = 0; r < CHB; ++r) *reinterpret_cast<pj_u32x4*>(Bs + buf * BN * LDK + lob[r]) = rb[r];
  };

  pj_f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int ra_row = wm * FM * 32 + (lane & 31), rb_row = wn * FN * 32 + (lane & 31), hk = lane >> 5;
  auto compute = [&](int buf) {
    if constexpr (BF16) {
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        pj_bf16x8 a[FM], bb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          a[i] = *reinterpret_cast<const pj_bf16x8*>(As + buf * BM * LDK + (ra_row + 32 * i) * LDK + 16 * s + 8 * hk);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bb[j] = *reinterpret_cast<const pj_bf16x8*>(Bs + buf * BN * LDK + (rb_row + 32 * j) * LDK + 16 * s + 8 * hk);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < BK / 2; ++s) {
        float a[FM], bb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = As[buf * BM * LDK + (ra_row + 32 * i) * LDK + 2 * s + hk];
#pragma unroll
        for (int j = 0; j < FN; ++j) bb[j] = Bs[buf * BN * LDK + (rb_row + 32 * j) * LDK + 2 * s + hk];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], bb[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  const int nk = (K + BK - 1) / BK, nfull = K / BK;
  if (nfull > 0) gload(0, false);
  else gload(0, true);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nfull) gload((kt + 1) * BK, false);
    else if (kt + 1 < nk) gload((kt + 1) * BK, true);
    compute(cur);
    // buffer cur ^ 1 was last read in the previous iteration, before the barrier that ended it
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: accumulator register v of lane (col, h) holds row 8 (v / 4) + 4 h + (v mod 4), column col
  const int h = lane >> 5, col = lane & 31;
  const int wc0 = c0 + wm * FM * 32, wt0 = t0 + wn * FN * 32;
  if constexpr (BF16) {
    if (vec_store) {
      // through LDS: the wave's 64 x 128 block as bf16 rows, then 16-byte stores of 8 tokens each
      constexpr int RW = FN * 32 + 8;                      // LDS row stride of the block (elements)
      static_assert(WM * C::WN * FM * 32 * RW <= 2 * (BM + BN) * LDK, "epilogue staging fits the tiles");
      __bf16* st = reinterpret_cast<__bf16*>(lds) + wave * (FM * 32 * RW);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          const int c = wc0 + r;
          const float bc = (bias && c < M) ? bias[c] : 0.0f;
#pragma unroll
          for (int jj = 0; jj < FN; ++jj) st[r * RW + 32 * jj + col] = (__bf16)(acc[i][jj][v] + bc);   // RNE
        }
      __syncthreads();
      constexpr int CPRW = FN * 32 / 8;                    // 16-byte chunks per block row
      constexpr int ITER = FM * 32 * CPRW / 64;
      constexpr int RSTEP = 64 / CPRW;                     // rows advanced per iteration
      // output chunk and channel of this lane's first row (wc0 is wave-uniform), then stepped by RSTEP
      int r = lane / CPRW;
      int j = (wc0 + r) / D, d = wc0 + r - j * D;
      const int ch = lane % CPRW, t = wt0 + 8 * ch;
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        if (wc0 + r < M && t < L) {
          E* dst = static_cast<E*>(out.p[j]) + ((size_t)b * D + d) * L + t;
          *reinterpret_cast<pj_u32x4*>(dst) = *reinterpret_cast<const pj_u32x4*>(&st[r * RW + 8 * ch]);
        }
        r += RSTEP;
        d += RSTEP;
        while (d >= D) {
          d -= D;
          ++j;
        }
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int c = wc0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
      if (c >= M) continue;
      const int j = c / D, d = c - j * D;
      const float bc = bias ? bias[c] : 0.0f;
      E* orow = static_cast<E*>(out.p[j]) + ((size_t)b * D + d) * L;
#pragma unroll
      for (int jj = 0; jj < FN; ++jj) {
        const int t = wt0 + 32 * jj + col;
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
  const int BM = es == 2 ? PCB::BM : PCF::BM, BN = es == 2 ? PCB::BN : PCF::BN;
  if (K % (16 / es)) return false;            // whole 16-byte chunks per row
  if ((M + BM) * K * es >= ((int64_t)1 << 31) || (L + BN) * K * es >= ((int64_t)1 << 31)) return false;
  const int64_t tiles = ((M + BM - 1) / BM) * ((L + BN - 1) / BN) * B;
  return tiles < ((int64_t)1 << 31);
}

namespace {
template <bool BF16, class C>
hipError_t proj_launch(const void* x, const void* W, const float* bias, const ProjOut& o, int nout, int B, int L,
                       int K, int M, int D, hipStream_t s) {
  const int tiles_c = (M + C::BM - 1) / C::BM, tiles_t = (L + C::BN - 1) / C::BN;
  const dim3 grid((unsigned)(tiles_c * tiles_t * B));
  // 16-byte stores of 8 bf16 tokens when every output row starts 16-byte aligned
  int vec = BF16 && L % 8 == 0;
  for (int j = 0; j < nout; ++j) vec = vec && (reinterpret_cast<uintptr_t>(o.p[j]) & 15u) == 0;
  hipLaunchKernelGGL((k_proj<BF16, C>), grid, dim3(C::T), 0, s, x, W, bias, o, L, K, M, D, tiles_c, tiles_t, vec);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_projection(int bf16, const void* x, const void* W, const float* bias, void* const* outs, int nout,
                             int B, int L, int K, int D, hipStream_t s) {
  if (nout < 1 || nout > kProjMaxOut) return hipErrorInvalidValue;
  ProjOut o{};
  for (int j = 0; j < nout; ++j) o.p[j] = outs[j];
  const int M = nout * D;
  return bf16 ? proj_launch<true, PCB>(x, W, bias, o, nout, B, L, K, M, D, s)
              : proj_launch<false, PCF>(x, W, bias, o, nout, B, L, K, M, D, s);
}

}  // namespace hyena
