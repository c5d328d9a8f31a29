// Implicit filter taps (Hyena study note, step 2: h(t) = FFN(pos_enc(t)) * w(t), w(t) = exp(-alpha t);
// listing ImplicitFilter: Linear(F -> hidden), SiLU, Linear(hidden -> D); EulerStack YAML
// filter_hidden = 64; HyenaND summary, method: a coordinate network on the grid offsets).
// Positions are normalised (t/L, r/n), so the same parameters serve any grid.
//
//   1-D: phi(t) = [sin(2 pi f t/L), f = 1..F/2] ++ [cos(2 pi f t/L), f = 1..F/2],   window exp(-alpha t/L)
//   3-D: per axis (x, y, z) [sin, cos](2 pi f r_a/n), f = 1..F/6, F/6 sines then F/6 cosines,
//        window exp(-alpha |r|/n); offsets r on [-(n-1), n-1]^3 (zero-padded grid) or the centred
//        period [-n/2, n/2)^3 (periodic grid)
//   g = W2 SiLU(W1 phi + b1) + b2,  W1 [H, F], W2 [D, H];  h[d, pos] = g_d(pos) * window_d(pos)
//
// Phases f t (f r) are reduced modulo L (n) in integers before the sine, so every angle is exact.
// A workgroup owns a tile of 64 positions x 128 channels: the features are formed once per tile, the
// hidden layer and the read-out run as small fp32 matrix-core GEMMs from LDS.  The input-dependent
// filters (one per sample) use the same tiling; see k_film_tiles below.
#include "launch.h"

namespace hyena {

namespace flt {
constexpr int TP = 64;     // positions per tile
constexpr int CB = 128;    // channels per tile
constexpr int T = 256;
}  // namespace flt

// 1-D positions t = 0..L-1
struct FilterGrid1D {
  int L;
  __device__ __forceinline__ int count() const { return L; }
  int count_host() const { return L; }
  // feature pair q (frequency q + 1): sine at column q, cosine at column F/2 + q
  template <int F>
  __device__ __forceinline__ void pair(int pos, int q, int& col_s, int& col_c, float& s, float& c) const {
    const long long ph = ((long long)(q + 1) * pos) % L;
    sincospif(2.0f * (float)ph / (float)L, &s, &c);
    col_s = q;
    col_c = F / 2 + q;
  }
  __device__ __forceinline__ float window_arg(int pos) const { return (float)pos / (float)L; }
  static constexpr int NC = 1;
  __device__ __forceinline__ void coords(int pos, float* c) const { c[0] = (float)pos / (float)L; }
};

// 3-D offsets: W taps per axis, tap index i <-> offset i - R0, grid size n
struct FilterGrid3D {
  int W, R0, n;
  __device__ __forceinline__ int count() const { return W * W * W; }
  int count_host() const { return W * W * W; }
  __device__ __forceinline__ int off(int pos, int ax) const {
    const int i = ax == 0 ? pos / (W * W) : (ax == 1 ? (pos / W) % W : pos % W);
    return i - R0;
  }
  template <int F>
  __device__ __forceinline__ void pair(int pos, int q, int& col_s, int& col_c, float& s, float& c) const {
    constexpr int PER = F / 6;
    const int ax = q / PER, k = q % PER;
    const int ph = (((k + 1) * off(pos, ax)) % n + n) % n;
    sincospif(2.0f * (float)ph / (float)n, &s, &c);
    col_s = ax * 2 * PER + k;
    col_c = ax * 2 * PER + PER + k;
  }
  __device__ __forceinline__ float window_arg(int pos) const {
    const float fx = (float)off(pos, 0) / n, fy = (float)off(pos, 1) / n, fz = (float)off(pos, 2) / n;
    return sqrtf(fx * fx + fy * fy + fz * fz);
  }
  static constexpr int NC = 3;
  __device__ __forceinline__ void coords(int pos, float* c) const {
    for (int ax = 0; ax < 3; ++ax) c[ax] = (float)off(pos, ax) / n;
  }
};

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float flt_f32x16;

// One tile: 64 positions x 128 channels, four waves.  The features go to LDS feature-major; the hidden
// layer (64 positions x 64 units x F) and the read-out (64 positions x 128 channels x 64) run on the fp32
// matrix cores (v_mfma_f32_32x32x2f32): the hidden layer one 32 x 32 block per wave (two accumulators
// over alternate k), the read-out two.  The read-out weights are fetched into registers before the
// hidden layer, so their latency overlaps it; the tile leaves through LDS as [channel][position] rows,
// so the stores run along positions.
template <int F, class G>
__global__ void __launch_bounds__(flt::T)
k_filter_tiles(FilterArgs a, G geo, float* __restrict__ h) {
  using namespace flt;
  constexpr int H = 64;
  constexpr int SK = TP + 4, SC = CB + 4, SH = H + 1, SP = TP + 1;
  constexpr int PHASE1 = 2 * F * SK;                    // w1t [f][j], phiT [f][p]
  constexpr int PHASE2 = H * SC + TP * SH;              // w2t [k][c], act [p][k]
  constexpr int LDSN = PHASE1 > PHASE2 ? PHASE1 : PHASE2;
  static_assert(CB * SP <= LDSN && T == 4 * 64, "tile shape");
  __shared__ __align__(16) float lds[LDSN];
  __shared__ float rarg[TP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hk = lane >> 5;
  const int npos = geo.count();
  const int p0 = blockIdx.x * TP, c0 = blockIdx.y * CB;

  // read-out weights of this channel block, transposed on the way: w2[k][c] = W2[c0 + c][k]
  constexpr int NW2 = H * CB / T;
  float w2r[NW2];
#pragma unroll
  for (int r = 0; r < NW2; ++r) {
    const int i = tid + T * r, k = i / CB, c = i % CB;
    w2r[r] = (c0 + c < a.D) ? a.W2[(size_t)(c0 + c) * H + k] : 0.0f;
  }

  float* w1t = lds;
  float* phiT = lds + F * SK;
  for (int i = tid; i < F * H; i += T) {
    const int j = i / F, f = i % F;
    w1t[f * SK + j] = a.W1[i];
  }
  for (int i = tid; i < TP * (F / 2); i += T) {
    const int p = i / (F / 2), q = i % (F / 2);
    const int pos = min(p0 + p, npos - 1);
    int cs, cc;
    float sv, cv;
    geo.template pair<F>(pos, q, cs, cc, sv, cv);
    phiT[cs * SK + p] = sv;
    phiT[cc * SK + p] = cv;
  }
  if (tid < TP) rarg[tid] = geo.window_arg(min(p0 + tid, npos - 1));
  __syncthreads();

  // hidden layer: wave owns positions 32 pb .. + 31 x units 32 jb .. + 31 (A: phi[p][f], B: W1^T[f][j])
  const int pb = wave & 1, jb = wave >> 1;
  flt_f32x16 acc1[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc1[u][v] = 0.0f;
#pragma unroll 8
  for (int s = 0; s < F / 2; ++s) {
    const int f = 2 * s + hk;
    acc1[s & 1] = __builtin_amdgcn_mfma_f32_32x32x2f32(phiT[f * SK + 32 * pb + l32], w1t[f * SK + 32 * jb + l32],
                                                       acc1[s & 1], 0, 0, 0);
  }
  // register v holds position 32 pb + 8 (v / 4) + 4 hk + (v mod 4) of unit j = 32 jb + l32; SiLU
  float hv[16];
  {
    const float bj = a.b1[32 * jb + l32];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float z = acc1[0][v] + acc1[1][v] + bj;
      hv[v] = __fdividef(z, 1.0f + __expf(-z));
    }
  }
  __syncthreads();                                      // every wave is done with w1t and phiT

  float* w2t = lds;
  float* act = lds + H * SC;
#pragma unroll
  for (int r = 0; r < NW2; ++r) {
    const int i = tid + T * r;
    w2t[(i / CB) * SC + i % CB] = w2r[r];
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) act[(32 * pb + 8 * (v >> 2) + 4 * hk + (v & 3)) * SH + 32 * jb + l32] = hv[v];
  __syncthreads();

  // read-out: wave owns positions 32 pb .. + 31 x channels 64 cq .. + 63 (two 32-column blocks)
  const int cq = wave >> 1;
  flt_f32x16 acc2[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc2[u][v] = 0.0f;
#pragma unroll 8
  for (int s = 0; s < H / 2; ++s) {
    const int k = 2 * s + hk;
    const float av = act[(32 * pb + l32) * SH + k];
#pragma unroll
    for (int u = 0; u < 2; ++u)
      acc2[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, w2t[k * SC + 64 * cq + 32 * u + l32], acc2[u], 0, 0, 0);
  }
  __syncthreads();                                      // every wave is done with w2t and act

  // bias and window, staged as [channel][position]
  float* st = lds;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int cl = 64 * cq + 32 * u + l32, d = c0 + cl;
    const float b2 = d < a.D ? a.b2[d] : 0.0f, al = d < a.D ? a.alpha[d] : 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int pl = 32 * pb + 8 * (v >> 2) + 4 * hk + (v & 3);
      st[cl * SP + pl] = (acc2[u][v] + b2) * __expf(-al * rarg[pl]);
    }
  }
  __syncthreads();
  for (int i = tid; i < CB * TP; i += T) {
    const int cl = i / TP, pl = i % TP;
    const int d = c0 + cl, pos = p0 + pl;
    if (d < a.D && pos < npos) h[(size_t)d * npos + pos] = st[cl * SP + pl];
  }
}

// ------------------------------------------------------------------ input-dependent (per-sample) filters
// HyenaND summary, method: R register tokens summarised per sample by a softmax-weighted mean z(x); z
// modulates (FiLM) a coordinate SIREN f(c; z); the kernel is K = w(c) f(c; z) with a Gaussian window w.
//   a[r] = softmax_r(q . reg[b, r]),  z = sum_r a[r] reg[b, r]
//   gamma_l = G_l z + g_l,  beta_l = P_l z + p_l                         (l = 1, 2; H values each)
//   h1 = sin(gamma_1 * omega0 * (A1 c + a1) + beta_1),  h2 = sin(gamma_2 * (A2 h1 + a2) + beta_2)
//   K[b, d, c] = (A3 h2 + a3)_d * exp(-|c|^2 / (2 sigma_d^2))
// Coordinates as for the exponential filter: c = t/L (1-D), c = r/n per axis (3-D offsets).

namespace {
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
}  // namespace

// One workgroup per sample: scores, softmax weights, z, then the four FiLM vectors
// mod[b] = {gamma_1, beta_1, gamma_2, beta_2} (H floats each).  Workgroup B writes the transposed
// weights A2t [H][H] and A3t [H][D] that the tile kernel stages row by row.
__global__ void __launch_bounds__(256)
k_film_prep(FilmArgs a, const float* __restrict__ reg, int B, int R, float* __restrict__ mod,
            float* __restrict__ a2t, float* __restrict__ a3t) {
  __shared__ float z[kFilmMaxE];
  __shared__ float wr[kFilmMaxR];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int E = a.E, H = a.H;
  if (b == B) {
    for (int i = tid; i < H * H; i += 256) a2t[i] = a.A2[(i % H) * H + i / H];
    for (int i = tid; i < H * a.D; i += 256) a3t[i] = a.A3[(size_t)(i % a.D) * H + i / a.D];
    return;
  }
  const float* rb = reg + (size_t)b * R * E;
  for (int r = wv; r < R; r += 4) {
    float acc = 0.0f;
    for (int e = lane; e < E; e += 64) acc = fmaf(a.q[e], rb[(size_t)r * E + e], acc);
    acc = wave_sum(acc);
    if (lane == 0) wr[r] = acc;
  }
  __syncthreads();
  float m = -INFINITY;
  for (int r = 0; r < R; ++r) m = fmaxf(m, wr[r]);
  float sum = 0.0f;
  for (int r = 0; r < R; ++r) sum += expf(wr[r] - m);
  __syncthreads();
  for (int r = tid; r < R; r += 256) wr[r] = expf(wr[r] - m) / sum;
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    float acc = 0.0f;
    for (int r = 0; r < R; ++r) acc = fmaf(wr[r], rb[(size_t)r * E + e], acc);
    z[e] = acc;
  }
  __syncthreads();
  // one output per thread (4 H = 256): independent row reads, so the loads of a thread overlap
  const float* Ms[4] = {a.G1, a.P1, a.G2, a.P2};
  const float* vs[4] = {a.g1, a.p1, a.g2, a.p2};
  for (int o = tid; o < 4 * H; o += 256) {
    const float* row = Ms[o / H] + (size_t)(o % H) * E;
    float acc0 = 0.0f, acc1 = 0.0f, acc2 = 0.0f, acc3 = 0.0f;
    int e = 0;
    for (; e + 4 <= E; e += 4) {
      acc0 = fmaf(row[e], z[e], acc0);
      acc1 = fmaf(row[e + 1], z[e + 1], acc1);
      acc2 = fmaf(row[e + 2], z[e + 2], acc2);
      acc3 = fmaf(row[e + 3], z[e + 3], acc3);
    }
    for (; e < E; ++e) acc0 = fmaf(row[e], z[e], acc0);
    mod[(size_t)b * 4 * H + o] = (acc0 + acc1) + (acc2 + acc3) + vs[o / H][o % H];
  }
}

namespace film {
constexpr int H = 64, TP = 64, CB = 128, T = 256;
constexpr int SK = TP + 4;        // row stride of the [k][position] layer-1 output
constexpr int SH = H + 1;         // row stride of the [position][unit] layer-2 output
constexpr int SP = TP + 1;        // row stride of the [channel][position] output staging
// one LDS region, reused: layer-1 output, then layer-2 output, then the output staging
constexpr int RS = (CB * SP > H * SK ? (CB * SP > TP * SH ? CB * SP : TP * SH) : (H * SK > TP * SH ? H * SK : TP * SH));
}  // namespace film

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float film_f32x16;

// sin x for the SIREN layers (|x| up to a few hundred): x is reduced by the nearest multiple of 2 pi,
// with 2 pi split into its fp32 value and the remainder (so the reduced argument keeps fp32 accuracy),
// then the hardware sine takes the reduced angle in revolutions (|r / 2 pi| <= 1/2).
__device__ __forceinline__ float siren_sin(float x) {
  constexpr float kInv2Pi = 0.15915493667125702f;          // fp32(1 / 2 pi)
  constexpr float k2PiHi = 6.2831854820251465f;            // fp32(2 pi)
  constexpr float k2PiLo = -1.7484555314695172e-07f;       // 2 pi - fp32(2 pi)
  const float k = rintf(x * kInv2Pi);
  float r = fmaf(-k, k2PiHi, x);
  r = fmaf(-k, k2PiLo, r);
  return __builtin_amdgcn_sinf(r * kInv2Pi);
}

// Taps of sample blockIdx.z: 64 positions x 128 channels per workgroup, four waves.  Layer 1 (n inputs)
// is evaluated directly into LDS; layer 2 (64 x 64 x 64) and the read-out (64 x 128 x 64) run on the
// matrix cores in fp32 (v_mfma_f32_32x32x2f32): layer 2 one 32 x 32 block per wave (two accumulators
// over alternate k), the read-out two.  The weight operands of both products (the same for every
// workgroup of a sample) are read straight from global memory, where they stay in L2; LDS holds only
// the activations, one 33 KB region that is reused by each phase, so four workgroups share a CU.  The
// output tile leaves through LDS as [channel][position] rows, so the stores run along positions.
template <class G>
__global__ void __launch_bounds__(film::T)
k_film_tiles(FilmArgs a, const float* __restrict__ mod, const float* __restrict__ a2t_g,
             const float* __restrict__ a3t_g, G geo, float* __restrict__ h) {
  using namespace film;
  constexpr int NC = G::NC;
  __shared__ __align__(16) float lds[RS];              // h1T [k][p], then h2 [p][j], then the staging [c][p]
  __shared__ float gm[4 * H];                           // gamma_1, beta_1, gamma_2, beta_2
  __shared__ float w1[H][NC + 2];                       // A1 row, a1, omega0 of each first-layer unit
  __shared__ float crd[NC][TP];
  __shared__ float rsq[TP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hk = lane >> 5;
  const int b = blockIdx.z;
  const int npos = geo.count();
  const int p0 = blockIdx.x * TP, c0 = blockIdx.y * CB;

  float* h1T = lds;
  gm[tid] = mod[(size_t)b * 4 * H + tid];
  if (tid < H) {
#pragma unroll
    for (int ax = 0; ax < NC; ++ax) w1[tid][ax] = a.A1[tid * NC + ax];
    w1[tid][NC] = a.a1[tid];
    w1[tid][NC + 1] = a.omega0[tid];
  } else if (tid < H + TP) {
    const int p = tid - H;
    float c[NC];
    geo.coords(min(p0 + p, npos - 1), c);
    float r2 = 0.0f;
#pragma unroll
    for (int ax = 0; ax < NC; ++ax) {
      crd[ax][p] = c[ax];
      r2 = fmaf(c[ax], c[ax], r2);
    }
    rsq[p] = r2;
  }
  __syncthreads();
  // layer 1: unit k of position p, positions fastest
  for (int i = tid; i < TP * H; i += T) {
    const int k = i / TP, p = i % TP;
    float s = w1[k][NC];
#pragma unroll
    for (int ax = 0; ax < NC; ++ax) s = fmaf(w1[k][ax], crd[ax][p], s);
    h1T[k * SK + p] = siren_sin(fmaf(gm[k], w1[k][NC + 1] * s, gm[H + k]));
  }
  __syncthreads();

  // layer 2: wave owns positions 32 pb .. + 31 x units 32 jb .. + 31 (A: h1[p][k], B: A2^T[k][j])
  const int pb = wave & 1, jb = wave >> 1;
  film_f32x16 acc2[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc2[u][v] = 0.0f;
#pragma unroll 8
  for (int s = 0; s < H / 2; ++s) {
    const int k = 2 * s + hk;
    acc2[s & 1] = __builtin_amdgcn_mfma_f32_32x32x2f32(h1T[k * SK + 32 * pb + l32], a2t_g[k * H + 32 * jb + l32],
                                                       acc2[s & 1], 0, 0, 0);
  }
  // register v holds position 32 pb + 8 (v / 4) + 4 hk + (v mod 4) of unit j = 32 jb + l32
  float h2v[16];
  {
    const int j = 32 * jb + l32;
    const float bj = a.a2[j], g2 = gm[2 * H + j], be2 = gm[3 * H + j];
#pragma unroll
    for (int v = 0; v < 16; ++v) h2v[v] = siren_sin(fmaf(g2, acc2[0][v] + acc2[1][v] + bj, be2));
  }
  __syncthreads();                                      // every wave is done with h1T

  float* h2 = lds;
  {
    const int j = 32 * jb + l32;
#pragma unroll
    for (int v = 0; v < 16; ++v) h2[(32 * pb + 8 * (v >> 2) + 4 * hk + (v & 3)) * SH + j] = h2v[v];
  }
  __syncthreads();

  // read-out: wave owns positions 32 pb .. + 31 x channels 64 cq .. + 63 (two 32-column blocks)
  const int cq = wave >> 1;
  // this lane's read-out weight columns (channels past D read as zero)
  const int ca = c0 + 64 * cq + l32, cb = ca + 32;
  const float* w3a = a3t_g + (ca < a.D ? ca : 0);
  const float* w3b = a3t_g + (cb < a.D ? cb : 0);
  const float ma = ca < a.D ? 1.0f : 0.0f, mb = cb < a.D ? 1.0f : 0.0f;
  film_f32x16 acc3[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc3[u][v] = 0.0f;
#pragma unroll 8
  for (int s = 0; s < H / 2; ++s) {
    const int k = 2 * s + hk;
    const float av = h2[(32 * pb + l32) * SH + k];
    acc3[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, ma * w3a[(size_t)k * a.D], acc3[0], 0, 0, 0);
    acc3[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, mb * w3b[(size_t)k * a.D], acc3[1], 0, 0, 0);
  }

  // bias and window; register v holds position 32 pb + 8 (v / 4) + 4 hk + (v mod 4) of channel d
  __syncthreads();                                      // every wave is done with h2
  float* st = lds;                                      // [CB][SP]
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int cl = 64 * cq + 32 * u + l32, d = c0 + cl;
    const float a3 = d < a.D ? a.a3[d] : 0.0f, sg = d < a.D ? a.sigma[d] : 1.0f;
    const float k2 = -0.5f / (sg * sg);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int pl = 32 * pb + 8 * (v >> 2) + 4 * hk + (v & 3);
      st[cl * SP + pl] = (acc3[u][v] + a3) * expf(k2 * rsq[pl]);
    }
  }
  __syncthreads();
  float* hb = h + (size_t)b * a.D * npos;
  for (int i = tid; i < CB * TP; i += T) {
    const int cl = i / TP, pl = i % TP;
    const int d = c0 + cl, pos = p0 + pl;
    if (d < a.D && pos < npos) hb[(size_t)d * npos + pos] = st[cl * SP + pl];
  }
}

size_t film_scratch_floats(int B, int D) { return (size_t)B * 4 * kFilmHidden + (size_t)kFilmHidden * (kFilmHidden + D); }

hipError_t launch_film_prep(const FilmArgs& a, const float* reg, int B, int R, float* scratch, hipStream_t s) {
  if (a.H != 64 || a.E < 1 || a.E > kFilmMaxE || R < 1 || R > kFilmMaxR || B < 1) return hipErrorInvalidValue;
  float* mod = scratch;
  float* a2t = scratch + (size_t)B * 4 * kFilmHidden;
  float* a3t = a2t + kFilmHidden * kFilmHidden;
  hipLaunchKernelGGL(k_film_prep, dim3(B + 1), dim3(256), 0, s, a, reg, B, R, mod, a2t, a3t);
  return hipGetLastError();
}

namespace {
template <class G>
hipError_t film_tiles_launch(const FilmArgs& a, const float* scratch, int B, const G& geo, float* h, hipStream_t s) {
  const float* a2t = scratch + (size_t)B * 4 * kFilmHidden;
  const float* a3t = a2t + kFilmHidden * kFilmHidden;
  const int np = geo.count_host();
  const dim3 grid((np + film::TP - 1) / film::TP, (a.D + film::CB - 1) / film::CB, B);
  hipLaunchKernelGGL((k_film_tiles<G>), grid, dim3(film::T), 0, s, a, scratch, a2t, a3t, geo, h);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_film_filter1d(const FilmArgs& a, const float* scratch, int B, int L, float* h, hipStream_t s) {
  if (a.H != 64 || a.NC != 1 || L <= 0 || B < 1) return hipErrorInvalidValue;
  return film_tiles_launch(a, scratch, B, FilterGrid1D{L}, h, s);
}

hipError_t launch_film_filter3d(const FilmArgs& a, const float* scratch, int B, float* h, hipStream_t s, int circ) {
  if (a.H != 64 || a.NC != 3 || B < 1) return hipErrorInvalidValue;
  constexpr int n = 64;
  const FilterGrid3D geo = circ ? FilterGrid3D{n, n / 2, n} : FilterGrid3D{2 * n - 1, n - 1, n};
  return film_tiles_launch(a, scratch, B, geo, h, s);
}

hipError_t launch_filter1d(const FilterArgs& a, int L, float* h, hipStream_t s) {
  if (a.F != 64 || a.H != 64 || L <= 0) return hipErrorInvalidValue;
  const dim3 grid((L + flt::TP - 1) / flt::TP, (a.D + flt::CB - 1) / flt::CB);
  hipLaunchKernelGGL((k_filter_tiles<64, FilterGrid1D>), grid, dim3(flt::T), 0, s, a, FilterGrid1D{L}, h);
  return hipGetLastError();
}

// 3-D taps on the 64^3 grid: zero-padded offsets [-63, 63]^3 (W = 127) or the periodic centred period
// [-32, 31]^3 (W = 64); h[d, W, W, W] with tap index = offset + R0.
hipError_t launch_filter3d(const FilterArgs& a, float* h, hipStream_t s, int circ) {
  if (a.F != 96 || a.H != 64) return hipErrorInvalidValue;
  constexpr int n = 64;
  const FilterGrid3D geo = circ ? FilterGrid3D{n, n / 2, n} : FilterGrid3D{2 * n - 1, n - 1, n};
  const int np = geo.W * geo.W * geo.W;
  const dim3 grid((np + flt::TP - 1) / flt::TP, (a.D + flt::CB - 1) / flt::CB);
  hipLaunchKernelGGL((k_filter_tiles<96, FilterGrid3D>), grid, dim3(flt::T), 0, s, a, geo, h);
  return hipGetLastError();
}

}  // namespace hyena
