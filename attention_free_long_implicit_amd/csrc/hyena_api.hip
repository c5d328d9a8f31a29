// C ABI of libhyena.so: argument validation, pass planning and launches on the caller's stream.
// Declarations and the contract of every entry point are in include/hyena.h.
#include <math.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/hyena.h"
#include "launch.h"

using namespace hyena;

// Constant tables: file-scope device arrays, so every device the library runs on holds its own copy from the
// moment the code object is loaded (nothing is allocated).  Host code never passes these names to a kernel:
// it takes each array's address on the device once (hipGetSymbolAddress, with that device current) and
// uses that address.
static __device__ __align__(256) float2 g_twiddle_table[kTwPow2Entries + kTwFine];
static __device__ __align__(256) uint16_t g_matrix_table[kMfmaMatrixCount];
// Workspace of hyena_operator_noalloc (the multi-pass intermediates), shared by every such call on a device.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
// Multi-pass plans: chunks of about kChunkMB of intermediate cycle over kChunkWays streams (the caller's and
// kChunkWays - 1 side streams); see pair_chunk_rows.
constexpr int kChunkWays = 2;      // streams the chunks cycle over (the caller's and kChunkWays - 1 side streams)
constexpr int kChunkMB = 64;
constexpr int kChunk3dMB = 96;    // the zero-padded 3-D plan (see pair_chunk_rows)
static_assert(kChunkWays >= 2 && kChunkWays <= kSideStreams + 1, "side streams");
std::mutex g_mu;
struct DeviceTables {
  Twiddles tw;
  const void* mats;       // DFT matrices of the matrix-core path (bf16, per lane)
  void* scratch;          // this device's copy of `scratch`
  SideStream side;        // the long-row plans' side streams (default priority) and their fork / join events
  bool ready;
};
// Held while a long-row plan forks onto a device's side streams, so that concurrent calls do not interleave
// their fork and join events.
std::mutex g_side_mu;
DeviceTables g_dev[kMaxDevices];

// W_N^j = exp(-2 pi i j / N) in double, rounded once to fp32.
float2 host_twiddle(long j, long n) {
  const double a = -2.0 * M_PI * (double)j / (double)n;
  return make_float2((float)cos(a), (float)sin(a));
}

// Fill the tables of the current device once (a blocking upload) and record the arrays' device addresses.
int init_current_device(DeviceTables** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HYENA_EHIP;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceTables& t = g_dev[dev];
  if (!t.ready) {
    void* tw = nullptr;
    void* mats = nullptr;
    void* scr = nullptr;
    if (hipGetSymbolAddress(&tw, HIP_SYMBOL(g_twiddle_table)) != hipSuccess || !tw) return HYENA_EHIP;
    if (hipGetSymbolAddress(&mats, HIP_SYMBOL(g_matrix_table)) != hipSuccess || !mats) return HYENA_EHIP;
    if (hipGetSymbolAddress(&scr, HIP_SYMBOL(scratch)) != hipSuccess || !scr) return HYENA_EHIP;
    std::vector<float2> host(kTwPow2Entries + kTwFine);
    host[0] = make_float2(1.f, 0.f);
    for (int sz = 1; sz <= (1 << kTwPow2Log2); sz <<= 1)
      for (int j = 0; j < sz; ++j) host[sz + j] = host_twiddle(j, sz);
    for (int b = 0; b < kTwFine; ++b) host[kTwPow2Entries + b] = host_twiddle(b, 1L << kTwMaxLog2);
    std::vector<uint16_t> m(kMfmaMatrixCount);
    mfma_matrices_host(m.data());
    if (hipMemcpy(tw, host.data(), host.size() * sizeof(float2), hipMemcpyHostToDevice) != hipSuccess)
      return HYENA_EHIP;
    if (hipMemcpy(mats, m.data(), m.size() * sizeof(uint16_t), hipMemcpyHostToDevice) != hipSuccess)
      return HYENA_EHIP;
    t.tw.pow2 = (const float2*)tw;
    t.tw.fine = (const float2*)tw + kTwPow2Entries;
    for (int j = 0; j < kSideStreams; ++j)
      if (hipStreamCreateWithFlags(&t.side.s[j], hipStreamNonBlocking) != hipSuccess ||
          hipEventCreateWithFlags(&t.side.join[j], hipEventDisableTiming) != hipSuccess)
        return HYENA_EHIP;
    if (hipEventCreateWithFlags(&t.side.fork, hipEventDisableTiming) != hipSuccess) return HYENA_EHIP;
    t.side.ways = kChunkWays;
    t.mats = mats;
    t.scratch = scr;
    t.ready = true;
  }
  *out = &t;
  return HYENA_OK;
}

int get_twiddles(Twiddles* out) {
  DeviceTables* t = nullptr;
  const int st = init_current_device(&t);
  if (st) return st;
  *out = t->tw;
  return HYENA_OK;
}

const void* device_mats() {
  DeviceTables* t = nullptr;
  return init_current_device(&t) ? nullptr : t->mats;
}

bool is_pow2(int64_t n) { return n > 0 && (n & (n - 1)) == 0; }
int log2i(int64_t n) { int k = 0; while ((int64_t(1) << k) < n) ++k; return k; }

size_t elem_bytes(int dtype) { return dtype == HYENA_BF16 ? 2 : 4; }

// Shape checks shared by every entry point.  On success *points = elements per (b, d) row.
int check_dims(hyena_dims dims, int mode, int64_t* points) {
  if (mode == HYENA_CIRCULAR) {
    // periodic boundary: 1-D rows of L = 2^11 .. 2^21 samples (a packed L/2-point transform: in LDS up to
    // 2^15, multi-pass above), or the 64^3 grid
    if (dims.ndim != 1 && dims.ndim != 3) return HYENA_EINVAL;
    for (int a = 0; a < dims.ndim; ++a)
      if (dims.n[a] <= 0) return HYENA_EINVAL;
    if (dims.ndim == 3) {
      if (!grid3d_supported(dims.n[0], dims.n[1], dims.n[2])) return HYENA_EUNSUPPORTED;
      *points = dims.n[0] * dims.n[1] * dims.n[2];
      return HYENA_OK;
    }
    const int64_t L = dims.n[0];
    if (!is_pow2(L) || L < (1 << 11) ||
        (!single_pass_supported(log2i(L) - 1) && !fourstep_supported(log2i(L) - 1)))
      return HYENA_EUNSUPPORTED;
    *points = L;
    return HYENA_OK;
  }
  if (mode == HYENA_CAUSAL) {
    if (dims.ndim != 1) return HYENA_EINVAL;
    const int64_t L = dims.n[0];
    if (L <= 0) return HYENA_EINVAL;
    if (!is_pow2(L) || L < (1 << 10) || L > (1 << 20)) return HYENA_EUNSUPPORTED;
    if (!single_pass_supported(log2i(L)) && !fourstep_supported(log2i(L))) return HYENA_EUNSUPPORTED;
    *points = L;
    return HYENA_OK;
  }
  if (mode == HYENA_LINEAR) {
    if (dims.ndim != 3) return HYENA_EINVAL;
    if (dims.n[0] <= 0 || dims.n[1] <= 0 || dims.n[2] <= 0) return HYENA_EINVAL;
    if (!grid3d_supported(dims.n[0], dims.n[1], dims.n[2])) return HYENA_EUNSUPPORTED;
    *points = dims.n[0] * dims.n[1] * dims.n[2];
    return HYENA_OK;
  }
  return HYENA_EINVAL;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* pa = (const char*)a;
  const char* pb = (const char*)b;
  return pa < pb + nb && pb < pa + na;
}

int hip_status(hipError_t e) { return e == hipSuccess ? HYENA_OK : HYENA_EHIP; }

bool is_multipass(int64_t L) { return !single_pass_supported(log2i(L)); }

// What a (mode, grid) pair runs: 1-D causal, 1-D periodic, 3-D zero-padded or 3-D periodic.
enum Kind { K_CAUSAL, K_CIRC1, K_LIN3, K_CIRC3 };
int kind_of(int mode, hyena_dims dims) {
  if (mode == HYENA_CAUSAL) return K_CAUSAL;
  if (mode == HYENA_LINEAR) return K_LIN3;
  return dims.ndim == 1 ? K_CIRC1 : K_CIRC3;
}
bool is3d(int kind) { return kind == K_LIN3 || kind == K_CIRC3; }
int circ3(int kind) { return kind == K_CIRC3 ? 1 : 0; }
// 1-D periodic rows of L samples run the 1-D engines on L/2 packed points (all of them filled).
int circular_log2(int64_t L) { return log2i(L) - 1; }
// log2 of the packed transform length of a 1-D plan
int engine_log2(int kind, int64_t L) { return kind == K_CIRC1 ? circular_log2(L) : log2i(L); }
bool multipass1d(int kind, int64_t L) { return !single_pass_supported(engine_log2(kind, L)); }

// Intermediate bytes per (b, d) row / volume for the multi-pass plans (0: single pass); the 1-D rows of bf16
// storage keep their intermediate in block-scaled fp16.
size_t row_intermediate_bytes(int kind, int64_t pts, int dtype) {
  if (is3d(kind)) return conv3d_volume_bytes(circ3(kind));
  return multipass1d(kind, pts) ? fourstep_row_bytes(engine_log2(kind, pts), dtype == HYENA_BF16) : 0;
}
size_t filter_intermediate_bytes(int kind, int64_t pts) {
  if (is3d(kind)) return conv3d_filter_volume_bytes(circ3(kind));
  return multipass1d(kind, pts) ? fourstep_row_bytes(engine_log2(kind, pts), 0) : 0;
}
size_t taps_per_channel(int kind, int64_t pts) { return is3d(kind) ? conv3d_taps_per_channel(circ3(kind)) : (size_t)pts; }

// Lengths whose spectrum also carries a matrix-core (bf16 storage) copy after the fp32 one: the row-pair
// copy of the single-workgroup kernel (L = 8192) and the split coefficients of the long-row kernels
// (L = 2^15 .. 2^17).
bool has_pair_copy(int64_t L) { return mfma_pair_supported(log2i(L), 2); }
bool has_long_row_copy(int64_t L) { return is_pow2(L) && mfl_supported(log2i(L)); }
size_t natural_bins_bytes(int64_t L, int64_t D) { return (size_t)D * (size_t)(L + 1) * sizeof(float2); }
size_t mfma_copy_bytes_per_channel(int64_t L) {
  if (has_pair_copy(L)) return mfma_pair_spectrum_bytes_per_channel();
  if (has_long_row_copy(L)) return mfl_spectrum_bytes_per_channel(log2i(L));
  return 0;
}

// Rows per multi-pass chunk by default on one stream: about 160 MB of intermediate (the decode state's
// prefix convolutions and the 3-D plans).  Smaller chunks on one stream (24-96 MB, sized for the 256 MB
// memory-side cache) measured slower, from fewer workgroups per launch; larger ones measured the same.
int64_t default_chunk_rows(int64_t per, int64_t rows) {
  int64_t c = ((int64_t)160 << 20) / per;
  if (c < 1) c = 1;
  return c < rows ? c : rows;
}

// The multi-pass plans (1-D long rows, 3-D volumes) run chunks of about 64 MB of intermediate two at a time,
// on the caller's stream and the library's side stream (32, 48, 64, 72 and 80 MB measured 5.12, 4.86, 4.77-4.84,
// 4.93 and 4.91 ms per step at L = 2^20, fp32, 256 rows, against 5.37 ms for one stream of 160 MB chunks).
// The zero-padded 3-D plan takes chunks of about 96 MB (128 volumes of 2.13 MB: ten, six and four equal
// chunks measured 1.437, 1.405 and 1.384 ms per step).  A whole batch of at most 192 MB of intermediate runs
// as one chunk on one stream (periodic 64^3, 138 MB: 0.41 ms, against 0.43 ms in 64 MB pairs).  Three streams
// measured slower (64 / 44 MB chunks: 5.28 / 4.96 ms at L = 2^20 against 4.83, 2.95 / 2.90 ms against 2.85
// for the order-3 L = 65536 bf16 workload).  The workspace holds kChunkWays chunks.
int chunk_mb(int kind) { return is3d(kind) && !circ3(kind) ? kChunk3dMB : kChunkMB; }
int64_t pair_chunk_rows(int64_t per, int64_t rows, int mb) {
  if ((size_t)rows * (size_t)per <= ((size_t)192 << 20)) return rows;
  int64_t c = ((int64_t)mb << 20) / per;
  if (c < 1) c = 1;
  return c < rows ? c : rows;
}
size_t pair_ws_bytes(size_t per, int64_t rows, int mb) {
  const int64_t c = pair_chunk_rows((int64_t)per, rows, mb);
  return (size_t)(rows > c ? kChunkWays : 1) * (size_t)c * per;
}
// Chunk rows of a multi-pass plan within a workspace of ws_bytes, and how many streams its chunks cycle over
// (0: the workspace does not hold one row).
int pair_chunk(size_t per, int64_t rows, size_t ws_bytes, int* ways, int mb) {
  const int64_t cap = (int64_t)(ws_bytes / per);
  *ways = 1;
  if (cap < 1) return 0;
  if (cap >= rows && pair_chunk_rows((int64_t)per, rows, mb) >= rows) return (int)rows;   // one chunk
  int64_t c = cap;
  if (cap >= 2 && rows > 1) {
    const int w = cap >= kChunkWays ? kChunkWays : (int)cap;
    c = cap / w;
    const int64_t want = pair_chunk_rows((int64_t)per, rows, mb);
    if (c > want) c = want;
    if (rows > c) *ways = w;
  }
  if (c >= rows) return (int)rows;
  // equal chunks, their number a multiple of the streams (never larger than c): no nearly empty last
  // chunk running alone at the end
  int64_t n = (rows + c - 1) / c;
  n = (n + *ways - 1) / *ways * *ways;
  return (int)((rows + n - 1) / n);
}

// Channels per chunk while building spectra from taps: about 1 GB of intermediate.  Nothing is reused
// across channels there, and fewer, larger launches lose less to the partly filled last round of
// workgroups than the 160 MB chunks of the convolution.
int64_t filter_chunk_rows(int64_t per, int64_t rows) {
  int64_t c = ((int64_t)1 << 30) / per;
  if (c < 1) c = 1;
  return c < rows ? c : rows;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The matrix-core kernel: bf16, L = 8192, rows in pairs, and (16-byte vector accesses) every activation
// pointer 16-byte aligned.
bool use_mfma(int dtype, int64_t B, int64_t L) { return dtype == HYENA_BF16 && mfma_pair_supported(log2i(L), (int)B); }

// Highest operator order sent to the long-row matrix-core kernels (same budget as kMfmaMaxOrder: fp16
// transform operands, plus the fp16 planes between passes).
constexpr int kMflMaxOrder = 3;

// Whether a causal bf16 call at length L, with these activation pointers, takes the long-row matrix-core
// kernels (16-byte vector accesses to every activation).
bool use_mfl(int kind, int dtype, int64_t L, int hsb, int order, const void* v, const void* const* x, const void* y) {
  if (kind != K_CAUSAL || hsb || dtype != HYENA_BF16 || order > kMflMaxOrder || !is_pow2(L) ||
      !mfl_supported(log2i(L)))
    return false;
  bool ok = aligned16(v) && aligned16(y);
  for (int i = 0; i < order; ++i) ok = ok && (!x[i] || aligned16(x[i]));
  return ok;
}

// Highest operator order sent to the matrix-core kernel.  Its fp16 transform operands and products cost a
// few 1e-4 of relative error per order, and later orders amplify what earlier ones leave: measured against
// the oracle (max over rows, with no decay window, the worst filter family) 3.4e-3 at order 2, 6.8e-3 at
// order 3 and 8.8e-3 at order 4, but 5.4e-2 at order 6 against the 2e-2 that bf16 storage allows.  Orders
// above 3 take the fp32 engine, whose only roundings are the bf16 stores, keeping a margin of about 3x.
constexpr int kMfmaMaxOrder = 3;

// Orders [0, order) through the matrix-core kernel, up to kMfmaMaxChain orders per launch with u_i on chip.
int conv_mfma_chain(int64_t B, int64_t D, int64_t L, const void* u, const void* const* gates,
                    const void* const* spectra, int order, void* y, hipStream_t s) {
  const void* mats = device_mats();
  if (!mats) return HYENA_EHIP;
  const void* cur = u;
  for (int i0 = 0; i0 < order; i0 += kMfmaMaxChain) {
    const int n = order - i0 < kMfmaMaxChain ? order - i0 : kMfmaMaxChain;
    const void* g[kMfmaMaxChain];
    const void* sp[kMfmaMaxChain];
    for (int k = 0; k < n; ++k) {
      g[k] = gates[i0 + k];
      sp[k] = (const char*)spectra[i0 + k] + (size_t)D * (size_t)L * sizeof(float2);
    }
    const int st = hip_status(launch_conv_mfma(cur, g, sp, n, y, mats, (int)B, (int)D, s));
    if (st) return st;
    cur = y;
  }
  return HYENA_OK;
}

int conv_once(int64_t B, int64_t D, int64_t L, int dtype, const void* u, const void* spectrum, const void* gate,
              void* y, const Twiddles& tw, hipStream_t s, int hsb) {
  if (!hsb && use_mfma(dtype, B, L) && aligned16(u) && aligned16(gate) && aligned16(y)) {
    const void* g[1] = {gate};
    const void* sp[1] = {spectrum};
    return conv_mfma_chain(B, D, L, u, g, sp, 1, y, s);
  }
  return hip_status(launch_conv1d_single(log2i(L), dtype == HYENA_BF16, u, gate, y, (const float2*)spectrum,
                                         (int)B, (int)D, tw, s, 0, hsb));
}

// Align a workspace cursor to 256 bytes; false when the remaining room is too small.
bool ws_align256(char*& p, size_t& n) {
  const size_t mis = (size_t)p & 255u;
  if (!mis) return true;
  const size_t adv = 256 - mis;
  if (n < adv) return false;
  p += adv;
  n -= adv;
  return true;
}

// Filter spectra of `nch` channels from their taps h [nch, taps] (the workspace [wsp, wsp + wsn) holds the
// multi-pass intermediate or the matrix-core copy's staging).  mfma_copy: also write the matrix-core copy of
// bf16 storage after the fp32 spectra (causal L = 8192: the row-pair copy; causal L = 2^15 .. 2^17: the
// long-row split coefficients; one filter per channel).
int spectra_from_taps(int kind, int64_t L, const float* h, int64_t nch, void* spectrum, char* wsp, size_t wsn,
                      bool mfma_copy, const Twiddles& tw, hipStream_t stream) {
  int st;
  const size_t row_b = filter_intermediate_bytes(kind, L);
  int chunk = 0;
  if (row_b) {
    if (!ws_align256(wsp, wsn)) return HYENA_EWORKSPACE;
    const int64_t c = (int64_t)(wsn / row_b);
    if (c < 1) return HYENA_EWORKSPACE;
    chunk = (int)(c < nch ? c : nch);
  }
  if (is3d(kind))
    return hip_status(launch_spectrum3d(h, (float2*)spectrum, (int)nch, (float2*)wsp, chunk, tw, stream, circ3(kind)));
  if (row_b) {
    if ((st = hip_status(launch_spectrum1d_fourstep(engine_log2(kind, L), h, (float2*)spectrum, (int)nch,
                                                    (float2*)wsp, chunk, tw, stream, kind == K_CIRC1 ? 1 : 0))))
      return st;
    if (!mfma_copy || kind != K_CAUSAL || !has_long_row_copy(L)) return HYENA_OK;
    // the long-row matrix-core copy after the fp32 spectra: natural-order bins of as many channels as the
    // workspace holds (free again: the same stream has finished with the intermediate), then their copy
    const size_t nat = natural_bins_bytes(L, 1);
    const int64_t c = (int64_t)(wsn / nat);
    if (c < 1) return HYENA_EWORKSPACE;
    const size_t pb = mfl_spectrum_bytes_per_channel(log2i(L));
    char* copy = (char*)spectrum + (size_t)nch * (size_t)L * sizeof(float2);
    for (int64_t d0 = 0; d0 < nch; d0 += c) {
      const int n = (int)(nch - d0 < c ? nch - d0 : c);
      if ((st = hip_status(launch_export1d_fourstep(log2i(L), (const float2*)spectrum + (size_t)d0 * (size_t)L,
                                                    (float2*)wsp, n, stream))))
        return st;
      if ((st = hip_status(launch_mfl_spectrum(log2i(L), (const float2*)wsp, copy + (size_t)d0 * pb, n, tw, stream))))
        return st;
    }
    return HYENA_OK;
  }
  if (kind == K_CIRC1)
    return hip_status(launch_spectrum1d_single(circular_log2(L), h, (float2*)spectrum, (int)nch, tw, stream, 1));
  if ((st = hip_status(launch_spectrum1d_single(log2i(L), h, (float2*)spectrum, (int)nch, tw, stream)))) return st;
  if (mfma_copy && has_pair_copy(L)) {
    // natural-order bins into the workspace, then the pair-order bf16 copy after the fp32 spectrum
    if (!ws_align256(wsp, wsn) || wsn < natural_bins_bytes(L, nch)) return HYENA_EWORKSPACE;
    float2* nat = (float2*)wsp;
    if ((st = hip_status(launch_export1d_single(log2i(L), (const float2*)spectrum, nat, (int)nch, stream)))) return st;
    void* pair = (char*)spectrum + (size_t)nch * (size_t)L * sizeof(float2);
    return hip_status(launch_pair_spectrum(nat, pair, (int)nch, stream));
  }
  return HYENA_OK;
}

// Whether spectra_from_taps finds the room it needs in [wsp, wsp + wsn) (checked before any launch).
bool spectra_ws_ok(int kind, int64_t L, int64_t nch, char* wsp, size_t wsn, bool mfma_copy) {
  const size_t row_b = filter_intermediate_bytes(kind, L);
  if (row_b)
    return ws_align256(wsp, wsn) && wsn >= row_b &&
           (!mfma_copy || kind != K_CAUSAL || !has_long_row_copy(L) || wsn >= natural_bins_bytes(L, 1));
  if (mfma_copy && kind == K_CAUSAL && has_pair_copy(L))
    return ws_align256(wsp, wsn) && wsn >= natural_bins_bytes(L, nch);
  return true;
}

// Split the per-sample flag off a mode argument.
int split_mode(int mode, bool* per_sample) {
  *per_sample = (mode & HYENA_PER_SAMPLE) != 0;
  return mode & ~HYENA_PER_SAMPLE;
}

// hyena_operator with the workspace [ws, ws + ws_bytes); noalloc: the workspace is this device's `scratch`
// (taken here, after validation), and a row whose intermediate does not fit it is rejected.
int run_operator(int order, int64_t B, int64_t D, hyena_dims dims, int dtype, int mode, const void* v,
                 const void* const* x, const void* const* spectra, void* y, void* ws, size_t ws_bytes,
                 hipStream_t stream, bool noalloc) {
  if (order < 1 || B <= 0 || D <= 0 || !v || !x || !spectra || !y || (dtype != HYENA_F32 && dtype != HYENA_BF16))
    return HYENA_EINVAL;
  for (int i = 0; i < order; ++i)
    if (!x[i] || !spectra[i]) return HYENA_EINVAL;
  if (B * D > (int64_t)INT32_MAX) return HYENA_EUNSUPPORTED;
  bool ps = false;
  mode = split_mode(mode, &ps);
  const int hsb = ps ? (int)D : 0;
  int64_t pts = 0;
  int st = check_dims(dims, mode, &pts);
  if (st) return st;
  const int kind = kind_of(mode, dims);
  const size_t tb = (size_t)B * D * pts * elem_bytes(dtype);
  if (y != v && overlaps(y, tb, v, tb)) return HYENA_EALIAS;
  for (int i = 0; i < order; ++i)
    if (overlaps(y, tb, x[i], tb)) return HYENA_EALIAS;
  int chunk = 0;
  const size_t per = row_intermediate_bytes(kind, pts, dtype);
  if (noalloc) {
    if (per > kNoallocScratchBytes) return HYENA_EWORKSPACE;
    DeviceTables* dt = nullptr;
    if ((st = init_current_device(&dt))) return st;
    ws = dt->scratch;
    ws_bytes = kNoallocScratchBytes;
  }
  int ways = 1;
  bool mfl = false;   // the long-row matrix-core kernels
  if (per) {
    const bool ws_ok = ws && !((size_t)ws & 255u);
    if (ws_ok && use_mfl(kind, dtype, pts, hsb, order, v, x, y)) {
      chunk = pair_chunk(mfl_row_bytes(log2i(pts)), B * D, ws_bytes, &ways, kChunkMB);
      mfl = chunk >= 1;
    }
    if (!mfl) chunk = ws_ok ? pair_chunk(per, B * D, ws_bytes, &ways, chunk_mb(kind)) : 0;
    if (chunk < 1) return HYENA_EWORKSPACE;
    if (overlaps(ws, ws_bytes, y, tb) || overlaps(ws, ws_bytes, v, tb)) return HYENA_EALIAS;
    for (int i = 0; i < order; ++i)
      if (overlaps(ws, ws_bytes, x[i], tb)) return HYENA_EALIAS;
  }
  Twiddles tw;
  if ((st = get_twiddles(&tw))) return st;
  if (chunk) {
    DeviceTables* dt = nullptr;
    if (ways > 1 && (st = init_current_device(&dt))) return st;
    std::unique_lock<std::mutex> lk(g_side_mu, std::defer_lock);
    SideStream sd{};
    if (ways > 1) {
      lk.lock();
      sd = dt->side;
      sd.ways = ways;
    }
    if (is3d(kind))
      return hip_status(launch_conv3d(dtype == HYENA_BF16, order, (int)B, (int)D, v, x, spectra, y, (float2*)ws,
                                      chunk, tw, stream, circ3(kind), hsb, ways > 1 ? &sd : nullptr));
    if (mfl) {
      const void* mats = device_mats();
      if (!mats) return HYENA_EHIP;
      std::vector<const void*> sp(order);
      for (int i = 0; i < order; ++i) sp[i] = (const char*)spectra[i] + (size_t)D * (size_t)pts * sizeof(float2);
      return hip_status(launch_conv_mfl(log2i(pts), order, (int)B, (int)D, v, x, sp.data(), y, ws, chunk, mats, tw,
                                        stream, ways > 1 ? &sd : nullptr));
    }
    return hip_status(launch_conv1d_fourstep(engine_log2(kind, pts), dtype == HYENA_BF16, order, (int)B, (int)D, v, x,
                                             spectra, y, (float2*)ws, chunk, tw, stream, kind == K_CIRC1 ? 1 : 0, hsb,
                                             ways > 1 ? &sd : nullptr));
  }
  if (kind == K_CAUSAL && !hsb && order <= kMfmaMaxOrder && use_mfma(dtype, B, pts)) {
    bool aligned = aligned16(v) && aligned16(y);
    for (int i = 0; i < order; ++i) aligned = aligned && aligned16(x[i]);
    if (aligned) return conv_mfma_chain(B, D, pts, v, x, spectra, order, y, stream);
  }
  // the single-pass fp32 engine: up to kConvMaxChain orders per launch with u_i on chip
  const int lg = kind == K_CIRC1 ? circular_log2(pts) : log2i(pts);
  const void* cur = v;
  for (int i0 = 0; i0 < order; i0 += kConvMaxChain) {
    const int n = order - i0 < kConvMaxChain ? order - i0 : kConvMaxChain;
    const float2* sp[kConvMaxChain];
    for (int k = 0; k < n; ++k) sp[k] = (const float2*)spectra[i0 + k];
    if ((st = hip_status(launch_conv1d_chain(lg, dtype == HYENA_BF16, cur, x + i0, sp, n, y, (int)B, (int)D, tw,
                                             stream, kind == K_CIRC1 ? 1 : 0, hsb))))
      return st;
    cur = y;
  }
  return HYENA_OK;
}

}  // namespace

extern "C" {

int hyena_version(void) { return 400; }   // 0.4.0: fp32 intermediates on every bf16 path, hyena_init

int hyena_init(void) {
  DeviceTables* t = nullptr;
  return init_current_device(&t);
}

const char* hyena_status_str(int status) {
  switch (status) {
    case HYENA_OK: return "ok";
    case HYENA_EINVAL: return "invalid argument";
    case HYENA_EUNSUPPORTED: return "unsupported size or mode";
    case HYENA_EWORKSPACE: return "workspace missing or too small";
    case HYENA_EHIP: return "HIP runtime error";
    case HYENA_EALIAS: return "output overlaps an input";
  }
  return "unknown status";
}

int hyena_spectrum_bytes(hyena_dims dims, int mode, int64_t D, size_t* bytes) {
  if (!bytes || D <= 0) return HYENA_EINVAL;
  bool ps = false;
  mode = split_mode(mode, &ps);
  int64_t pts = 0;
  int st = check_dims(dims, mode, &pts);
  if (st) return st;
  const int kind = kind_of(mode, dims);
  if (is3d(kind)) *bytes = (size_t)D * conv3d_spectrum_bytes_per_channel(circ3(kind));
  else if (kind == K_CIRC1) *bytes = (size_t)D * (size_t)(pts / 2) * sizeof(float2);
  else *bytes = (size_t)D * (size_t)pts * sizeof(float2) + (ps ? 0 : (size_t)D * mfma_copy_bytes_per_channel(pts));
  return HYENA_OK;
}

int hyena_filter_workspace_bytes(hyena_dims dims, int mode, int64_t D, size_t* bytes) {
  if (!bytes || D <= 0) return HYENA_EINVAL;
  int64_t pts = 0;
  int st = check_dims(dims, mode, &pts);
  if (st) return st;
  const int kind = kind_of(mode, dims);
  *bytes = (size_t)D * taps_per_channel(kind, pts) * sizeof(float);
  if (kind == K_CAUSAL && has_pair_copy(pts)) *bytes += 256 + natural_bins_bytes(pts, D);
  const size_t per = filter_intermediate_bytes(kind, pts);
  if (per) {
    size_t room = (size_t)filter_chunk_rows((int64_t)per, D) * per;
    if (kind == K_CAUSAL && has_long_row_copy(pts) && room < natural_bins_bytes(pts, 1))
      room = natural_bins_bytes(pts, 1);
    *bytes += 256 + room;
  }
  return HYENA_OK;
}

int hyena_workspace_bytes(int order, int64_t B, int64_t D, hyena_dims dims, int dtype, int mode, size_t* bytes) {
  if (!bytes || order < 1 || B <= 0 || D <= 0 || (dtype != HYENA_F32 && dtype != HYENA_BF16)) return HYENA_EINVAL;
  bool ps = false;
  mode = split_mode(mode, &ps);
  int64_t pts = 0;
  int st = check_dims(dims, mode, &pts);
  if (st) return st;
  const int kind = kind_of(mode, dims);
  *bytes = 0;
  const size_t per = row_intermediate_bytes(kind, pts, dtype);
  if (per) *bytes = pair_ws_bytes(per, B * D, chunk_mb(kind));
  // (the long-row matrix-core kernels need less per row than the per-row plan, which stays possible for
  // misaligned activations)
  return HYENA_OK;
}

int hyena_filter_gen(const hyena_filter_params* p, hyena_dims dims, int mode, float* h_time, void* spectrum,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!p || !spectrum || !p->W1 || !p->b1 || !p->W2 || !p->b2 || !p->alpha || p->D <= 0) return HYENA_EINVAL;
  int64_t pts = 0;
  int st = check_dims(dims, mode, &pts);
  if (st) return st;
  const int kind = kind_of(mode, dims);
  if (p->H != 64 || p->F != (dims.ndim == 1 ? 64 : 96)) return HYENA_EUNSUPPORTED;
  const size_t hbytes = (size_t)p->D * taps_per_channel(kind, pts) * sizeof(float);
  char* wsp = (char*)ws;
  size_t wsn = ws ? ws_bytes : 0;
  float* h = h_time;
  if (!h) {
    if (wsn < hbytes) return HYENA_EWORKSPACE;
    h = (float*)wsp;
    wsp += hbytes;
    wsn -= hbytes;
  }
  if (!spectra_ws_ok(kind, pts, p->D, wsp, wsn, true)) return HYENA_EWORKSPACE;
  Twiddles tw;
  if ((st = get_twiddles(&tw))) return st;
  FilterArgs a{p->F, p->H, p->D, p->W1, p->b1, p->W2, p->b2, p->alpha};
  if (is3d(kind)) st = hip_status(launch_filter3d(a, h, stream, circ3(kind)));
  else st = hip_status(launch_filter1d(a, (int)pts, h, stream));
  if (st) return st;
  return spectra_from_taps(kind, pts, h, p->D, spectrum, wsp, wsn, true, tw, stream);
}

int hyena_film_filter_workspace_bytes(int64_t B, hyena_dims dims, int mode, int64_t D, size_t* bytes) {
  if (!bytes || B <= 0 || D <= 0) return HYENA_EINVAL;
  bool ps = false;
  mode = split_mode(mode, &ps);
  int64_t pts = 0;
  int st = check_dims(dims, mode, &pts);
  if (st) return st;
  const int kind = kind_of(mode, dims);
  const int64_t nch = B * D;
  *bytes = film_scratch_floats((int)B, (int)D) * sizeof(float);
  *bytes = (*bytes + 255) / 256 * 256 + (size_t)nch * taps_per_channel(kind, pts) * sizeof(float);
  const size_t per = filter_intermediate_bytes(kind, pts);
  if (per) *bytes += 256 + (size_t)filter_chunk_rows((int64_t)per, nch) * per;
  return HYENA_OK;
}

int hyena_film_filter_gen(const hyena_film_params* p, int64_t B, int32_t R, const float* registers, hyena_dims dims,
                          int mode, float* h_time, void* spectrum, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!p || !registers || (!spectrum && !h_time) || !ws || B <= 0 || R <= 0 || p->D <= 0 || p->E <= 0)
    return HYENA_EINVAL;
  const float* need[] = {p->q, p->A1, p->a1, p->omega0, p->A2, p->a2, p->A3, p->a3, p->G1, p->g1,
                         p->P1, p->p1, p->G2, p->g2, p->P2, p->p2, p->sigma};
  for (const float* q : need)
    if (!q) return HYENA_EINVAL;
  bool ps = false;
  mode = split_mode(mode, &ps);
  int64_t pts = 0;
  int st = check_dims(dims, mode, &pts);
  if (st) return st;
  const int kind = kind_of(mode, dims);
  if (p->H != kFilmHidden || p->E > kFilmMaxE || R > kFilmMaxR || B > 65535) return HYENA_EUNSUPPORTED;
  const int64_t nch = B * p->D;
  if (nch > (int64_t)INT32_MAX) return HYENA_EUNSUPPORTED;
  char* wsp = (char*)ws;
  size_t wsn = ws_bytes;
  const size_t mod_b = film_scratch_floats((int)B, p->D) * sizeof(float);
  if (!ws_align256(wsp, wsn) || wsn < mod_b) return HYENA_EWORKSPACE;
  float* mod = (float*)wsp;
  wsp += mod_b;
  wsn -= mod_b;
  float* h = h_time;
  if (!h) {
    const size_t hbytes = (size_t)nch * taps_per_channel(kind, pts) * sizeof(float);
    if (!ws_align256(wsp, wsn) || wsn < hbytes) return HYENA_EWORKSPACE;
    h = (float*)wsp;
    wsp += hbytes;
    wsn -= hbytes;
  }
  if (spectrum && !spectra_ws_ok(kind, pts, nch, wsp, wsn, false)) return HYENA_EWORKSPACE;
  Twiddles tw;
  if ((st = get_twiddles(&tw))) return st;
  FilmArgs a{p->E, p->H, p->D, dims.ndim, p->q, p->A1, p->a1, p->omega0, p->A2, p->a2, p->A3, p->a3,
             p->G1, p->g1, p->P1, p->p1, p->G2, p->g2, p->P2, p->p2, p->sigma};
  if ((st = hip_status(launch_film_prep(a, registers, (int)B, R, mod, stream)))) return st;
  if (is3d(kind)) st = hip_status(launch_film_filter3d(a, mod, (int)B, h, stream, circ3(kind)));
  else st = hip_status(launch_film_filter1d(a, mod, (int)B, (int)pts, h, stream));
  if (st || !spectrum) return st;
  return spectra_from_taps(kind, pts, h, nch, spectrum, wsp, wsn, false, tw, stream);
}

int hyena_fftconv(int64_t B, int64_t D, hyena_dims dims, int dtype, int mode, const void* u, const void* spectrum,
                  const void* gate, void* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (B <= 0 || D <= 0 || !u || !spectrum || !y || (dtype != HYENA_F32 && dtype != HYENA_BF16)) return HYENA_EINVAL;
  if (B * D > (int64_t)INT32_MAX) return HYENA_EUNSUPPORTED;
  bool ps = false;
  mode = split_mode(mode, &ps);
  const int hsb = ps ? (int)D : 0;
  int64_t pts = 0;
  int st = check_dims(dims, mode, &pts);
  if (st) return st;
  const int kind = kind_of(mode, dims);
  const size_t tb = (size_t)B * D * pts * elem_bytes(dtype);
  if (y != u && overlaps(y, tb, u, tb)) return HYENA_EALIAS;
  if (gate && y != gate && overlaps(y, tb, gate, tb)) return HYENA_EALIAS;
  int chunk = 0;
  const size_t per = row_intermediate_bytes(kind, pts, dtype);
  int ways = 1;
  bool mfl = false;   // the long-row matrix-core kernels
  const void* xs[1] = {gate};
  if (per) {
    const bool ws_ok = ws && !((size_t)ws & 255u);
    if (ws_ok && use_mfl(kind, dtype, pts, hsb, 1, u, xs, y)) {
      chunk = pair_chunk(mfl_row_bytes(log2i(pts)), B * D, ws_bytes, &ways, kChunkMB);
      mfl = chunk >= 1;
    }
    if (!mfl) chunk = ws_ok ? pair_chunk(per, B * D, ws_bytes, &ways, chunk_mb(kind)) : 0;
    if (chunk < 1) return HYENA_EWORKSPACE;
    if (overlaps(ws, ws_bytes, y, tb) || overlaps(ws, ws_bytes, u, tb) || (gate && overlaps(ws, ws_bytes, gate, tb)))
      return HYENA_EALIAS;
  }
  Twiddles tw;
  if ((st = get_twiddles(&tw))) return st;
  if (chunk) {
    const void* sp[1] = {spectrum};
    DeviceTables* dt = nullptr;
    if (ways > 1 && (st = init_current_device(&dt))) return st;
    std::unique_lock<std::mutex> lk(g_side_mu, std::defer_lock);
    SideStream sd{};
    if (ways > 1) {
      lk.lock();
      sd = dt->side;
      sd.ways = ways;
    }
    if (is3d(kind))
      return hip_status(launch_conv3d(dtype == HYENA_BF16, 1, (int)B, (int)D, u, xs, sp, y, (float2*)ws, chunk, tw,
                                      stream, circ3(kind), hsb, ways > 1 ? &sd : nullptr));
    if (mfl) {
      const void* mats = device_mats();
      if (!mats) return HYENA_EHIP;
      const void* mp[1] = {(const char*)spectrum + (size_t)D * (size_t)pts * sizeof(float2)};
      return hip_status(launch_conv_mfl(log2i(pts), 1, (int)B, (int)D, u, xs, mp, y, ws, chunk, mats, tw, stream,
                                        ways > 1 ? &sd : nullptr));
    }
    return hip_status(launch_conv1d_fourstep(engine_log2(kind, pts), dtype == HYENA_BF16, 1, (int)B, (int)D, u, xs,
                                             sp, y, (float2*)ws, chunk, tw, stream, kind == K_CIRC1 ? 1 : 0, hsb,
                                             ways > 1 ? &sd : nullptr));
  }
  if (kind == K_CIRC1)
    return hip_status(launch_conv1d_single(circular_log2(pts), dtype == HYENA_BF16, u, gate, y,
                                           (const float2*)spectrum, (int)B, (int)D, tw, stream, 1, hsb));
  return conv_once(B, D, pts, dtype, u, spectrum, gate, y, tw, stream, hsb);
}

int hyena_operator(int order, int64_t B, int64_t D, hyena_dims dims, int dtype, int mode, const void* v,
                   const void* const* x, const void* const* spectra, void* y, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  return run_operator(order, B, D, dims, dtype, mode, v, x, spectra, y, ws, ws_bytes, stream, false);
}

int hyena_operator_noalloc(int order, int64_t B, int64_t D, hyena_dims dims, int dtype, int mode, const void* v,
                           const void* const* x, const void* const* spectra, void* y, hipStream_t stream) {
  return run_operator(order, B, D, dims, dtype, mode, v, x, spectra, y, nullptr, 0, stream, true);
}

int hyena_projection(int order, int64_t B, int64_t L, int64_t d_model, int64_t D, int dtype, const void* x,
                     const void* W, const float* bias, void* const* out, hipStream_t stream) {
  if (order < 1 || B <= 0 || L <= 0 || d_model <= 0 || D <= 0 || !x || !W || !out ||
      (dtype != HYENA_F32 && dtype != HYENA_BF16))
    return HYENA_EINVAL;
  const int nout = order + 1;
  if (nout > kProjMaxOut) return HYENA_EUNSUPPORTED;
  for (int j = 0; j < nout; ++j)
    if (!out[j]) return HYENA_EINVAL;
  const int es = (int)elem_bytes(dtype);
  const int64_t M = nout * D;
  if (B > INT32_MAX || L > INT32_MAX || M > INT32_MAX || !projection_supported(B, L, d_model, M, es))
    return HYENA_EUNSUPPORTED;
  const size_t ob = (size_t)B * D * L * es;
  const size_t xb = (size_t)B * L * d_model * es, wb = (size_t)M * d_model * es;
  for (int j = 0; j < nout; ++j) {
    if (overlaps(out[j], ob, x, xb) || overlaps(out[j], ob, W, wb) || (bias && overlaps(out[j], ob, bias, M * 4)))
      return HYENA_EALIAS;
    for (int i = 0; i < j; ++i)
      if (overlaps(out[j], ob, out[i], ob)) return HYENA_EALIAS;
  }
  return hip_status(launch_projection(dtype == HYENA_BF16, x, W, bias, out, nout, (int)B, (int)L, (int)d_model,
                                      (int)D, stream));
}

// ---- streaming decode.  State: hist [order][B*D][L] fp32, fut [order][B*D][L] fp32, then the multi-pass
// workspace of one order's convolution (long L only).
namespace {
int decode_check(int order, int64_t B, int64_t D, int64_t L, int64_t* rows) {
  if (order < 1 || B <= 0 || D <= 0 || L <= 0) return HYENA_EINVAL;
  if (order > kDecodeMaxOrder) return HYENA_EUNSUPPORTED;
  if (B * D > (int64_t)INT32_MAX / 64) return HYENA_EUNSUPPORTED;
  hyena_dims dims{};
  dims.ndim = 1;
  dims.n[0] = L;
  int64_t pts = 0;
  const int st = check_dims(dims, HYENA_CAUSAL, &pts);
  if (st) return st;
  *rows = B * D;
  return HYENA_OK;
}
size_t decode_plane_bytes(int64_t rows, int64_t L) { return (size_t)rows * (size_t)L * sizeof(float); }
size_t decode_ws_bytes(int64_t rows, int64_t L) {
  const size_t per = row_intermediate_bytes(K_CAUSAL, L, HYENA_F32);   // decode convolutions run in fp32
  return per ? (size_t)default_chunk_rows((int64_t)per, rows) * per : 0;
}
}  // namespace

int hyena_decode_state_bytes(int order, int64_t B, int64_t D, int64_t L, size_t* bytes) {
  if (!bytes) return HYENA_EINVAL;
  int64_t rows = 0;
  const int st = decode_check(order, B, D, L, &rows);
  if (st) return st;
  *bytes = 2 * (size_t)order * decode_plane_bytes(rows, L) + decode_ws_bytes(rows, L);
  return HYENA_OK;
}

int hyena_decode_reset(int order, int64_t B, int64_t D, int64_t L, void* state, size_t state_bytes,
                       hipStream_t stream) {
  int64_t rows = 0;
  int st = decode_check(order, B, D, L, &rows);
  if (st) return st;
  if (!state) return HYENA_EINVAL;
  size_t need = 0;
  hyena_decode_state_bytes(order, B, D, L, &need);
  if (((size_t)state & 255u) || state_bytes < need) return HYENA_EWORKSPACE;
  // the prefix convolutions read whole history rows: everything past the last token must be zero; the
  // prefix contributions are cleared too, so that a state holds no values of an earlier sequence
  return hip_status(hipMemsetAsync(state, 0, 2 * (size_t)order * decode_plane_bytes(rows, L), stream));
}

int hyena_decode_step(int order, int64_t B, int64_t D, int64_t L, int64_t block, int64_t t, int dtype, int mode,
                      const void* v_t, const void* const* x_t, const float* const* taps, const void* const* spectra,
                      void* y_t, void* state, size_t state_bytes, hipStream_t stream) {
  int64_t rows = 0;
  int st = decode_check(order, B, D, L, &rows);
  if (st) return st;
  bool ps = false;
  if (split_mode(mode, &ps) != HYENA_CAUSAL) return HYENA_EUNSUPPORTED;
  const int hsb = ps ? (int)D : 0;
  if (!v_t || !x_t || !taps || !spectra || !y_t || !state) return HYENA_EINVAL;
  if (dtype != HYENA_F32 && dtype != HYENA_BF16) return HYENA_EINVAL;
  for (int i = 0; i < order; ++i)
    if (!x_t[i] || !taps[i] || !spectra[i]) return HYENA_EINVAL;
  if (t < 0 || t >= L) return HYENA_EINVAL;
  if (!is_pow2(block) || block > L) return HYENA_EUNSUPPORTED;
  size_t need = 0;
  hyena_decode_state_bytes(order, B, D, L, &need);
  if (((size_t)state & 255u) || state_bytes < need) return HYENA_EWORKSPACE;
  const size_t tok = (size_t)rows * elem_bytes(dtype);
  if (overlaps(y_t, tok, state, need) || overlaps(y_t, tok, v_t, tok) || overlaps(v_t, tok, state, need))
    return HYENA_EALIAS;
  hyena_dims dims{};
  dims.ndim = 1;
  dims.n[0] = L;
  size_t spb = 0;
  if ((st = hyena_spectrum_bytes(dims, mode, ps ? rows : D, &spb))) return st;
  const size_t tapb = (size_t)(ps ? rows : D) * (size_t)L * sizeof(float);
  for (int i = 0; i < order; ++i)
    if (overlaps(y_t, tok, x_t[i], tok) || overlaps(x_t[i], tok, state, need) || overlaps(taps[i], tapb, state, need) ||
        overlaps(spectra[i], spb, state, need) || overlaps(y_t, tok, taps[i], tapb) || overlaps(y_t, tok, spectra[i], spb))
      return HYENA_EALIAS;
  float* hist = (float*)state;
  const size_t plane = (size_t)rows * (size_t)L;
  float* fut = hist + (size_t)order * plane;
  const int64_t t0 = t - t % block;
  if (t > 0 && t0 == t) {
    // block boundary: the contribution of the whole stored prefix to every later position, by the FFT
    // convolution of each order's history row with that order's cached spectrum (no gate)
    Twiddles tw;
    if ((st = get_twiddles(&tw))) return st;
    const int lg = log2i(L);
    const size_t per = row_intermediate_bytes(K_CAUSAL, L, HYENA_F32);   // decode convolutions run in fp32
    const int chunk = per ? (int)default_chunk_rows((int64_t)per, rows) : 0;
    for (int i = 0; i < order; ++i) {
      float* h_i = hist + (size_t)i * plane;
      float* f_i = fut + (size_t)i * plane;
      if (chunk) {
        const void* xs[1] = {nullptr};
        const void* sp[1] = {spectra[i]};
        st = hip_status(launch_conv1d_fourstep(lg, 0, 1, (int)B, (int)D, h_i, xs, sp, f_i,
                                               (float2*)(fut + (size_t)order * plane), chunk, tw, stream, 0, hsb));
      } else {
        st = hip_status(launch_conv1d_single(lg, 0, h_i, nullptr, f_i, (const float2*)spectra[i], (int)B, (int)D, tw,
                                             stream, 0, hsb));
      }
      if (st) return st;
    }
  }
  return hip_status(launch_decode_step(order, dtype == HYENA_BF16, v_t, x_t, taps, hist, fut, y_t, (int)rows, (int)D,
                                       (int)L, (int)t, (int)t0, ps ? 1 : 0, stream));
}

int hyena_decode_prefill(int order, int64_t B, int64_t D, int64_t L, int64_t block, int64_t P, int dtype, int mode,
                         const void* v, const void* const* x, const void* const* spectra, void* y, void* state,
                         size_t state_bytes, hipStream_t stream) {
  int64_t rows = 0;
  int st = decode_check(order, B, D, L, &rows);
  if (st) return st;
  bool ps = false;
  if (split_mode(mode, &ps) != HYENA_CAUSAL) return HYENA_EUNSUPPORTED;
  const int hsb = ps ? (int)D : 0;
  if (!v || !x || !spectra || !y || !state) return HYENA_EINVAL;
  for (int i = 0; i < order; ++i)
    if (!x[i] || !spectra[i]) return HYENA_EINVAL;
  if (dtype != HYENA_F32 && dtype != HYENA_BF16) return HYENA_EINVAL;
  if (!is_pow2(block) || block > L) return HYENA_EUNSUPPORTED;
  if (P < 1 || P > L || P % block) return HYENA_EINVAL;
  size_t need = 0;
  hyena_decode_state_bytes(order, B, D, L, &need);
  if (((size_t)state & 255u) || state_bytes < need) return HYENA_EWORKSPACE;
  const size_t pb = (size_t)rows * (size_t)P * elem_bytes(dtype);
  if (overlaps(y, pb, v, pb) || overlaps(y, pb, state, need) || overlaps(v, pb, state, need)) return HYENA_EALIAS;
  hyena_dims dims{};
  dims.ndim = 1;
  dims.n[0] = L;
  size_t spb = 0;
  if ((st = hyena_spectrum_bytes(dims, mode, ps ? rows : D, &spb))) return st;
  for (int i = 0; i < order; ++i)
    if (overlaps(y, pb, x[i], pb) || overlaps(x[i], pb, state, need) || overlaps(spectra[i], spb, state, need) ||
        overlaps(y, pb, spectra[i], spb))
      return HYENA_EALIAS;
  Twiddles tw;
  if ((st = get_twiddles(&tw))) return st;
  float* hist = (float*)state;
  const size_t plane = (size_t)rows * (size_t)L;
  float* fut = hist + (size_t)order * plane;
  const int bf = dtype == HYENA_BF16;
  const int lg = log2i(L);
  const size_t per = row_intermediate_bytes(K_CAUSAL, L, HYENA_F32);   // decode convolutions run in fp32
  const int chunk = per ? (int)default_chunk_rows((int64_t)per, rows) : 0;
  // the prompt through the orders on the whole-row FFT path, each order's input kept as its history
  if ((st = hip_status(launch_decode_prefill(0, bf, v, nullptr, hist, nullptr, (int)rows, (int)L, (int)P, stream))))
    return st;
  for (int i = 0; i < order; ++i) {
    float* h_i = hist + (size_t)i * plane;
    const bool last = i + 1 == order;
    float* c = last ? fut : hist + (size_t)(i + 1) * plane;   // the prefix contributions are rebuilt at t = P
    if (chunk) {
      const void* xs[1] = {nullptr};
      const void* sp[1] = {spectra[i]};
      st = hip_status(launch_conv1d_fourstep(lg, 0, 1, (int)B, (int)D, h_i, xs, sp, c,
                                             (float2*)(fut + (size_t)order * plane), chunk, tw, stream, 0, hsb));
    } else {
      st = hip_status(launch_conv1d_single(lg, 0, h_i, nullptr, c, (const float2*)spectra[i], (int)B, (int)D, tw,
                                           stream, 0, hsb));
    }
    if (st) return st;
    if ((st = hip_status(launch_decode_prefill(1, bf, x[i], c, c, last ? y : nullptr, (int)rows, (int)L, (int)P,
                                               stream))))
      return st;
  }
  return HYENA_OK;
}

int hyena_spectrum_export(hyena_dims dims, int mode, int64_t D, const void* spectrum, void* H, hipStream_t stream) {
  if (D <= 0 || !spectrum || !H) return HYENA_EINVAL;
  bool ps = false;
  mode = split_mode(mode, &ps);
  if (D > (int64_t)INT32_MAX) return HYENA_EUNSUPPORTED;
  int64_t pts = 0;
  int st = check_dims(dims, mode, &pts);
  if (st) return st;
  const int kind = kind_of(mode, dims);
  if (is3d(kind))
    return hip_status(launch_export3d((const float2*)spectrum, (float2*)H, (int)D, stream, circ3(kind)));
  if (kind == K_CIRC1 && multipass1d(kind, pts))
    return hip_status(launch_export1d_fourstep(circular_log2(pts), (const float2*)spectrum, (float2*)H, (int)D, stream));
  if (kind == K_CIRC1)
    return hip_status(launch_export1d_single(circular_log2(pts), (const float2*)spectrum, (float2*)H, (int)D, stream));
  if (is_multipass(pts))
    return hip_status(launch_export1d_fourstep(log2i(pts), (const float2*)spectrum, (float2*)H, (int)D, stream));
  return hip_status(launch_export1d_single(log2i(pts), (const float2*)spectrum, (float2*)H, (int)D, stream));
}

}  // extern "C"
