// Host-side launchers exported by each kernel translation unit to the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include "fft_core.h"

namespace hyena {

// Scratch of the entry point that allocates nothing (hyena_operator_noalloc): its multi-pass workspace.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;

// ---- 1-D, one workgroup per row: an M = 2^log2L point packed transform, 10 <= log2L <= 14.
// full = 0: causal, rows of M samples (zero-padded to 2M); full = 1: periodic, rows of 2M samples.
bool single_pass_supported(int log2L);
// hsb (every conv launcher): 0 when the spectrum holds one filter per channel d, D when it holds one per
// (b, d) in [B, D] order (input-dependent filters).
hipError_t launch_conv1d_single(int log2L, int bf16, const void* u, const void* gate, void* y, const float2* Hs,
                                int B, int D, const Twiddles& tw, hipStream_t s, int full = 0, int hsb = 0);
// Orders 0..order-1 (order <= kConvMaxChain) in one launch, u_i kept on chip in fp32 between them.
// gates[i] may be NULL only when order == 1.
constexpr int kConvMaxChain = 8;
struct ConvChain {
  const void* gate[kConvMaxChain];
  const float2* spectrum[kConvMaxChain];
};
hipError_t launch_conv1d_chain(int log2L, int bf16, const void* u, const void* const* gates,
                               const float2* const* spectra, int order, void* y, int B, int D, const Twiddles& tw,
                               hipStream_t s, int full = 0, int hsb = 0);
hipError_t launch_spectrum1d_single(int log2L, const float* h, float2* Hs, int D, const Twiddles& tw,
                                    hipStream_t s, int full = 0);
hipError_t launch_export1d_single(int log2L, const float2* Hs, float2* H, int D, hipStream_t s);

// ---- 1-D, multi-pass: an M = 2^log2L point packed transform, 15 <= log2L <= 20; I is a workspace of
// `chunk` rows of M complex values.  full = 0: causal, rows of M samples; full = 1: periodic, rows of
// 2M samples.  x[i] may be NULL for the last order only (no gate).
bool fourstep_supported(int log2L);
// Workspace bytes per row: the fp32 intermediate (M complex fp32), or with bf16 storage its block-scaled fp16
// form (M fp16 pairs and 1024 words of block exponents).  u_i stays fp32 between orders either way.
size_t fourstep_row_bytes(int log2L, int bf16);
// side (optional): side streams and their events; the chunks then cycle over the caller's stream and
// ways - 1 side streams (forked from and joined back into the caller's stream), each stream with its own
// part of I, which must hold ways * chunk rows.
constexpr int kSideStreams = 2;
struct SideStream {
  hipStream_t s[kSideStreams];
  hipEvent_t fork, join[kSideStreams];
  int ways;                      // streams the chunks cycle over, the caller's included (2 .. kSideStreams + 1)
};
// the side streams start after the caller's work so far
inline hipError_t side_fork(const SideStream* sd, hipStream_t s0) {
  hipError_t e = hipEventRecord(sd->fork, s0);
  for (int j = 0; j + 1 < sd->ways && e == hipSuccess; ++j) e = hipStreamWaitEvent(sd->s[j], sd->fork, 0);
  return e;
}
// the caller's stream continues after the side streams' work
inline hipError_t side_join(const SideStream* sd, hipStream_t s0) {
  hipError_t e = hipSuccess;
  for (int j = 0; j + 1 < sd->ways && e == hipSuccess; ++j) {
    e = hipEventRecord(sd->join[j], sd->s[j]);
    if (e == hipSuccess) e = hipStreamWaitEvent(s0, sd->join[j], 0);
  }
  return e;
}
hipError_t launch_conv1d_fourstep(int log2L, int bf16, int order, int B, int D, const void* v,
                                  const void* const* x, const void* const* spectra, void* y, float2* I, int chunk,
                                  const Twiddles& tw, hipStream_t s, int full = 0, int hsb = 0,
                                  const SideStream* side = nullptr);
hipError_t launch_spectrum1d_fourstep(int log2L, const float* h, float2* Hs, int D, float2* I, int chunk,
                                      const Twiddles& tw, hipStream_t s, int full = 0);
hipError_t launch_export1d_fourstep(int log2L, const float2* Hs, float2* H, int D, hipStream_t s);

// ---- 3-D, 64^3 grid: circ = 0 zero-padded to 128^3 (non-causal "same" convolution),
//      circ = 1 periodic on the 64^3 grid itself
bool grid3d_supported(int64_t nx, int64_t ny, int64_t nz);
size_t conv3d_volume_bytes(int circ);                 // intermediate per (b, d) volume
size_t conv3d_filter_volume_bytes(int circ);          // intermediate per channel while building a spectrum
size_t conv3d_spectrum_bytes_per_channel(int circ);
size_t conv3d_taps_per_channel(int circ);             // (2n-1)^3 or n^3
// side (optional): as for launch_conv1d_fourstep; I then holds 2 * chunk volumes.
hipError_t launch_conv3d(int bf16, int order, int B, int D, const void* v, const void* const* x,
                         const void* const* spectra, void* y, float2* I, int chunk, const Twiddles& tw, hipStream_t s,
                         int circ, int hsb = 0, const SideStream* side = nullptr);
hipError_t launch_spectrum3d(const float* h, float2* Hs, int D, float2* I, int chunk, const Twiddles& tw,
                             hipStream_t s, int circ);
hipError_t launch_export3d(const float2* Hs, float2* H, int D, hipStream_t s, int circ);

// ---- matrix-core path: bf16 storage, L = 8192, rows in pairs of one channel (B even)
bool mfma_pair_supported(int log2L, int B);
size_t mfma_pair_spectrum_bytes_per_channel();
constexpr size_t kMfmaMatrixCount = (9 + 16 * 16 + 1) * 64 * 8;   // 16-bit values in the DFT-matrix table
void mfma_matrices_host(uint16_t* out);
// Orders 1..order back to back in one launch (u_i stays on chip); spectra[i] = matrix-core copies.
constexpr int kMfmaMaxChain = 8;
hipError_t launch_conv_mfma(const void* u, const void* const* gates, const void* const* spectra, int order,
                            void* y, const void* mats, int B, int D, hipStream_t s);
hipError_t launch_pair_spectrum(const float2* Hnat, void* Hc, int D, hipStream_t s);

// ---- matrix-core path for long rows: bf16 storage, L = 2^15, 2^16 or 2^17, each row alone (any B).
// The workspace holds chunk_rows rows of mfl_row_bytes each (ways * chunk_rows with side streams);
// spectra[i] = the long-row split-coefficient copies (mfl_spectrum_bytes_per_channel per channel).
bool mfl_supported(int log2L);
size_t mfl_row_bytes(int log2L);
size_t mfl_spectrum_bytes_per_channel(int log2L);
hipError_t launch_conv_mfl(int log2L, int order, int B, int D, const void* v, const void* const* x,
                           const void* const* spectra, void* y, void* ws, int chunk_rows, const void* mats,
                           const Twiddles& tw, hipStream_t s, const SideStream* side = nullptr);
// from the natural-order bins 0..L of each channel's 2L-point spectrum ([D][L + 1])
hipError_t launch_mfl_spectrum(int log2L, const float2* Hnat, void* Hc, int D, const Twiddles& tw, hipStream_t s);

// ---- implicit filter taps
struct FilterArgs {
  int F, H, D;
  const float *W1, *b1, *W2, *b2, *alpha;
};
hipError_t launch_filter1d(const FilterArgs& a, int L, float* h, hipStream_t s);
hipError_t launch_filter3d(const FilterArgs& a, float* h, hipStream_t s, int circ);

// ---- input projection: x [B, L, K] token-major, W [nout * D, K] -> nout channel-major outputs [B, D, L]
constexpr int kProjMaxOut = 9;      // v and up to 8 gates
bool projection_supported(int64_t B, int64_t L, int64_t K, int64_t M, int es);
hipError_t launch_projection(int bf16, const void* x, const void* W, const float* bias, void* const* outs, int nout,
                             int B, int L, int K, int D, hipStream_t s);

// ---- streaming decode: one token of every (b, d) row through all orders.  hist, fut: [order][rows][L]
// fp32 (history of each order's input; contributions of the positions before t0, the start of t's
// block); taps[i]: [D][L] fp32, or [rows][L] with per_sample (only the first t - t0 + 1 taps of a row are
// read); v_t, x_t[i], y_t: [rows] of fp32 or (bf16 = 1) bf16.
constexpr int kDecodeMaxOrder = 8;
hipError_t launch_decode_step(int order, int bf16, const void* v_t, const void* const* x_t,
                              const float* const* taps, float* hist, const float* fut, void* y_t, int rows, int D,
                              int L, int t, int t0, int per_sample, hipStream_t s);
// prompt staging for rows of L (positions >= P zero): mode 0 dst = v; mode 1 dst = x * c, or y = x * c when y
// is not NULL (a and y: [rows][P] tokens; c, dst: [rows][L] fp32)
hipError_t launch_decode_prefill(int mode, int bf16, const void* a, const float* c, float* dst, void* y, int rows,
                                 int L, int P, hipStream_t s);

// ---- input-dependent filters: FiLM-modulated SIREN with a Gaussian window, one filter per (b, d)
constexpr int kFilmHidden = 64;     // SIREN units per layer
constexpr int kFilmMaxE = 4096;     // register width
constexpr int kFilmMaxR = 1024;     // register tokens per sample
struct FilmArgs {
  int E, H, D, NC;                  // register width, hidden units, channels, coordinates (1 or 3)
  const float *q, *A1, *a1, *omega0, *A2, *a2, *A3, *a3, *G1, *g1, *P1, *p1, *G2, *g2, *P2, *p2, *sigma;
};
// scratch (film_scratch_floats floats): [B, 4, H] FiLM vectors (gamma_1, beta_1, gamma_2, beta_2) from the
// registers reg [B, R, E], then A2 and A3 transposed ([H][H], [H][D])
size_t film_scratch_floats(int B, int D);
hipError_t launch_film_prep(const FilmArgs& a, const float* reg, int B, int R, float* scratch, hipStream_t s);
// taps h[B, D, points] (1-D t = 0..L-1; 3-D offsets as launch_filter3d), after launch_film_prep
hipError_t launch_film_filter1d(const FilmArgs& a, const float* scratch, int B, int L, float* h, hipStream_t s);
hipError_t launch_film_filter3d(const FilmArgs& a, const float* scratch, int B, float* h, hipStream_t s, int circ);

}  // namespace hyena
