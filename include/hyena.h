/*
 * hyena.h -- C ABI of the MI355X (gfx950) Hyena operator library, libhyena.so.
 *
 * The operator (Hyena study note, obsidian-dorae222.pages.dev/20.AI/22.SSM/hyena, section
 * "아키텍처 상세", step 3 equation, and its listing hyena_operator):
 *
 *     u_0 = v,   u_i = x_i * (h_i conv u_{i-1})   (i = 1..order),   y = u_order
 *
 * with x_1 the innermost gate, paired with h_1.  Each h_i is an implicit filter (same page, step 2:
 * h(t) = FFN(pos_enc(t)) * exp(-alpha t); EulerStack "4. Hyena 상세", how it works 1: small MLP over
 * sinusoidal features with an exponential decay window), and "conv" is
 *   - 1-D (HYENA_CAUSAL): c[t] = sum_{s<=t} h[t-s] u[s], t < L, by FFT on a 2L zero-padded grid
 *     (EulerStack page, how it works 2; HyenaND summary, boundary handling);
 *   - 3-D (HYENA_LINEAR): c[p] = sum_{q in grid} h[p-q] u[q] over an n^3 grid, offsets p-q in
 *     [-(n-1), n-1]^3, by 3-D FFT on a (2n)^3 zero-padded grid ("Native Multi-Dimensional
 *     Subquadratic Operators via Input Dependent Long Convolutions" summary, method: native N-D
 *     convolution; boundary handling: zero-pad to twice the size);
 *   - periodic (HYENA_CIRCULAR), by FFT on the grid itself, no padding (same summary, boundary
 *     handling: circular convolutions for periodic systems): 1-D c[t] = sum_{s<L} h[(t-s) mod L] u[s]
 *     with the 1-D filter's taps t = 0..L-1 (one period); 3-D c[p] = sum_q h[(p-q) mod n] u[q] with
 *     the 3-D filter on the centred offsets [-n/2, n/2)^3 (one period).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library never frees them.
 *   - Activations are channel-major and contiguous: [B, D, L] (1-D) or [B, D, nx, ny, nz] (3-D),
 *     element type given by hyena_dtype.  bf16 is a storage type only: v, the gates and y are bf16 (stores
 *     round to nearest even); the intermediates u_i of the recurrence stay fp32, and so does every transform
 *     intermediate except two: the matrix-core paths' operands (below) and, with bf16 storage, the
 *     multi-pass 1-D plans' workspace, held as fp16 with a power-of-two scale per block of values (each
 *     block's largest component at most 2^15; 1.7e-3 -> 2.6e-3 on the order-3, 65536-sample workload with the
 *     fp32 transforms).
 *   - Arithmetic: fp32 on every path (radix butterflies on the vector units, fp32 twiddles, fp32 spectra and
 *     spectral products), with two exceptions, the matrix-core paths of hyena_fftconv / hyena_operator with
 *     bf16 storage and order <= 3: causal L = 8192 with even B (rows b and b+1 of a channel transformed
 *     together, each with its own scale), and causal L = 2^15, 2^16, 2^17 (each row on its own; column
 *     passes in fp32, 16384-point plane transforms on the matrix cores).  Their DFT steps are matrix products
 *     with fp32 accumulation whose operands are fp16 -- the DFT matrices, a copy of the filter spectrum (for
 *     the long rows, two split coefficients per bin) and the data entering each product are rounded to fp16
 *     after an exact power-of-two scaling that keeps them in fp16's range -- except the first product at
 *     L = 8192, which takes the bf16 inputs exactly against a matrix split into two bf16 parts; at L = 8192
 *     u_i passes between orders in fp16 the same way; the twiddle, split and spectral products between the
 *     matrix products are packed fp16 multiplies.  Measured error against an fp64 evaluation (relative L2
 *     per row, max over rows): 3.2e-3 at order 2 on the 8192-sample workload, 4.9e-3 at order 3 on the
 *     65536-sample workload, at most 4.9e-3 at order 3 without a decay window, against 1.7e-3 to 2e-3 for the
 *     fp32 paths with bf16 storage.  At L = 8192 the two rows of a pair share the transform's rounding: a row
 *     holding a single impulse beside a full row measured 1.0e-2, and a non-finite value in one row makes
 *     its partner's output non-finite too.
 *   - Calls are asynchronous on the caller's HIP stream and never synchronise the host, except the
 *     first call on a device, which uploads the library's constant tables (about 800 KB) once with a
 *     blocking copy; hyena_init() does that upload ahead of time (for example before graph capture).
 *   - The library holds no state across calls besides those immutable tables, which live in device arrays
 *     of the library's code object (the library never calls hipMalloc).
 *   - Return value: HYENA_OK or a negative status (below); arguments are validated before anything
 *     is launched, so an error return means nothing was enqueued.  Device faults surface at the
 *     caller's next synchronisation.  hyena_status_str() names a status.
 */
#ifndef HYENA_H_
#define HYENA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  HYENA_OK = 0,
  HYENA_EINVAL = -1,        /* null pointer, order < 1, non-positive size, mode/ndim mismatch       */
  HYENA_EUNSUPPORTED = -2,  /* size not a power of two or outside the supported range; F/H not 64  */
  HYENA_EWORKSPACE = -3,    /* workspace missing or smaller than the size the query returned      */
  HYENA_EHIP = -4,          /* a HIP runtime call or launch failed                                   */
  HYENA_EALIAS = -5         /* the output overlaps an input in a way that is not allowed            */
};

typedef enum { HYENA_F32 = 0, HYENA_BF16 = 1 } hyena_dtype;

typedef enum {
  HYENA_CAUSAL = 0,   /* 1-D causal linear convolution (pad to 2L, keep [0, L))                  */
  HYENA_LINEAR = 1,   /* 3-D non-causal zero-padded "same" convolution (pad each axis to 2n)      */
  HYENA_CIRCULAR = 2  /* periodic boundary, no padding: 1-D rows or the 3-D grid                    */
} hyena_mode;

/* Flag OR'ed into a mode: the spectra hold one filter per (b, d) in [B, D] order -- the input-dependent
 * filters of hyena_film_filter_gen -- instead of one per channel.  Accepted by every entry point that
 * takes a mode; hyena_fftconv / hyena_operator then read filter b*D + d for row (b, d) (always on the
 * fp32 transform engine), and hyena_spectrum_bytes / hyena_spectrum_export take D = B * channels. */
#define HYENA_PER_SAMPLE 8

/* Grid shape: 1-D {1, {L, 0, 0}}; 3-D {3, {nx, ny, nz}}.
 * Supported: HYENA_CAUSAL L = 2^k, 2^10 <= L <= 2^20; HYENA_CIRCULAR 1-D L = 2^k, 2^11 <= L <= 2^21,
 * or nx = ny = nz = 64; HYENA_LINEAR nx = ny = nz = 64. */
typedef struct {
  int32_t ndim;
  int64_t n[3];
} hyena_dims;

/* One order's implicit-filter parameters (device pointers, fp32, row-major):
 *   W1 [H, F], b1 [H], W2 [D, H], b2 [D], alpha [D] (alpha >= 0 is a precondition, not checked).
 * Supported: H = 64; F = 64 for 1-D, F = 96 for 3-D (16 frequencies x {sin, cos} per axis). */
typedef struct {
  int32_t F, H, D;
  const float *W1, *b1, *W2, *b2, *alpha;
} hyena_filter_params;

/* Size in bytes of one order's filter spectrum for D channels (an opaque, engine-ordered array):
 * causal 8L bytes per channel (except with HYENA_PER_SAMPLE, followed for L = 8192 by an fp16 copy laid out
 * for the matrix-core kernel, 36.25 KB per channel, and for L = 2^15 .. 2^17 by the long-row matrix-core
 * kernels' fp16 split coefficients, 8L + 256 bytes per channel); periodic 1-D 4L bytes per channel; 3-D
 * 128*128*65*8 bytes per channel (zero-padded) or 64*64*33*8 (periodic).  With HYENA_PER_SAMPLE, D counts
 * filters (B*D). */
int hyena_spectrum_bytes(hyena_dims dims, int mode, int64_t D, size_t *bytes);

/* Workspace bytes hyena_filter_gen needs: room for the taps (used when h_time is NULL) plus, for
 * multi-pass lengths (causal L > 16384, periodic L > 32768, 3-D), the transform intermediate of a
 * chunk of channels. */
int hyena_filter_workspace_bytes(hyena_dims dims, int mode, int64_t D, size_t *bytes);

/* Workspace bytes hyena_fftconv / hyena_operator need (0 when the transform fits on chip). */
int hyena_workspace_bytes(int order, int64_t B, int64_t D, hyena_dims dims, int dtype, int mode, size_t *bytes);

/* Implicit filter of one order: writes the taps (1-D: h_time[D, L]; 3-D zero-padded:
 * h_time[D, 2n-1, 2n-1, 2n-1], index = offset + n-1; 3-D periodic: h_time[D, n, n, n], index =
 * offset + n/2) when h_time is not NULL, and the filter spectrum into `spectrum`
 * (hyena_spectrum_bytes bytes).  ws/ws_bytes: scratch of hyena_filter_workspace_bytes bytes (may be
 * NULL/0 when h_time is given and the length runs in one pass, L <= 16384, except causal L = 8192,
 * whose matrix-core copy is staged there, as is the long-row copy of causal L = 2^15 .. 2^17 after the
 * multi-pass intermediate; HYENA_EWORKSPACE when too small).  The spectrum depends
 * only on (params, dims), so callers cache it per length. */
int hyena_filter_gen(const hyena_filter_params *p, hyena_dims dims, int mode, float *h_time, void *spectrum,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/* Input-dependent filter parameters of one order (HyenaND summary, method: registers, FiLM conditioning,
 * kernel synthesis K(x) = w(c) f(c; z(x)) and the SIREN parameterisation with multi-frequency omega_0).
 * Device pointers, fp32, row-major; n = dims.ndim coordinates (c = t/L in 1-D, r/n per axis in 3-D):
 *   z = sum_r a_r reg[b, r],  a = softmax_r(q . reg[b, r])               q [E]
 *   h1 = sin(gamma1 * omega0 * (A1 c + a1) + beta1)                     A1 [H, n], a1 [H], omega0 [H]
 *   h2 = sin(gamma2 * (A2 h1 + a2) + beta2)                             A2 [H, H], a2 [H]
 *   gamma_l = G_l z + g_l,  beta_l = P_l z + p_l                        G_l, P_l [H, E], g_l, p_l [H]
 *   K[b, d, c] = (A3 h2 + a3)_d * exp(-|c|^2 / (2 sigma_d^2))          A3 [D, H], a3 [D], sigma [D] > 0
 * Supported: H = 64, E <= 4096. */
typedef struct {
  int32_t E, H, D;
  const float *q, *A1, *a1, *omega0, *A2, *a2, *A3, *a3;
  const float *G1, *g1, *P1, *p1, *G2, *g2, *P2, *p2, *sigma;
} hyena_film_params;

/* Workspace bytes hyena_film_filter_gen needs: the FiLM vectors (4*H floats per sample) and A2, A3
 * transposed (H*(H + D) floats), the taps of B*D filters (used when h_time is NULL) and, for multi-pass
 * lengths and 3-D, a transform chunk. */
int hyena_film_filter_workspace_bytes(int64_t B, hyena_dims dims, int mode, int64_t D, size_t *bytes);

/* Input-dependent filters of one order for B samples: registers [B, R, E] (device, fp32; the R register
 * tokens' activations, R <= 1024) -> taps h_time [B, D, points as hyena_filter_gen] when not NULL, and
 * the spectra of the B*D filters into `spectrum` (hyena_spectrum_bytes(dims, mode | HYENA_PER_SAMPLE,
 * B*D) bytes), for hyena_fftconv / hyena_operator with mode | HYENA_PER_SAMPLE.  spectrum may be NULL
 * when h_time is given (taps only).  ws (required): hyena_film_filter_workspace_bytes bytes.
 * B <= 65535. */
int hyena_film_filter_gen(const hyena_film_params *p, int64_t B, int32_t R, const float *registers,
                          hyena_dims dims, int mode, float *h_time, void *spectrum, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/* One long convolution with optional gate: y = gate * (h conv u), or y = h conv u when gate == NULL.
 * u, gate, y: [B, D, points] of dtype.  spectrum: from hyena_filter_gen for the same dims and D.
 * bf16 storage with 16-byte-aligned u, gate and y runs on the matrix cores for causal L = 8192 with even B
 * (rows b and b+1 of a channel transformed together) and for causal L = 2^15 .. 2^17 (fp16 operands, see
 * the conventions above); every other case runs the fp32 transform engines.
 * y may equal u or gate exactly (in place); any other overlap returns HYENA_EALIAS. */
int hyena_fftconv(int64_t B, int64_t D, hyena_dims dims, int dtype, int mode, const void *u,
                  const void *spectrum, const void *gate, void *y, void *ws, size_t ws_bytes,
                  hipStream_t stream);

/* The order-N operator y = x_N * (h_N conv (... x_1 * (h_1 conv v))).
 * x: host array of `order` device pointers (x[0] = x_1); spectra: host array of `order` spectra
 * (spectra[i] pairs with x[i]).  y doubles as the buffer between orders; y may equal v exactly but
 * must not overlap any x_i.  ws: hyena_workspace_bytes bytes.
 * Engines: order <= 3 on the matrix-core case (see hyena_fftconv) runs every order in one launch with u_i
 * kept on chip (as fp16 operands, see the conventions above).  Every other single-pass case (causal
 * L <= 16384, periodic L <= 32768) runs up to 8 orders per launch of the fp32 engine with u_i kept on chip in
 * fp32 (beyond 8 orders u passes through y, in the storage type, between launches); the multi-pass plans
 * (longer rows, 3-D; the long-row matrix-core case for orders <= 3) chain the orders through the workspace
 * (u_i itself fp32).  Orders above 3 never take the matrix cores: their 16-bit operands compound across
 * orders towards the bf16 tolerance. */
int hyena_operator(int order, int64_t B, int64_t D, hyena_dims dims, int dtype, int mode, const void *v,
                   const void *const *x, const void *const *spectra, void *y, void *ws, size_t ws_bytes,
                   hipStream_t stream);

/* hyena_operator without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the multi-pass
 * intermediates go to a scratch array of 64 MiB that the library holds in every device's copy of its code
 * object until the process ends; no call allocates (the first call on a device, unless hyena_init came
 * first, uploads the constant tables with a blocking copy).  Same arguments, semantics and results as
 * hyena_operator; the caller still owns v, x, spectra and y.  Rows whose intermediate exceeds the scratch
 * return HYENA_EWORKSPACE (none of the supported sizes does: the largest is 8 MiB per row).  Every call
 * on one device shares that device's scratch, which keeps the last call's contents: calls that overlap in
 * time on one device (on different streams, or from different threads without ordering) race and give
 * wrong results; calls ordered on one stream are safe. */
int hyena_operator_noalloc(int order, int64_t B, int64_t D, hyena_dims dims, int dtype, int mode, const void *v,
                           const void *const *x, const void *const *spectra, void *y, hipStream_t stream);

/* The input projection (Hyena study note, step 1: v, x_1, ..., x_N = split(W_proj x); the listing
 * chunks the projected channels into N + 1 equal parts, v first):
 *   out[j][b, d, t] = sum_k W[j*D + d, k] * x[b, t, k] + bias[j*D + d],   j = 0..order
 * x: token-major [B, L, d_model]; W: [(order+1)*D, d_model] row-major (one row per output channel);
 * both of dtype (bf16: matrix-core products, fp32 accumulation; fp32: fp32 matrix-core products).
 * bias: fp32 [(order+1)*D] or NULL.  out: host array of order+1 device pointers, each [B, D, L] of dtype
 * (channel-major, the layout hyena_operator takes: out[0] = v, out[j] = x_j), written with bf16 rounding
 * to nearest even.  Supported: d_model a multiple of 8 (bf16) or 4 (fp32), order <= 8, W and one
 * sample of x below 2^31 bytes.  Outputs must not overlap x, W, bias or each other. */
int hyena_projection(int order, int64_t B, int64_t L, int64_t d_model, int64_t D, int dtype, const void *x,
                     const void *W, const float *bias, void *const *out, hipStream_t stream);

/* Streaming decode of the causal 1-D operator, one token at a time, with a prefix-spectrum cache (SPECTRE
 * digest, token mixer and generation support: a cache in the role of the KV cache lets a spectral mixer
 * generate without transforming the whole prefix again at every step; the operator itself is the Hyena
 * study note's step 3 equation).  After the tokens t = 0..L-1 of a sequence have gone through
 * hyena_decode_step in order, y_t holds exactly what hyena_operator computes at position t (up to fp32
 * rounding order):  u_0[t] = v[t],  u_i[t] = x_i[t] * sum_{s<=t} h_i[t-s] u_{i-1}[s],  y[t] = u_order[t].
 *
 * How: the positions are grouped in blocks of `block` tokens.  At each block start the library convolves
 * every order's stored history (the tokens so far, zero after them) with that order's cached spectrum by
 * FFT, once, which gives the whole prefix's contribution to every later position; within the block each
 * token adds a direct sum over at most `block` taps.  A larger block means fewer prefix convolutions and
 * longer direct sums.
 *
 * State: one caller-owned device buffer of hyena_decode_state_bytes bytes, 256-byte aligned, holding
 * fp32 [order][B*D][L] histories, fp32 [order][B*D][L] prefix contributions and (L >= 32768) the multi-pass
 * workspace.  It belongs to one sequence: call hyena_decode_reset before the first token of each sequence,
 * then hyena_decode_step for t = 0, 1, 2, ... in order on one stream (the library cannot check the order;
 * skipped or repeated positions give wrong results, not an error).  Calls that share a state buffer must
 * not run concurrently.
 *
 * Sizes: 1 <= order <= 8; L a power of two with 1024 <= L <= 2^20 (the causal sizes of hyena_operator);
 * block a power of two, 1 <= block <= L (block == L: no prefix convolution at all).  Tokens are fp32 or bf16
 * (dtype); the state is fp32 either way.  mode: HYENA_CAUSAL, or HYENA_CAUSAL | HYENA_PER_SAMPLE for input-dependent
 * filters (one per (b, d) from hyena_film_filter_gen: taps [B, D, L], spectra of B*D filters); other modes
 * return HYENA_EUNSUPPORTED.  With bf16 tokens each intermediate u_i (i < order) is rounded to
 * bf16 before it is used, as hyena_operator rounds a stored intermediate. */
int hyena_decode_state_bytes(int order, int64_t B, int64_t D, int64_t L, size_t *bytes);

/* Clears a state buffer -- histories and prefix contributions -- before a new sequence (enqueued on
 * `stream`). */
int hyena_decode_reset(int order, int64_t B, int64_t D, int64_t L, void *state, size_t state_bytes,
                       hipStream_t stream);

/* Token t of the sequence for every (b, d) row.  v_t, x_t[i] (i = 0..order-1, x_t[0] = x_1) and y_t: [B, D]
 * of dtype (index b*D + d; bf16 stores round to nearest even).  taps[i]: fp32 [D, L] (per sample: [B, D, L]),
 * the time-domain filter of order i as the filter generator's h_time (only the first `block` taps of a
 * row are read); spectra[i]: that order's spectrum from the same generator (causal, same L).  y_t must not
 * overlap the inputs, taps, spectra or the state; none of those may overlap the state.  HYENA_EINVAL for t
 * outside [0, L); HYENA_EWORKSPACE for a state that is too small or misaligned. */
int hyena_decode_step(int order, int64_t B, int64_t D, int64_t L, int64_t block, int64_t t, int dtype, int mode,
                      const void *v_t, const void *const *x_t, const float *const *taps, const void *const *spectra,
                      void *y_t, void *state, size_t state_bytes, hipStream_t stream);

/* A prompt of P tokens in one pass (P a multiple of block, 1 <= P <= L), in place of hyena_decode_reset and
 * the steps t = 0..P-1: v, x[i]: [B, D, P] of dtype (channel-major, like hyena_operator's inputs); y: [B, D, P]
 * receives the operator's output on the prompt.  Each order runs the whole-row FFT convolution of its
 * history (the prompt, zero after it) and stores its gated output as the next order's history, so the next
 * call is hyena_decode_step at t = P, which starts a block.  spectra as for hyena_decode_step (no taps
 * needed).  y must not overlap the inputs, the spectra or the state; the inputs and spectra must not overlap
 * the state.  The steps that follow must pass the same `block` as the prefill (the state does not record it:
 * with another block, t = P need not start a block and the step would read prefix contributions the prefill
 * never wrote). */
int hyena_decode_prefill(int order, int64_t B, int64_t D, int64_t L, int64_t block, int64_t P, int dtype, int mode,
                         const void *v, const void *const *x, const void *const *spectra, void *y, void *state,
                         size_t state_bytes, hipStream_t stream);

/* Testing aid: the engine-ordered spectrum as natural-order DFT bins of the filter, complex64:
 * causal H[D, L+1] (bins of the 2L-point transform of the zero-padded taps), periodic H[D, L/2+1]
 * (bins of the L-point transform of the taps), 3-D H[D, 2nx, 2ny, nz+1] (zero-padded) or
 * H[D, nx, ny, nz/2+1] (periodic). */
int hyena_spectrum_export(hyena_dims dims, int mode, int64_t D, const void *spectrum, void *H,
                          hipStream_t stream);

/* Uploads the library's constant tables to the current device (once per device; later calls return at
 * once).  Optional: every other entry point does it on its first call on a device.  Call it before
 * capturing library calls into a HIP graph, or to keep the first call free of the blocking upload. */
int hyena_init(void);

/* Static description of a status code. */
const char *hyena_status_str(int status);

/* Library version as major*10000 + minor*100 + patch. */
int hyena_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HYENA_H_ */
