"""MI355X (gfx950) Hyena operator: hand-written HIP FFT long-convolution kernels behind a C ABI
(include/hyena.h, libhyena.so) with a thin ctypes binding.

    from attention_free_long_implicit_amd import filter_gen, fftconv, operator
"""
from ._lib import (BF16, CAUSAL, CIRCULAR, F32, LINEAR, PER_SAMPLE, HyenaError, declared_symbols,  # noqa: F401
                   decode_prefill, decode_reset, decode_state_bytes, decode_step, fftconv, film_filter_gen,
                   film_filter_workspace_bytes, filter_gen, filter_workspace_bytes, lib, operator, operator_noalloc,
                   projection, SpectrumCache, default_spectrum_cache, hyena,
                   spectrum_bytes, spectrum_export, status_str, workspace_bytes)

__all__ = ["filter_gen", "fftconv", "operator", "spectrum_bytes", "workspace_bytes", "filter_workspace_bytes",
           "spectrum_export", "HyenaError", "lib", "declared_symbols", "F32", "BF16", "CAUSAL", "LINEAR",
           "CIRCULAR", "status_str", "film_filter_gen", "film_filter_workspace_bytes", "PER_SAMPLE", "projection",
           "decode_state_bytes", "decode_reset", "decode_step", "decode_prefill", "operator_noalloc", "SpectrumCache",
           "default_spectrum_cache", "hyena"]
