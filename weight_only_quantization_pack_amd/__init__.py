"""AWQ W4A16 g128 hot path for MI355X (gfx950).

The compute lives in the HIP library ``libawq.so`` (C ABI declared in
``include/awq.h``); this package is a thin ctypes binding over it plus the
seeded synthetic workloads.  The library is loaded on first use and a
missing build raises immediately: there is no CPU fallback.
"""
from .binding import (AwqError, quantize_pack, search_scale, search_scale_shared,  # noqa: F401
                      search_scale_mlp, search_mlp_workspace_bytes,
                      search_workspace_bytes,
                      gemv, gemv_gate_up, gemm, gemm_splitk_workspace_bytes, scale_activations,
                      gemm_splitk_noalloc, gemm_splitk_noalloc_max_bytes,
                      fake_quantize,
                      library_path,
                      load_library,
                      pack_format_version, packed_words_per_row, packed_words)

__all__ = ["AwqError", "quantize_pack", "search_scale", "search_scale_shared", "search_workspace_bytes",
           "search_scale_mlp", "search_mlp_workspace_bytes",
           "gemv", "gemv_gate_up", "gemm", "gemm_splitk_workspace_bytes",
           "gemm_splitk_noalloc", "gemm_splitk_noalloc_max_bytes", "scale_activations", "fake_quantize", "library_path", "load_library",
           "pack_format_version", "packed_words_per_row", "packed_words"]
