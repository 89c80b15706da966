"""MI355X (gfx950) implementation of the gated delta rule scan.

The computation lives in libgdn.so (hand-written HIP kernels behind the C ABI
of include/gdn.h); this package holds its Python binding, the build script and
the seeded synthetic-input generator.
"""
from .binding import (GdnError, Shape, conv1d_qkv, conv_state_snapshot, decode_step, gated_rmsnorm,
                      header_functions, library_path, load_library, make_shape, prefill_chunked,
                      prefill_chunked_gated_rmsnorm, prefill_chunked_noalloc, prepare_conv1d_qkv, prepare_decode,
                      prepare_gated_rmsnorm, prepare_prefill, prepare_prefill_gated_rmsnorm, profile_collect,
                      profile_enable, state_snapshot, version, workspace_bytes, workspace_bytes_for)

__all__ = ["GdnError", "Shape", "conv1d_qkv", "conv_state_snapshot", "decode_step", "gated_rmsnorm", "header_functions",
           "library_path", "load_library", "make_shape", "prefill_chunked", "prefill_chunked_gated_rmsnorm", "prefill_chunked_noalloc",
           "prepare_conv1d_qkv", "prepare_decode", "prepare_prefill_gated_rmsnorm",
           "prepare_gated_rmsnorm", "prepare_prefill", "profile_collect", "profile_enable", "state_snapshot", "version",
           "workspace_bytes", "workspace_bytes_for"]
