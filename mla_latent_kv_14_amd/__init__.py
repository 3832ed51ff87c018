"""MI355X (gfx950) absorbed MLA decode over a paged latent KV cache.

The compute path is libmla_decode.so (hand-written HIP kernels behind a C ABI, see
include/mla_decode.h); this package is its thin Python binding.
"""
from .binding import (NOALLOC_SCRATCH_BYTES, AppendDims, Dims, MlaError, STATUS, cache_append,
                      decode, decode_out, gather_pages, header_symbols, lib, make_dims,
                      workspace_bytes)

__all__ = ["NOALLOC_SCRATCH_BYTES", "AppendDims", "Dims", "MlaError", "STATUS", "cache_append", "decode", "decode_out",
           "gather_pages",
           "header_symbols", "lib", "make_dims", "workspace_bytes"]
