"""MI355X (gfx950) single-token decode attention for hybrid sliding/global stacks.

The computation lives in libgemma_attn.so (HIP kernels behind the C ABI declared in
include/gemma_attn.h); this package is its Python binding plus the workload
geometries, the per-layer-type caches and the seeded synthetic inputs.  Importing the
package does not load the library; the first call does, and fails loudly if it has not
been built.
"""
from .api import (IMPL_AUTO, IMPL_MFMA, IMPL_VALU, LINEAR, RING, GemmaAttnError, debug_ranges,
                  decode, decode_append, decode_rope_append, kv_append, make_opts, make_shape,
                  rope_append, rope_table, validate, version, workspace_bytes)

__all__ = ["IMPL_AUTO", "IMPL_MFMA", "IMPL_VALU", "LINEAR", "RING", "GemmaAttnError",
           "debug_ranges", "decode", "decode_append", "decode_rope_append", "kv_append",
           "make_opts", "make_shape", "rope_append", "rope_table", "validate", "version",
           "workspace_bytes"]
