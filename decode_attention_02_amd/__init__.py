"""GQLA decode attention for AMD Instinct MI355X (gfx950).

The computation lives in libgqla.so (hand-written HIP kernels behind a C ABI declared in
include/gqla.h); this package is its thin Python binding. Importing it fails loudly when
the library has not been built.
"""
from ._lib import (  # noqa: F401
    EXPORTED, GQLA_BF16, GQLA_F32, GQLA_PATH_ABSORB, GQLA_PATH_GQA, Dims, GqlaError, Paged,
    gqla_absorb_query, gqla_append_tokens, gqla_cache_bytes_per_token, gqla_decode_absorb,
    gqla_decode_absorb_noalloc, gqla_decode_absorb_out, gqla_decode_gqa, NOALLOC_SCRATCH_BYTES,
    gqla_expand_cache, gqla_fold_out_weight, gqla_num_splits, gqla_out_hidden, gqla_out_proj, gqla_pick_path,
    gqla_stream_read, gqla_validate_paged, gqla_version,
    gqla_workspace_bytes, LIB, LIB_PATH,
)
