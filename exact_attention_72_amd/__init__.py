"""MI355X-native fused exact-attention forward (gfx950 HIP kernels behind a C ABI).

The entry points mirror include/fa.h: fa_fwd, fa_fwd_varlen,
fa_fwd_kvcache_paged, fa_combine (plus helpers).  The shared library is loaded
on first use and must have been built (exact_attention_72_amd._build.build()).
"""
from .api import (FaError, fa_combine, fa_fwd, fa_fwd_kvcache_paged, fa_fwd_varlen,  # noqa: F401
                  fa_kvcache_workspace_size, fa_last_error, fa_tile_class, fa_version)
