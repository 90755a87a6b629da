"""kvsel: attention-score-based KV-cache selection for AMD MI355X (gfx950).

The compute lives in libkvsel.so (hand-written HIP kernels behind the C ABI
in include/kvsel.h); this package only builds and binds it.
"""

from .kvsel import (  # noqa: F401
    KvselError,
    Problem,
    abi_version,
    alloc_outputs,
    bind_compress,
    compress,
    exported_functions,
    kvsel_allocate_budgets,
    kvsel_compress,
    kvsel_compress_noalloc,
    kvsel_gather,
    kvsel_plan,
    kvsel_pool_topk,
    kvsel_profile_layer,
    kvsel_row_stats,
    kvsel_score,
    kvsel_score_from_stats,
    kvsel_tier_rank,
    kvsel_topk_mass,
)
