"""MI355X-native ragged per-row top-K (gfx950 HIP kernels behind a C ABI).

``topk_ragged`` returns, for every row of an fp32 score matrix, the int32
indices of the K largest scores among the first ``lengths[row]`` entries --
ties to the lower index, ascending order, -1 padding.  The work runs in the
HIP library ``lib/libtopk_ragged.so``; this package only marshals arguments.
"""

from .binding import (  # noqa: F401
    MAX_K,
    NOALLOC_SCRATCH_BYTES,
    RADIX_THRESHOLD,
    PATH_MULTI,
    PATH_NONE,
    PATH_SINGLE,
    TopKError,
    debug_keys,
    last_error,
    new_workspace,
    plan_for_props,
    query_plan,
    read_reference,
    strided_workspace_size,
    topk_ragged,
    topk_ragged_bf16,
    topk_ragged_noalloc,
    topk_ragged_strided,
    topk_ragged_values,
    workspace_init,
    workspace_size,
    workspace_status,
)
