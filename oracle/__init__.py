"""CPU oracle for ragged per-row top-K.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The HIP library never calls it
and shares no code with it.

Every function cites the passage it follows.  The pages (vLLM
``persistent_topk``; PR #54110 excerpt: ``top_k_per_row_decode(logits, next_n,
lengths, output, ...)``; PR #41189 excerpt: ``FilteredTopKRaggedTransform<float,
int32_t, TopK>``) name the op and its tensors but not the tie rule, the output
order or the padding; the readings used are stated in ``oracle_topk.cpp`` and
``topk_ragged_oracle`` below.
"""

from .oracle import (  # noqa: F401
    load_library,
    topk_ragged_bf16_oracle,
    widen_bf16,
    topk_ragged_offsets_oracle,
    topk_ragged_oracle,
    topk_ragged_strided_oracle,
    topk_ragged_values_oracle,
)
