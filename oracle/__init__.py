"""CPU oracle for verification attention over a paged KV cache and for the
write of the drafts' keys and values into that cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this package: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (no kernels, headers, helpers or tables); the two meet only at the
seeded inputs drawn by ``workloads``.

Every function here is pinned by CPU tests against facts that do not come
from this code: worked tiny cases written as closed forms, library routines
(``torch.nn.functional.scaled_dot_product_attention`` in float64,
``torch.logsumexp``, torch's float8/bfloat16 casts and float32 division) and the invariants the
pages state (chain mask = causal, paged = contiguous, GQA = expanded heads,
single-query decode, split invariance, additive -inf/-5e4 masks).
"""

from .verify_attention import (  # noqa: F401
    E4M3FN_TABLE,
    decode_bf16,
    decode_e4m3fn,
    decode_storage,
    request_lengths,
    gather_request_kv,
    allowed_keys,
    attend_rows,
    verify_attention,
    verify_attention_partials,
    merge_partials,
    unpack_mask_block,
    unpack_mask_rows,
    mask_block_of,
)
from .append_kv import (  # noqa: F401
    append_kv,
    quantise,
    round_to_bf16,
    round_to_e4m3fn_sat,
    round_to_f32,
    source_values,
)
from .rope import rotate as rope_rotate, rotate_f32 as rope_rotate_f32  # noqa: F401
