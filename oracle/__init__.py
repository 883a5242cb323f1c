"""CPU oracle for sparse latent attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never import it, and it imports nothing from them.

Pinning status: every public function is pinned by the CPU tests
(tests/test_oracle_pins.py) to invariants, closed forms and library routines
independent of this code; none is "parity unpinned".
"""
from .mla_oracle import (  # noqa: F401
    D_LATENT,
    D_MODEL,
    D_NOPE,
    D_QK,
    D_ROPE,
    D_V,
    FP8_BLOCK,
    N_HEADS,
    SOFTMAX_SCALE,
    absorbed_scores,
    attend_explicit,
    attend_explicit_gather,
    cache_append,
    decode,
    decode_absorbed,
    explicit_scores,
    fp8_block_dequant,
    fp8_e4m3_decode,
    index_mask,
    join_keys,
    join_query,
    mix_values,
    output_projection,
    prefill,
    rms_norm,
    rotate_pairs,
    scores,
    selected_rows,
    softmax_rows,
    stack_wkv_b,
    to_f64,
    up_project,
    wkv_b_dequant,
)
