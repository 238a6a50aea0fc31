"""Float64 CPU oracle for causal linear attention (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  It imports nothing from the HIP library.
"""
from .linattn_oracle import (  # noqa: F401
    ELU1,
    MAPS,
    TAYLOR2,
    TAYLOR2_SYM,
    attention_gated_quadratic,
    attention_gated_recurrent,
    attention_gated_rows,
    attention_quadratic,
    attention_recurrent,
    attention_rows,
    decay_matrix,
    decode_step,
    feature_dim,
    feature_map,
    final_state,
    gated_decode_step,
    gated_final_state,
    kernel_value,
    phi_elu1,
    phi_taylor2,
    phi_taylor2_sym,
    swa_attention,
    swa_cache_after_prefill,
    swa_decode_step,
    swa_rows,
    sym_pairs,
)
