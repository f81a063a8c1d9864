"""fp64 CPU oracle for absorbed-MQA MLA decode and LSE merge (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import it.
"""
from .mla_oracle import (  # noqa: F401
    LATENT_DIM, ROPE_DIM, QK_DIM, PAGE_SIZE,
    bf16_bits_to_f64, e4m3_bits_to_f64, gather_request_rows, visible_lengths,
    attend_rows, decode_partial_ref, merge_ref, dcp_shard_len, dcp_shard_positions,
    absorb_query, mha_unabsorbed_ref,
    query_prep_ref, bf16_encode, e4m3_encode, E4M3_MAX, query_prep_codes,
    up_project_ref, gather_cache_ref, merge_two_ref,
)
