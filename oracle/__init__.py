"""CPU oracle of the heterogeneous KV decode path (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The GPU path never imports it, and it shares no code with the
GPU path (the seeded input generator in `synth` serves both sides and holds
none of the method's arithmetic).

See oracle/cache.py for what is computed and which passage each step follows.
"""

from .cache import (  # noqa: F401
    BLOCK, C4_PER_BLOCK, M_CSA, M_HCA, N_HEADS, HEAD_DIM, IDX_HEADS, IDX_DIM,
    OracleError, Oracle, bf16_round, gated_pool, token_scores, c4_scores,
    select_topk, attention, length_split, block_range_summary, decode_reference,
    E4M3_MAX, e4m3_decode, e4m3_encode, quantize_e4m3_rows,
    MX_BLOCK, e2m1_decode, e2m1_encode, quantize_mxfp4_rows,
)
