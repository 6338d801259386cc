"""CPU oracle for the ReAttention hot path -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The GPU library neither imports nor links anything from here.
All functions carry a parity pin in tests/test_oracle_pins.py.
"""
from .rea_oracle import (  # noqa: F401
    regions, span_list, token_scores, span_scores_from_tokens, exact_span_score,
    select_topk, window_src, rope, attend_rows, score_select, gather_rope,
    window_attend, step,
)
