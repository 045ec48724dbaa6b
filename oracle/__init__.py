"""CPU oracle for the DASH prefill path — test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  It shares no code with the HIP
library or its binding.
"""
from .dash_oracle import (  # noqa: F401
    causal_gqa_attention, output_projection, delta_attn, attention_layer,
    topk_count, select_topk, effective_keep_count, select_topk_forced,
    order_statistic, percentile_rank, threshold_step,
    compact, attn_active, decode_step, run_one_shot, run_multi_shot, run_threshold,
)
