"""CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  It shares no code with the
HIP library or its binding.
"""
from .basa_oracle import (  # noqa: F401
    SCHED_ALTERNATE, SCHED_FOUR_PHASE, SCHED_NONE, dense_flops, full_attention,
    masked_attention_bruteforce, mem_tokens, pool_mean, shift_for_block,
    theoretical_speedup, window_attention, window_attention_head, window_flops,
    window_id, window_token_index)
from .basa_backward import (  # noqa: F401
    attention_backward_rows, pool_backward, window_attention_backward,
    window_attention_backward_head)
from .basa_curve import (  # noqa: F401
    center_region, curve_attention, curve_attention_bruteforce, hilbert_curve_xy,
    hilbert_order)
