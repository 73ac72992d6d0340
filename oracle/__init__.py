"""CPU float64 oracle for exact attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package. The product (the HIP library and its Python
binding) never does.
"""
from .attention import (attention, attention_head, decode, decode_paged, merge,  # noqa: F401
                        online_softmax_rows, part_state)
from .backward import attention_backward, attention_backward_head  # noqa: F401
from .fp8 import attention_fp8, attention_fp8_head, e4m3_decode, e4m3_round  # noqa: F401
