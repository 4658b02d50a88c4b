"""CPU oracle for UPipe causal GQA attention (test infrastructure only).

This package is the checker, not the product. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. It shares no code with the HIP path and never imports it.
"""

from .attention import (  # noqa: F401
    attention_forward,
    attention_backward,
    forward_rows,
    backward_rows_dq,
    rows_forward_dq,
    backward_cols_dkdv,
    cols_rows_needed,
    kv_head_of,
)
from .block import attention_block_forward, attention_block_rows, round_bf16  # noqa: F401,E402
from .loss import cross_entropy  # noqa: F401,E402
from .mlp import swiglu_mlp  # noqa: F401,E402
