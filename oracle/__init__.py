"""CPU oracles of the ARL2 layer's forward hot path and its backward, and of the retained softmax layer.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  The product library never does.
"""
from .arl2_oracle import (  # noqa: F401
    Arl2Oracle,
    delta_write,
    feature_map,
    gate_projections,
    inter_read,
    softmax_attention,
    unit_rows,
)
from .softmax_oracle import SoftmaxOracle, cached_attention  # noqa: F401,E402
from .stack_oracle import StackOracle, linear, linear_parts, to_bf16  # noqa: F401,E402
from .seq_oracle import Arl2SeqOracle, sequential_frame, sequential_frame_chunked  # noqa: F401,E402
from .bwd_oracle import (  # noqa: F401,E402
    layer_backward,
    pass_backward,
    softmax_attention_bwd,
    write_backward,
)
