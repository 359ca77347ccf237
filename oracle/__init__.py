"""CPU oracle of the ARL2 layer's forward hot path.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  The product library never does.
"""
from .arl2_oracle import (  # noqa: F401
    Arl2Oracle,
    delta_write,
    feature_map,
    inter_read,
    softmax_attention,
    unit_rows,
)
