"""ARL2 hybrid attention layer for AMD Instinct MI355X (gfx950): the forward hot path, its
backward, and the retained softmax attention layer with its K/V cache that an ARL2 model keeps
beside it.

The computation lives in libarl2.so (HIP kernels behind the C interfaces of include/arl2.h,
include/arl2_bwd.h and include/arl2_softmax.h); this package only binds it.
"""
from .arl2 import (  # noqa: F401
    ARL2_BF16,
    ARL2_F32,
    Arl2Backward,
    Arl2Config,
    Arl2Error,
    Arl2Layer,
    LIB_PATH,
    SoftmaxConfig,
    SoftmaxLayer,
    load_library,
    status_string,
)
