"""ARL2 hybrid attention layer (forward hot path) for AMD Instinct MI355X (gfx950).

The computation lives in libarl2.so (HIP kernels behind the C interface of include/arl2.h);
this package only binds it.
"""
from .arl2 import (  # noqa: F401
    ARL2_BF16,
    ARL2_F32,
    Arl2Config,
    Arl2Error,
    Arl2Layer,
    LIB_PATH,
    load_library,
    status_string,
)
