"""Layer-streamed LoRA training on AMD MI355X (gfx950).

The HIP library ``liblsl.so`` (C ABI in include/lsl.h) does all the compute;
this package marshals torch tensors into it and drives the layer sweep.
"""
from .ops import *  # noqa: F401,F403
from .ops import lib, LslError  # noqa: F401
from . import _abi  # noqa: F401
