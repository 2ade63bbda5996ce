"""MI355X (gfx950) MoE-layer hot path: sigmoid noaux_tc router, batch-union dispatch, packed-int4 SwiGLU experts
on Q8_0 int8 activations, weighted combine; optional per-layer LRU expert cache over pinned host memory.

The work runs in libmoe.so (include/moe.h); this package is its ctypes binding."""
from ._lib import *  # noqa: F401,F403
from ._lib import Config, MoeError, EXPORTED, LIB_PATH  # noqa: F401
