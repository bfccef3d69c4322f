"""MI355X (gfx950) routed mixture-of-experts FFN layer on GGUF Q8_0 / Q4_0
expert weights.  The layer runs in hand-written HIP kernels behind the C ABI
of include/fwmoe.h (libfwmoe.so); `fwmoe` is its Python binding."""
from . import fwmoe  # noqa: F401
from .fwmoe import *  # noqa: F401,F403
