"""Decode attention over a mixed-precision (INT2 / INT4 / FP16) paged KV cache on MI355X.

The computation lives in libkvq.so (hand-written HIP for gfx950 plus host C++);
`kvq` is the ctypes binding with the same names as the C ABI in include/kvq.h."""
from . import kvq  # noqa: F401  (raises ImportError when libkvq.so is not built)
