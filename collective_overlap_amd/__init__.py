"""Looped CollectiveEinsum with a fused reduce epilogue, native to MI355X.

The compute path is libcce.so (hand-written gfx950 HIP kernels behind a C
ABI, include/cce.h); this package is its thin ctypes binding.  Importing the
package does not load the library; the first call does, and fails loudly if
the library has not been built.
"""

from .api import *  # noqa: F401,F403
from .api import __all__  # noqa: F401
