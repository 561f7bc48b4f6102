"""MI355X-native Adasum gradient combiner.

The combine runs in the gfx950 HIP library ``libadasum.so`` (C ABI declared
in include/adasum.h); this package is its thin Python binding.  Importing it
loads the library and fails loudly when the library has not been built.
"""

from ._native import AdasumError, lib as _lib  # noqa: F401
from .combine import Combiner, combine, combine_cached, plain_sum, workspace_bytes  # noqa: F401

_lib()  # fail at import time when the HIP library is missing
