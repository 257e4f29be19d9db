"""MI355X (gfx950) DMS attention: paged cache with delayed eviction, split-K
decode attention over the retained entries, masked prefill.

The compute lives in libdms.so (HIP kernels behind the C ABI of include/dms.h);
this package only binds it and owns device memory through PyTorch.
"""

from . import lib  # noqa: F401
from .cache import DmsCache, prefill  # noqa: F401

__all__ = ["lib", "DmsCache", "prefill"]
