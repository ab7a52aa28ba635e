"""CacheBlend blended prefill on AMD Instinct MI355X (gfx950).

The product is the HIP library ``libcacheblend.so`` (C ABI in
``include/cacheblend.h``); ``api`` is its thin Python binding.  Importing the
package does not load the library; the first call does, and raises if the
library has not been built (there is no fallback path).
"""
from . import _abi  # noqa: F401

__all__ = ["api", "build"]
