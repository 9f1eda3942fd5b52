"""outlier_aware_bit_amd: the outlier-aware quantized linear layer on MI355X.

The compute lives in ``libqlin.so`` (HIP C++ for gfx950, C ABI declared in
``include/qlin.h``); ``qlin`` is its thin PyTorch binding.  Importing the
package loads the library and raises if it has not been built.
"""
from . import _lib

_lib.load()

from .qlin import *  # noqa: E402,F401,F403
from . import qlin  # noqa: E402,F401
