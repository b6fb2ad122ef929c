"""MI355X-native ART (Attention Run-time Termination) decode attention.

The compute path is libart.so (HIP kernels for gfx950 behind the C ABI in
include/art.h); this package holds its sources, its build script and a thin
ctypes binding.
"""
from . import art  # noqa: F401
from .art import (ART_DT_BF16, ART_DT_F32, ART_FLAG_DETECT_ONLY, ART_FLAG_NO_DIR, ART_FLAG_NO_SCALE,  # noqa: F401
                  ART_MODE_ART, ART_MODE_FULL, ART_ORDER_GIVEN, ART_ORDER_NATURAL, ART_ORDER_RECENT_FIRST,
                  ART_SELECT_ASCENDING, ART_SELECT_IMPORTANCE, ArtDecoder, ArtError, DecodeResult)
