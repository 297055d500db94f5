"""KIVI KV-cache quantization hot path for MI355X (gfx950).

The arithmetic lives in the HIP library ``libkivi.so`` (C ABI in
``include/kivi.h``); ``kivi`` is its Python binding and ``synth`` draws the
seeded synthetic inputs.
"""
from . import kivi  # noqa: F401
from .kivi import (KIVI_KEYS, KIVI_VALUES, KiviError, Store, decode_attend,  # noqa: F401
                   dequantize, quantize_keys, quantize_values)
