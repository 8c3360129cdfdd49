"""MI355X-native ONNX MatMul: a plan/execute C-ABI library with HIP kernels
for gfx950, and a thin ctypes binding.

Importing the package does not load the native library; the binding loads
``libmm.so`` on first use and raises if it is missing.
"""
from .synth import BFLOAT16, FLOAT, FLOAT16  # noqa: F401

__all__ = ["FLOAT", "FLOAT16", "BFLOAT16"]
