"""MI355X-native chain-and-schedule step of DSpark confidence-scheduled verification.

The hot path lives in the HIP library ``libdspark.so`` (kernels for gfx950 behind a
C ABI declared in ``include/dspark.h``); ``binding`` marshals arguments to it.
``inputs`` holds the seeded synthetic workloads.  Importing the package does not
load the library; ``binding.lib()`` does, and raises if it is missing.
"""
__all__ = ["inputs", "binding"]
