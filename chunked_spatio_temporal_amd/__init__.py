"""MI355X-native chunked spatio-temporal attention (DualParal queue step).

The compute lives in a C-ABI shared library of hand-written gfx950 HIP kernels
(``lib/libchunkattn.so``, interface in ``include/chunkattn.h``).  The Python
layer only marshals arguments:

* ``chunked_spatio_temporal_amd.chunkattn`` -- ctypes binding with the
  library's entry-point names (``queue_step``, ``full``, ...).
* ``chunked_spatio_temporal_amd.synth`` -- seeded synthetic inputs.
* ``chunked_spatio_temporal_amd.configs`` -- the workload shapes.

Importing this package does not load the library; the binding loads it on
first use and raises if it is missing.
"""
__all__ = ["chunkattn", "synth", "configs"]
