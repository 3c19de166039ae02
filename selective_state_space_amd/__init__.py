"""MI355X (gfx950) Mamba-2 SSD layer scan: HIP kernels behind a C ABI.

The computation lives in ``libssd.so`` (``csrc/``, declared in
``include/ssd.h``); :mod:`selective_state_space_amd.ssd` is its ctypes
binding and :mod:`selective_state_space_amd.inputs` the seeded synthetic input
generator.  Importing the package loads nothing; the binding loads the
library on first use and raises if it is not built.
"""

__all__ = ["ssd", "inputs", "build"]
