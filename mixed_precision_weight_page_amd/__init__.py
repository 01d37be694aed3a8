"""MI355X-native per-expert mixed-precision MoE expert layer (PagedWeight).

The compute path is libpagedweight.so (HIP kernels for gfx950 behind the C
ABI in include/pagedweight.h); this package only binds it.
"""
from .pagedweight import (BITS, PagedMoELayer, PagedWeightError, lib, library_path,  # noqa: F401
                          solve_allocation)
