"""MI355X-native per-expert mixed-precision MoE expert layer (PagedWeight).

The compute path is libpagedweight.so (HIP kernels for gfx950 behind the C
ABI in include/pagedweight.h); this package only binds it.
"""
from .pagedweight import (BITS, BUDGET_GROW, BUDGET_INIT, BUDGET_KEEP, BUDGET_SHRINK,  # noqa: F401
                          PagedMoELayer, PagedWeightError, budget_decide, lib, library_path,
                          proportional_bits, set_budget_layers, solve_allocation,
                          solve_allocation_layers)
