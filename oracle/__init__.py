"""CPU oracle for the per-expert mixed-precision MoE expert layer (PagedWeight).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this package. The GPU library never imports, links or
calls it, and it shares no code with the library: the only common dependency
is the seeded input generator in ``synth``.

Plain, slow and written to be checked by eye against the pages. The
reference of the GPU parity tests is the plain C++ oracle:

* ``c_oracle`` ``cpu_oracle.cpp`` (Eq. 2's scale, codes, pages and loss;
             Eq. 1's allocation; the router and the float64 forward pass)
             through ctypes; built with g++ on first use.

A second oracle, written separately in float64 PyTorch, agrees with it and
covers the rest:

* ``quant``  Eq. 2 of the PagedWeight page (section "Implementation Details"):
             per-expert scale, codes, the page byte layout, the loss table.
* ``alloc``  Eq. 1 of the PagedWeight page (section "Quality-Aware
             Quantization"): brute force and an exact dynamic programme.
* ``moe``    the forward pass of section "Dynamic Paging": top-k router,
             SwiGLU experts on dequantized weights, weighted combine.
* ``sched``  the KV-pressure budget scheduler (section "Implementation
             Details", memory management): occupancy -> budget with
             hysteresis.
* ``swap``   the host tier of section "Dynamic Paging": which expert pages
             a device cache of page slots holds, pass by pass.
* ``bitplane`` the PagedMoE page's prefix-compatible bitplane layout (its
             Abstract), read as a tree codebook over Eq. 2's 8-bit codes:
             depth-b weights, pages of b bitplanes, the loss table.

All floating-point arithmetic is float64 except where a rounding step is part
of the definition (the fp32 scale, the bf16 activations).
"""
from . import quant, alloc, moe, sched, swap, bitplane  # noqa: F401
