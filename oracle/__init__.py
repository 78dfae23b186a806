"""CPU oracle for the Looped CollectiveEinsum and the fused reduce epilogue.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import anything from this package.  The
product path (the HIP library and its Python binding) never calls it, and this
package never imports the product path: the two share no code.

Sources, cited by page title and section throughout:

* [OV]  Wang et al., "Overlap Communication with Dependent Computation via
        Decomposition in Large Deep Learning Models", ASPLOS'23 -- the loop,
        the shard movement and the update rules (its Sections 2.1, 4, 5.1,
        5.4.1).
* [CC]  Jangda et al., "Breaking the Computation and Communication Abstraction
        Barrier in Distributed Machine Learning Workloads" (CoCoNet),
        ASPLOS'22 -- the order of the fused epilogue (its Figure 3 program and
        the FusedAllReduce description).
* [SMDS] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
        1, 2, 3", SC'11 -- the Philox4x32-10 bijection used for the dropout
        mask (the pages name no generator).

Everything is plain NumPy in float64 (inputs that the device holds in bf16 are
upcast exactly).  Nothing here is blocked, fused or reordered beyond what the
definitions state.

Parity status per function is listed in each module's header.
"""

from . import ring, einsum, numerics, philox, epilogue  # noqa: F401
