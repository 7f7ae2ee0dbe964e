"""Plain CPU oracle for the swizzled tile-movement path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
Python binding) may import, call, link or execute anything in this package.
Its only users are the test suite, the smoke check and the CPU-baseline leg
of the benchmark.  It shares no code, tables or constants with the GPU path;
the only module both sides use is the seeded input generator in
``workloads``, which holds none of the method's arithmetic.

Every function cites the passage of the source pages it follows, by page
title and section.  The four pages are:

* "NVIDIA CuTe Swizzle"                    (CUTLASS Python DSL notes)
* "CuTe Swizzle 学习手册"                   (a CuTe swizzle handbook)
* "cutlass 入门"                            (CUTLASS introduction notes)
* "CUDA 013 - Swizzle 的工作原理"            (how swizzling works)
"""

from .swz_oracle import *  # noqa: F401,F403
