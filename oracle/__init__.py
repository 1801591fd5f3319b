"""CPU oracle for chunked linear attention -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark may import
this package.  The product path (``chunked_scan_amd``) never imports it, and this package
never imports the product: the two share nothing but the seeded input generators, which hold
none of the method's arithmetic.

The arithmetic lives in ``la_oracle.c`` (plain C, IEEE double, one token at a time); this
module only builds it with gcc, loads it with ctypes and marshals numpy arrays.  See the C
file's header for the definition it follows and the passages of the ZeCO review page it
cites.
"""
from .oracle import (  # noqa: F401
    NONE, HEAD, GATE, build, lib_path, recurrence, recurrence_bwd, cumdecay, state_scan, state_correct,
    default_threads,
)
