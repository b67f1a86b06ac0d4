"""fp64 CPU oracle for the gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, step-by-step statement
of what the recurrence computes, used to check the HIP path. Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it; the
library itself never calls it and has no CPU fallback.

It shares no code with the HIP path: inputs come from the caller as numpy
arrays, every operation is evaluated in float64, and no value it returns is
ever taken from the GPU.

Pins (tests that fix the oracle to something other than itself) are listed in
each function's docstring. Parity unpinned: nothing — every public function has
at least one pin; the float64 handling of products below about 1e-300
(underflow) is the only behaviour no pin covers.
"""
from .recurrence import (  # noqa: F401
    VARIANTS,
    erase_write_vectors,
    step,
    decode_step,
    step_recurrence,
    transition_matrix,
    rel_err,
)
from .chunked import chunked_reference  # noqa: F401
from . import states  # noqa: F401
from . import prep  # noqa: F401
from . import backward  # noqa: F401
from . import product  # noqa: F401
