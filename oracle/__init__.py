"""Plain fp64 CPU oracle for the mixture draft tree path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package; only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP path.

Parity pins: every function here is pinned by a CPU test against something
other than itself (closed forms, library routines, brute force, properties the
pages fix).  The one part with no pin is the pages' own worked example (the
15-node tree of the "In one minute" animation): its per-mode probabilities are
not printed, so that example is "parity unpinned".
"""

from .mfd_oracle import *  # noqa: F401,F403
