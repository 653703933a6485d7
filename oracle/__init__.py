"""fp64 CPU oracle for the exact BoB of softmax attention (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this
package. The product path never imports it.
"""

from .bob_oracle import *  # noqa: F401,F403
from .bob_oracle import __all__  # noqa: F401
