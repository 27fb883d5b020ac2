"""CPU oracle for the tree-verify MLA-absorb attention step (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import this
package; the HIP product path never does.
"""
from .tv_oracle import *  # noqa: F401,F403
from . import tv_oracle  # noqa: F401
