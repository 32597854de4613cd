"""CPU oracle for one MoE FFN layer: the forward pass and the routed experts' backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding, the timed part of the benchmark) may import or call this
package.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code, constants or helpers with the HIP implementation.
"""

from .moe_oracle import *  # noqa: F401,F403
