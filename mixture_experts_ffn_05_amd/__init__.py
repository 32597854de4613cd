"""libmoe: forward pass of one MoE FFN layer as hand-written CDNA4 (gfx950) HIP kernels.

The compute lives in the C-ABI shared library ``libmoe.so`` (sources under
``csrc/``, declarations in ``include/libmoe.h``).  ``binding`` marshals torch
tensors into that library's calls; ``workloads`` draws the seeded synthetic
inputs.  Importing the package loads nothing; ``binding.load()`` loads the
library and fails loudly if it is missing.
"""

__version__ = "0.1.0"
