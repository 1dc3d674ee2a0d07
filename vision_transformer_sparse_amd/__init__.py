"""MI355X (gfx950) Bi-Level Routing Attention forward pass.

The computation lives in libbra.so (C ABI: include/bra.h), built from the HIP
sources in csrc/ by `python -m vision_transformer_sparse_amd.build`; `bra` is
its Python binding.
"""
from . import bra  # noqa: F401
from .bra import forward, region_means, route, attend, lce  # noqa: F401
