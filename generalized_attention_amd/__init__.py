"""MI355X (gfx950) generalized dot-product attention (GDPA).

The computation lives in ``libgdpa.so`` (hand-written HIP kernels behind the C ABI of
``include/gdpa.h``). This package is its thin Python front end: ``_lib`` mirrors the C
structures and entry points; ``ops`` marshals torch device tensors into them (torch provides
device memory and the current stream; it computes nothing of the operator).
"""

from . import _lib  # noqa: F401
from .ops import (  # noqa: F401
    GroupArgs,
    device_error,
    gdpa_bwd,
    gdpa_bwd_grouped,
    gdpa_fwd,
    gdpa_fwd_grouped,
    gdpa_plan,
    make_group,
    workspace,
)
