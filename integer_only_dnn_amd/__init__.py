"""Integer-only (C, e) layer step for MI355X (gfx950).

The compute path is the HIP library libie.so (C ABI in include/ie.h); the
binding in ``integer_only_dnn_amd.ie`` only marshals arguments.
"""

from . import ie  # noqa: F401
from .ie import (  # noqa: F401
    ROW, TENSOR, IeError, Mat, Workspace, conv_desc, ie_conv_bwd, ie_conv_fwd, ie_linear_bwd_dw,
    ie_linear_bwd_dx, ie_linear_fwd, ie_sgd_update,
)
