"""MI355X (gfx950) fused wavelet-convolution (WTConv) layer: forward, input
gradient and parameter gradients as hand-written HIP kernels behind a C ABI
(include/wtconv.h, libwtconv.so).  This package holds the kernels (csrc/), their
build step (build.py) and the Python binding (wtconv.py)."""
from .wtconv import (  # noqa: F401
    BF16, F16, F32, MAX_LEVELS, OP_BACKWARD_INPUT, OP_BACKWARD_WEIGHT, OP_FORWARD, STATIC_SCRATCH_BYTES, Desc,
    WTConvError, library, make_desc, profile_begin, profile_end, wtconv_backward_input, wtconv_backward_weight,
    wtconv_backward_weight_noalloc, wtconv_forward, wtconv_plan_launches, wtconv_workspace_size,
)
