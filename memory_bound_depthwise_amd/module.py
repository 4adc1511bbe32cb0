"""The WTConv layer as a trainable torch layer over the C ABI.

"Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware Reformulation",
§2.1 (Algorithm 1): the layer maps x[B, C, H, W] to a tensor of the same shape,
with a base depthwise kernel W0, bias b and scale s0, and, for each of L levels,
a depthwise kernel on the four Haar bands of every channel, W(l) [C, 4, k, k],
with one scale per (channel, band), s(l) [C, 4].

WTConvFunction is an autograd.Function whose forward is wtconv_forward and whose
backward is wtconv_backward_input (dx) and wtconv_backward_weight (all parameter
gradients, §4.3 Eq. 9).  This file only marshals arguments: every step of the
layer runs in the library's HIP kernels, and tensors that are not on the GPU are
refused by the binding (there is no CPU path).
"""
from __future__ import annotations

import math

import torch

from . import wtconv as _w


class WTConvFunction(torch.autograd.Function):
    """y = WTConv(x; w0, b0, s0, wl, sl) with `levels` Haar levels.

    x: [n, C, H, W] float32 or bfloat16, contiguous, on the GPU.  Parameters are
    float32: w0 [C, k, k], b0 [C] or None, s0 [C], wl [L, C, 4, k, k], sl [L, C, 4]
    (wl and sl may be None when levels == 0).  The backward recomputes what it needs
    from x and dy; nothing but the inputs is kept between the passes."""

    @staticmethod
    def forward(ctx, x, w0, b0, s0, wl, sl, levels: int):
        x = x.contiguous()
        y = _w.wtconv_forward(x, w0, b0, s0, wl, sl, levels)
        ctx.levels = levels
        ctx.save_for_backward(x, w0, b0, s0, wl, sl)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w0, b0, s0, wl, sl = ctx.saved_tensors
        L = ctx.levels
        dy = dy.to(x.dtype).contiguous()
        need = ctx.needs_input_grad
        dx = _w.wtconv_backward_input(dy, w0, s0, wl, sl, L) if need[0] else None
        dw0 = db0 = ds0 = dwl = dsl = None
        if any(need[1:6]):
            g = _w.wtconv_backward_weight(x, dy, w0, b0, s0, wl, sl, L)
            dw0, db0, ds0 = g["dw0"], g["db0"], g["ds0"]
            if L > 0:
                dwl, dsl = g["dwl"], g["dsl"]
        return (dx, dw0 if need[1] else None, db0 if need[2] else None, ds0 if need[3] else None,
                dwl if need[4] else None, dsl if need[5] else None, None)


def wtconv(x, w0, b0, s0, wl, sl, levels: int):
    """Functional form of the layer (differentiable in x and every parameter)."""
    return WTConvFunction.apply(x, w0, b0, s0, wl, sl, levels)


class WTConv2d(torch.nn.Module):
    """Depthwise wavelet convolution: channels in = channels out, odd kernel size k
    (3, 5 or 7), 0 <= levels <= 8.

    Initialisation (the pages give none): every kernel as torch's default for a
    depthwise conv (uniform in +-1/k, i.e. +-1/sqrt(fan_in)), bias zero, every scale
    one."""

    def __init__(self, channels: int, kernel_size: int = 5, levels: int = 1, bias: bool = True,
                 device=None):
        super().__init__()
        if kernel_size % 2 != 1:
            raise ValueError("kernel_size must be odd")
        if not 0 <= levels <= _w.MAX_LEVELS:
            raise ValueError(f"levels must be in [0, {_w.MAX_LEVELS}]")
        C, k, L = channels, kernel_size, levels
        f32 = dict(dtype=torch.float32, device=device)
        self.channels, self.kernel_size, self.levels = C, k, L
        bound = 1.0 / math.sqrt(k * k)
        self.weight = torch.nn.Parameter(torch.empty((C, k, k), **f32).uniform_(-bound, bound))
        self.bias = torch.nn.Parameter(torch.zeros((C,), **f32)) if bias else None
        self.scale = torch.nn.Parameter(torch.ones((C,), **f32))
        if L > 0:
            self.level_weight = torch.nn.Parameter(torch.empty((L, C, 4, k, k), **f32).uniform_(-bound, bound))
            self.level_scale = torch.nn.Parameter(torch.ones((L, C, 4), **f32))
        else:
            self.register_parameter("level_weight", None)
            self.register_parameter("level_scale", None)

    def forward(self, x):
        return wtconv(x, self.weight, self.bias, self.scale, self.level_weight, self.level_scale, self.levels)

    def extra_repr(self) -> str:
        return (f"channels={self.channels}, kernel_size={self.kernel_size}, levels={self.levels}, "
                f"bias={self.bias is not None}")
