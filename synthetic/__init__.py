"""Seeded synthetic inputs for the WTConv layer.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds no part of the layer's arithmetic: it only draws random
numbers and rounds them to the storage dtype.

Generator (counter based, so values depend on nothing but seed, tensor name and
element index, never on a numpy or torch version):

* stream key  = splitmix64_mix(seed XOR fnv1a64(name))
* word i      = splitmix64_mix(key + (i + 1) * 0x9E3779B97F4A7C15)
  where splitmix64_mix is the output function of Steele, Lea and Flood's
  SplitMix64 (xor-shift 30/27/31 with multipliers 0xBF58476D1CE4E5B9 and
  0x94D049BB133111EB).
* uniform u   = (word >> 11) * 2**-53, in [0, 1)
* normal      = Box-Muller on the word pair (2i, 2i+1):
                sqrt(-2 ln(1 - u0)) * cos(2 pi u1)
* fp32 values are the float64 draws rounded to float32; bf16 values are those
  float32 values rounded to nearest even in the top 16 bits.
"""
from __future__ import annotations

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def fnv1a64(name: str) -> int:
    h = 0xCBF29CE484222325
    for byte in name.encode("utf-8"):
        h ^= byte
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def _words(seed: int, name: str, count: int) -> np.ndarray:
    key = _mix(np.array([(seed ^ fnv1a64(name)) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))[0]
    with np.errstate(over="ignore"):
        idx = np.arange(1, count + 1, dtype=np.uint64)
        return _mix(key + idx * _GAMMA)


def uniform(seed: int, name: str, shape, low: float = 0.0, high: float = 1.0) -> np.ndarray:
    """float32 array, U(low, high)."""
    count = int(np.prod(shape, dtype=np.int64))
    u = (_words(seed, name, count) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    return (low + (high - low) * u).astype(np.float32).reshape(shape)


def normal(seed: int, name: str, shape, std: float = 1.0) -> np.ndarray:
    """float32 array, N(0, std**2) (std is the standard deviation)."""
    count = int(np.prod(shape, dtype=np.int64))
    w = _words(seed, name, 2 * count)
    u0 = (w[0::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    u1 = (w[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    z = np.sqrt(-2.0 * np.log1p(-u0)) * np.cos(2.0 * np.pi * u1)
    return (std * z).astype(np.float32).reshape(shape)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bit patterns."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((bits >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    with np.errstate(over="ignore"):
        out = ((bits + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 values that are exactly representable in bfloat16 (RNE)."""
    return bf16_bits_to_f32(to_bf16_bits(a))


def round_to_f16(a: np.ndarray) -> np.ndarray:
    """float32 values that are exactly representable in IEEE half (numpy's
    conversion rounds to nearest, ties to even)."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).astype(np.float32)


# ---------------------------------------------------------------------------
# Layer inputs.  A "case" describes one WTConv layer invocation.
# ---------------------------------------------------------------------------

class Case:
    """One synthetic layer invocation.

    n, c, h, w: activation shape (NCHW); k: odd kernel size; levels: Haar levels;
    dtype: "f32", "bf16" or "f16" (activation storage; parameters are always float32).
    x_std / dy_std: std of the activation and upstream-gradient draws;
    w_std: std of every depthwise kernel; b_std: std of the bias (0 -> zero bias);
    s_low/s_high: scale range.
    """

    def __init__(self, n, c, h, w, k=5, levels=1, dtype="f32", seed=0,
                 x_std=1.0, dy_std=1.0, w_std=0.05, b_std=0.05,
                 s_low=0.5, s_high=1.5, name="case"):
        self.n, self.c, self.h, self.w = int(n), int(c), int(h), int(w)
        self.k, self.levels, self.dtype, self.seed = int(k), int(levels), dtype, int(seed)
        self.x_std, self.dy_std, self.w_std, self.b_std = x_std, dy_std, w_std, b_std
        self.s_low, self.s_high = s_low, s_high
        self.name = name

    @property
    def numel(self) -> int:
        return self.n * self.c * self.h * self.w

    def __repr__(self):
        return (f"Case({self.name}: x[{self.n},{self.c},{self.h},{self.w}] k={self.k} "
                f"L={self.levels} {self.dtype} seed={self.seed})")

    def _act(self, tag, std):
        a = normal(self.seed, f"{self.name}/{tag}", (self.n, self.c, self.h, self.w), std)
        if self.dtype == "bf16":
            return round_to_bf16(a)
        return round_to_f16(a) if self.dtype == "f16" else a

    def x(self) -> np.ndarray:
        """float32 activation values (already representable in the storage dtype)."""
        return self._act("x", self.x_std)

    def dy(self) -> np.ndarray:
        return self._act("dy", self.dy_std)

    def params(self) -> dict:
        c, k, L = self.c, self.k, self.levels
        s = self.seed
        p = {
            "w0": normal(s, f"{self.name}/w0", (c, k, k), self.w_std),
            "s0": uniform(s, f"{self.name}/s0", (c,), self.s_low, self.s_high),
            "wl": normal(s, f"{self.name}/wl", (L, c, 4, k, k), self.w_std),
            "sl": uniform(s, f"{self.name}/sl", (L, c, 4), self.s_low, self.s_high),
        }
        if self.b_std > 0:
            p["b0"] = normal(s, f"{self.name}/b0", (c,), self.b_std)
        else:
            p["b0"] = np.zeros((c,), np.float32)
        return p


def baseline_cases() -> dict:
    """The workloads of the layer study, as seeded synthetic cases (seed 0).

    tiny: x[1,8,16,16] fp32, kernels N(0, 0.1), zero bias, L=2.
    stage1/stage2/stage3: WTConvNeXt-T stage shapes at batch 64 (bf16).
    hires_L1..L5: x[8,128,256,256] bf16 for L = 1..5.
    stack_1..stack_4: the four WTConvNeXt-T stage layers at batch 128 (bf16).
    stage1_f16: the stage1 shape with IEEE half activations.
    dw5, dw7: plain depthwise convolutions (levels = 0) on the stage1 shape, k = 5
    (the wavelet path's own kernel size) and k = 7 (the kernel a WTConv layer
    replaces in ConvNeXt): the two comparison protocols of the paper's §5.
    """
    cases = {
        "tiny": Case(1, 8, 16, 16, 5, 2, "f32", 0, w_std=0.1, b_std=0.0, name="tiny"),
        "stage1": Case(64, 96, 56, 56, 5, 3, "bf16", 0, name="stage1"),
        "stage2": Case(64, 192, 28, 28, 5, 2, "bf16", 0, name="stage2"),
        "stage3": Case(64, 384, 14, 14, 5, 1, "bf16", 0, name="stage3"),
    }
    for L in range(1, 6):
        cases[f"hires_L{L}"] = Case(8, 128, 256, 256, 5, L, "bf16", 0, name=f"hires_L{L}")
    for i, (c, hw, L) in enumerate([(96, 56, 3), (192, 28, 2), (384, 14, 1), (768, 7, 1)], 1):
        cases[f"stack_{i}"] = Case(128, c, hw, hw, 5, L, "bf16", 0, name=f"stack_{i}")
    cases["stage1_f16"] = Case(64, 96, 56, 56, 5, 3, "f16", 0, name="stage1_f16")
    for k in (5, 7):
        cases[f"dw{k}"] = Case(64, 96, 56, 56, k, 0, "bf16", 0, name=f"dw{k}")
    return cases
