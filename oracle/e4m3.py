"""fp64 model of fp8 (OCP e4m3fn) per-tensor quantisation, for the oracle.

TEST INFRASTRUCTURE ONLY (same rules as gpt_oracle: tests, the smoke check and
the benchmark's CPU baseline may use it; the product path never does).

The nanochat articles switch on fp8 training with a flag (the Turkish dev.to
page "ChatGPT'nizi 50 Dolara Nasil Egitirsiniz?", the note closing section
"3. Hassasiyet Yonetimi" and the d24 command of "Adim 4"; the German quick-start
page, "Problem 4", which ties it to torchao).  No page prints the recipe, so the
plainest one is taken: every operand of a Linear GEMM is scaled per tensor so
that its largest magnitude lands on the format's largest finite value, rounded
to the nearest e4m3 value (ties to even, saturating), multiplied exactly, and
the product divided by both scales.

e4m3fn: 1 sign, 4 exponent (bias 7) and 3 mantissa bits, no infinities,
largest finite value 448 = 1.75 * 2^8, smallest normal 2^-6, subnormal
spacing 2^-9.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_round(x):
    """Nearest e4m3fn value to each element (ties to even), saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                 # a = f * 2^e with f in [0.5, 1)
    e = np.maximum(e - 1, -6)          # binade of a; subnormals share the 2^-6 spacing rule
    step = np.ldexp(1.0, e - 3)        # 3 fraction bits per binade
    q = np.round(a / step) * step      # exact division by a power of two; numpy rounds half to even
    return np.copysign(np.minimum(q, E4M3_MAX), x)


def to_bf16(t):
    """Round to the nearest bfloat16 value (ties to even), via float32."""
    b = np.ascontiguousarray(np.asarray(t, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def scale_of(t):
    """Per-tensor current scale s = 448 / max|t| (1 for an all-zero tensor)."""
    amax = float(np.max(np.abs(t))) if np.size(t) else 0.0
    return E4M3_MAX / amax if amax > 0 else 1.0


def quantise(t, store=None):
    """Quantise-dequantise one tensor: e4m3(t * s) / s with s = 448 / max|t|.

    store=None takes every decision in fp64.  store="bf16" or "fp32" first rounds
    the tensor to the type it is held in and forms s and t * s in fp32, which is
    where a kernel that reads that tensor takes the same rounding decisions.
    """
    t = np.asarray(t, dtype=np.float64)
    if store is None:
        s = scale_of(t)
        return e4m3_round(t * s) / s
    x = (to_bf16(t) if store == "bf16" else t).astype(np.float32)
    amax = np.max(np.abs(x)) if x.size else np.float32(0)
    s = np.float32(E4M3_MAX) / amax if amax > 0 else np.float32(1)
    return e4m3_round((x * s).astype(np.float64)) / np.float64(s)
