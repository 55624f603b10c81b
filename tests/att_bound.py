"""The tolerance of the decode-attention GPU parity tests, fixed from the
definition's arithmetic and not from any kernel's order of operations.

The onnx-light-cpu roadmap ("Persistent KV Cache and Decode Performance
Roadmap", section "Phase 1") prescribes the precision: fp32 scores, softmax
and accumulation, in a streaming evaluation (per KV block the scores, the
online-softmax update, the V accumulation). The oracle evaluates the
definition in float64 from exactly decoded elements; the tolerance is the
forward error of any binary32 streaming evaluation of it in which every
elementary operation is rounded once (u = 2^-24), in any order and grouping,
with gamma_k = k u / (1 - k u):

  score     s_r = scale * sum_d q_d k_rd: D products, D - 1 additions and the
            scaling (an affine page element decoded with one more rounding),
            so |s_r error| <= delta = gamma_{D+2} S1 (paged: gamma_{D+3} S1),
            S1 = |scale| * max_r sum_d |q_d k_rd|;
  weight    w_r = exp(s_r - m): the two scores' errors, the rounding of the
            difference and of a change of base for exp2 (2 u (R + 8), where
            R = max_r |s_r - max s| and 8 allows an online maximum that lags
            the true one by up to 8 binary orders), exp within 2 u:
            relative error <= eps = exp(2 delta + 2 u (R + 8)) - 1 + 4 u;
            weights off by at most eps move the softmax average by at most
            2 eps / (1 - eps) * Vmax (Vmax = max |v| over the visible rows);
  sums      per visible row a product, an online rescale and an addition on
            the numerator (gamma_{3n} Vmax) and a rescale and an addition on
            the denominator (gamma_{2n} Vmax), one division (u Vmax); paged:
            the decoded values carry one rounding (u Vmax).

  tol_f32 = Vmax * (2 eps / (1 - eps) + gamma_{3n} + gamma_{2n} + u [+ u paged])

A 16-bit output adds its own rounding: tol = tol_f32 + u16 * (|ref| + tol_f32)
with u16 = 2^-8 (bf16) or 2^-11 (f16), plus half the f16 subnormal spacing.
Dropping or adding a row, a wrong window edge, a wrong KV head or a missing
scale moves the output by about Vmax / n, orders of magnitude more.
"""
from __future__ import annotations

import math

import numpy as np
import torch

U = 2.0 ** -24
U16 = {torch.float32: 0.0, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}
ABS16 = {torch.float32: 0.0, torch.float16: 2.0 ** -25, torch.bfloat16: 0.0}


def gamma(k: float) -> float:
    return k * U / (1.0 - k * U)


def window_tolerance(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                     paged: bool = False) -> float:
    """tol_f32 for one query row q [D] over visible rows k, v [n, D] (float64
    arrays of the exactly decoded elements)."""
    n, D = k.shape
    if n == 0:
        return 0.0
    prods = np.abs(q[None, :] * k).sum(axis=1)
    s1 = abs(scale) * prods.max()
    s = scale * (k @ q)
    R = float(np.max(s) - np.min(s))
    delta = gamma(D + (3 if paged else 2)) * s1
    eps = math.expm1(2 * delta + 2 * U * (R + 8)) + 4 * U
    vmax = float(np.abs(v).max())
    acc = gamma(3 * n) + gamma(2 * n) + U + (U if paged else 0.0)
    return vmax * (2 * eps / (1 - eps) + acc)


def with_output_rounding(tol32: np.ndarray, ref: np.ndarray, out_dtype) -> np.ndarray:
    """The tolerance of an output of out_dtype: tol_f32 plus its own rounding."""
    u16 = U16[out_dtype]
    return tol32 + u16 * (np.abs(ref) + tol32) + ABS16[out_dtype] + 1e-300
