"""Exact-rational brute force for tiny inputs (TEST INFRASTRUCTURE ONLY).

This is a second, independent way to evaluate the selection path. It is used to
pin the float64 oracle. Every stored input value (float32, bfloat16, or e4m3fn
times a float32 scale) is a dyadic rational, so `fractions.Fraction` holds it
exactly and the whole path down to the sign of each logit is evaluated with no
rounding. Loops are pure Python, so this is for tiny shapes only.

Formulas: [BLOG] §3.1 ("arXiv'26 | FlashMemory-DeepSeek-V4 …",
marsggbo.github.io). c = h W^DQ, q = c W^IUQ, w = h W^w, and
x_s = sum_j w_j ReLU(q_j . K_s). The threshold at theta = 0.5 is x_s >= 0.
The union is an OR over layers. The native top-k orders by (-y, s).
"""
from __future__ import annotations

from fractions import Fraction


def frac(v) -> Fraction:
    return Fraction(float(v))


def mat(a):
    """2-D array-like of floats -> list of lists of Fractions."""
    return [[frac(v) for v in row] for row in a]


def e4m3fn(byte: int) -> Fraction:
    """Exact value of one OCP FP8 E4M3 ("fn") byte, from its bit fields.

    Sign bit 7; exponent field bits 6..3 (bias 7); mantissa field bits 2..0.
    A zero exponent field is a subnormal, mantissa/8 * 2^-6. S.1111.111 is NaN
    and is refused here (keys are finite).
    """
    sign = -1 if byte & 0x80 else 1
    ef, mf = (byte >> 3) & 0xF, byte & 0x7
    if ef == 0xF and mf == 0x7:
        raise ValueError("NaN byte")
    if ef == 0:
        return sign * Fraction(mf, 8) * Fraction(1, 64)
    mag = Fraction(8 + mf, 8)
    return sign * (mag * 2 ** (ef - 7) if ef >= 7 else mag / 2 ** (7 - ef))


def fp8_keys(key_bytes, scales):
    """Exact keys of e4m3fn rows with one float32 scale per row: K_s = scale_s * value(byte)."""
    return [[frac(sc) * e4m3fn(int(b)) for b in row] for row, sc in zip(key_bytes, scales)]


def project(h_row, W_dq, W_iuq, W_w, n_h, d_h):
    """Exact c, q, w for one hidden state.

    The weights are in math layout: W_dq [d][r], W_iuq [r][n_h*d_h], W_w [d][n_h].
    """
    d, r = len(W_dq), len(W_dq[0])
    c = [sum(h_row[i] * W_dq[i][n] for i in range(d)) for n in range(r)]
    qf = [sum(c[i] * W_iuq[i][m] for i in range(r)) for m in range(n_h * d_h)]
    q = [qf[j * d_h:(j + 1) * d_h] for j in range(n_h)]
    w = [sum(h_row[i] * W_w[i][j] for i in range(d)) for j in range(n_h)]
    return c, q, w


def logit(q, w, key):
    """Exact x = sum_j w_j * max(0, q_j . key)."""
    tot = Fraction(0)
    for qj, wj in zip(q, w):
        dot = sum(a * b for a, b in zip(qj, key))
        if dot > 0:
            tot += wj * dot
    return tot


def selected_half(x: Fraction) -> bool:
    """I = sigma(x) >= 1/2  <=>  x >= 0 (sigma is strictly increasing, sigma(0) = 1/2)."""
    return x >= 0


def topk(y, idx, k):
    """Full sort by (-y, s). Return the first min(k, M) indices, ascending."""
    order = sorted(range(len(idx)), key=lambda i: (-y[i], idx[i]))
    return sorted(idx[i] for i in order[:min(k, len(idx))])
