"""Dense-grid brute force of the sampling core, for pinning the oracle on tiny inputs.

Independent of the oracle: no floor, no corner selection and no padding rule.
Each sample's bilinear read is written as a dense sum over every pixel (i, j)
of its level with the tent weights max(0, 1-|y-i|) * max(0, 1-|x-j|), which is
bilinear interpolation with zero outside the map. Summing those rows over the
samples of a (query, head) gives a dense sampling matrix, so the forward is a
plain matrix product with the value map: the "sampling points cover all
locations" degenerate case on page "Deformable DETR" (section "Multi-scale
deformable attention"). Index-space coordinates come from exact rational
arithmetic, rounded once to binary32.
"""
from fractions import Fraction

import numpy as np


def round_fraction_to_f32(fr):
    """Round an exact rational to the nearest binary32 (ties to even); normal range only."""
    if fr == 0:
        return 0.0
    sign = -1.0 if fr < 0 else 1.0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length() - 24
    while a / Fraction(2) ** e >= 2 ** 24:
        e += 1
    while a / Fraction(2) ** e < 2 ** 23:
        e -= 1
    assert e + 23 >= -126, "subnormal results are not handled"
    scaled = a / Fraction(2) ** e
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n) * 2.0 ** e


def exact_index_coordinate(loc32, size):
    """loc*size - 1/2 computed exactly from the float32 value, then rounded once to binary32."""
    return round_fraction_to_f32(Fraction(float(np.float32(loc32))) * size - Fraction(1, 2))


def tent(t):
    return np.maximum(0.0, 1.0 - np.abs(t))


def tent_right_derivative(t):
    """Derivative from the right of max(0, 1-|t|): +1 on [-1,0), -1 on [0,1), else 0."""
    return np.where((t >= -1) & (t < 0), 1.0, np.where((t >= 0) & (t < 1), -1.0, 0.0))


def dense_forward_backward(value, spatial_shapes, level_start, loc, attn, grad_out=None,
                           exact=True):
    """Returns out and, with grad_out, (grad_value, grad_loc, grad_attn), all float64.
    ``exact=False`` forms coordinates in float64 without the binary32 rounding."""
    value = np.asarray(value, dtype=np.float64)
    N, S, M, D = value.shape
    _, Lq, _, L, K, _ = loc.shape
    Gm = np.zeros((N, Lq, M, S))
    # per-sample dense tent rows and their x/y right-derivative rows
    rows = np.zeros((N, Lq, M, L, K, S))
    drow_x = np.zeros((N, Lq, M, L, K, S))
    drow_y = np.zeros((N, Lq, M, L, K, S))
    for l in range(L):
        H, W = int(spatial_shapes[l][0]), int(spatial_shapes[l][1])
        s0 = int(level_start[l])
        ii, jj = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
        ii, jj = ii.ravel().astype(np.float64), jj.ravel().astype(np.float64)
        for n in range(N):
            for q in range(Lq):
                for m in range(M):
                    for k in range(K):
                        lx, ly = loc[n, q, m, l, k]
                        if exact:
                            x = exact_index_coordinate(lx, W)
                            y = exact_index_coordinate(ly, H)
                        else:
                            x = float(lx) * W - 0.5
                            y = float(ly) * H - 0.5
                        tx, ty = tent(x - jj), tent(y - ii)
                        rows[n, q, m, l, k, s0:s0 + H * W] = ty * tx
                        drow_x[n, q, m, l, k, s0:s0 + H * W] = W * ty * tent_right_derivative(x - jj)
                        drow_y[n, q, m, l, k, s0:s0 + H * W] = H * tx * tent_right_derivative(y - ii)
    A = np.asarray(attn, dtype=np.float64)
    Gm = np.einsum("nqmlk,nqmlks->nqms", A, rows)
    out = np.zeros((N, Lq, M, D))
    for n in range(N):
        for m in range(M):
            out[n, :, m, :] = np.matmul(Gm[n, :, m, :], value[n, :, m, :])
    if grad_out is None:
        return out
    G = np.asarray(grad_out, dtype=np.float64)
    grad_value = np.zeros_like(value)
    # <G[n,q,m], V[n,s,m]> for every pixel s
    GV = np.zeros((N, Lq, M, S))
    for n in range(N):
        for m in range(M):
            grad_value[n, :, m, :] = np.matmul(Gm[n, :, m, :].T, G[n, :, m, :])
            GV[n, :, m, :] = np.matmul(G[n, :, m, :], value[n, :, m, :].T)
    grad_attn = np.einsum("nqmlks,nqms->nqmlk", rows, GV)
    grad_loc = np.stack([np.einsum("nqmlks,nqms->nqmlk", drow_x, GV) * A,
                         np.einsum("nqmlks,nqms->nqmlk", drow_y, GV) * A], axis=-1)
    return out, grad_value, grad_loc, grad_attn
