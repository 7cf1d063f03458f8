"""fp64 CPU oracle of the multi-scale deformable attention sampling core.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import or run this module. The HIP library and its Python
binding never call it, and it imports nothing from them.

What is computed (page "Deformable DETR", section "Multi-scale deformable
attention", equation MSDeformAttn, restricted to the part inside the outer
projection W_m and with W'_m already applied to the value map): for every batch
image n, query q and head m,

    out[n,q,m,:] = sum_l sum_k A[n,q,m,l,k] * x^l_m( phi_l(p_hat_q) + dp[n,q,m,l,k] )

where x^l_m(.) reads level l of head m's value map at a fractional location by
bilinear interpolation of the four surrounding pixels (same page, section
"Deformable attention module", symbol list; page "Deformable Attention
Module", its definition of the module: the bilinear sampling follows Dai et
al. 2017; page "Deformable Attention", bilinear from the four nearest pixels). The library receives the
sampling location already formed, as normalised coordinates
loc = phi_l-normalised reference + offset, so loc[...,0] is x (width) and
loc[...,1] is y (height), both in [0,1] inside the image.

Readings of what the pages leave open (each is documented with the repository):

* R1 pixel centres. (0,0) and (1,1) are the image's outer corners (section
  "Multi-scale deformable attention"), and phi_l multiplies by the level's
  width/height. A pixel is then a unit cell, pixel j's centre is at (j+0.5)/W,
  and the index-space coordinate is x = loc_x * W - 0.5 (likewise y with H).
* R2 zero padding. Offsets are unconstrained; the pages never say what lies
  outside the map. A corner outside the map reads 0, so a sample with
  -1 <= x < W and -1 <= y < H gets partial weight and any other contributes 0.
* R3 one rounding of the index coordinate. x is rounded once to binary32 (the
  GPU forms it with one fused multiply-add); everything after x is float64.
  For float32 loc with |loc| >= 2^-30 and W < 2^24 the float64 product and
  difference below are exact, so the single cast equals a correctly rounded
  fused multiply-add wherever floor(x) could change.
* R4 the floor rule at kinks. Bilinear interpolation is not differentiable in x
  at integer x; the oracle uses x0 = floor(x) everywhere, i.e. the
  right-derivative, including at x = -1 (which the in-map test keeps).
* R5 level flattening. Row of pixel (i, j) of level l is level_start[l] + i*W_l + j.
* R6 weights are used as given: no renormalisation and no softmax inside.

Gradients (page "Deformable Attention", differentiability of the bilinear
sampling, gradients flowing through the interpolation grid to the offsets):
out is linear in A and in the value map, and piecewise bilinear in (x, y); the
chain rule through x = loc_x*W - 0.5 gives d/dloc_x = W * d/dx (the rounding in
R3 is taken to have derivative 1).
"""
from __future__ import annotations

import numpy as np

# Corner order used throughout: (dy, dx) offsets from (y0, x0).
_CORNERS = ((0, 0), (0, 1), (1, 0), (1, 1))


def pixel_coordinate(loc, size, round_coords=True):
    """Index-space coordinate of a normalised location on an axis of ``size``
    pixels: loc*size - 0.5 (reading R1), rounded once to binary32 (R3) unless
    ``round_coords`` is False (used by finite-difference checks)."""
    t = np.asarray(loc, dtype=np.float64) * float(size) - 0.5
    if round_coords:
        t = t.astype(np.float32).astype(np.float64)
    return t


def _check(value, spatial_shapes, level_start, loc, attn):
    value = np.asarray(value)
    spatial_shapes = np.asarray(spatial_shapes, dtype=np.int64)
    level_start = np.asarray(level_start, dtype=np.int64)
    N, S, M, D = value.shape
    L = spatial_shapes.shape[0]
    assert spatial_shapes.shape == (L, 2) and level_start.shape == (L,)
    assert loc.shape[0] == N and loc.shape[2] == M and loc.shape[3] == L and loc.shape[5] == 2
    assert attn.shape == loc.shape[:5]
    for l in range(L):
        h, w = spatial_shapes[l]
        assert h >= 1 and w >= 1 and 0 <= level_start[l] and level_start[l] + h * w <= S
    return spatial_shapes, level_start


def _bilinear_terms(value, n, m, px, py, H, W, s0, round_coords):
    """For P samples on one level (batch index n[P], head m[P], normalised
    location (px, py)[P]), return the fractional parts a, b, the in-map flag of
    each sample, and the four corner reads Vpad[c] (each [P, D], zero where the
    corner is outside the map, reading R2) together with each corner's row and
    in-map flag."""
    x = pixel_coordinate(px, W, round_coords)
    y = pixel_coordinate(py, H, round_coords)
    # NaN fails every comparison, so a NaN location contributes nothing.
    inside = (x >= -1.0) & (x < W) & (y >= -1.0) & (y < H)
    x0 = np.floor(np.where(inside, x, 0.0))
    y0 = np.floor(np.where(inside, y, 0.0))
    a = np.where(inside, x, 0.0) - x0
    b = np.where(inside, y, 0.0) - y0
    reads, rows, oks = [], [], []
    D = value.shape[3]
    for dy, dx in _CORNERS:
        i = (y0 + dy).astype(np.int64)
        j = (x0 + dx).astype(np.int64)
        ok = inside & (i >= 0) & (i < H) & (j >= 0) & (j < W)
        row = s0 + np.where(ok, i * W + j, 0)
        v = np.where(ok[:, None], value[n, row, m, :], 0.0) if len(n) else np.zeros((0, D))
        reads.append(v)
        rows.append(row)
        oks.append(ok)
    return a, b, inside, reads, rows, oks


def _pairs_all(N, Lq, M):
    n, q, m = np.meshgrid(np.arange(N), np.arange(Lq), np.arange(M), indexing="ij")
    return n.ravel(), q.ravel(), m.ravel()


def msda_forward(value, spatial_shapes, level_start, loc, attn, pairs=None,
                 round_coords=True, chunk=1 << 16):
    """out[n,q,m,:] for every (n, q, m), or for the (n[P], q[P], m[P]) listed in
    ``pairs`` (then the result is [P, D]). float64 throughout."""
    spatial_shapes, level_start = _check(value, spatial_shapes, level_start, loc, attn)
    value = np.asarray(value, dtype=np.float64)
    N, S, M, D = value.shape
    Lq, L, K = loc.shape[1], loc.shape[3], loc.shape[4]
    full = pairs is None
    pn, pq, pm = _pairs_all(N, Lq, M) if full else (np.asarray(p, dtype=np.int64) for p in pairs)
    P = len(pn)
    out = np.zeros((P, D), dtype=np.float64)
    for c0 in range(0, P, chunk):
        n, q, m = pn[c0:c0 + chunk], pq[c0:c0 + chunk], pm[c0:c0 + chunk]
        acc = np.zeros((len(n), D), dtype=np.float64)
        for l in range(L):
            H, W = int(spatial_shapes[l, 0]), int(spatial_shapes[l, 1])
            s0 = int(level_start[l])
            for k in range(K):
                A = np.asarray(attn[n, q, m, l, k], dtype=np.float64)
                a, b, inside, V, _, _ = _bilinear_terms(
                    value, n, m, loc[n, q, m, l, k, 0], loc[n, q, m, l, k, 1], H, W, s0, round_coords)
                samp = (((1 - b) * (1 - a))[:, None] * V[0] + ((1 - b) * a)[:, None] * V[1]
                        + (b * (1 - a))[:, None] * V[2] + (b * a)[:, None] * V[3])
                acc += np.where(inside, A, 0.0)[:, None] * samp
        out[c0:c0 + chunk] = acc
    return out.reshape(N, Lq, M, D) if full else out


def msda_backward(value, spatial_shapes, level_start, loc, attn, grad_out, pairs=None,
                  round_coords=True, chunk=1 << 16, with_grad_value=True):
    """Gradients of sum(grad_out * out) with respect to value, loc and attn.

    Returns (grad_value [N,S,M,D] or None, grad_loc, grad_attn); with ``pairs``
    the last two are [P,L,K,2] and [P,L,K] for the listed pairs and grad_value
    (if requested) holds only their contributions."""
    spatial_shapes, level_start = _check(value, spatial_shapes, level_start, loc, attn)
    value = np.asarray(value, dtype=np.float64)
    grad_out = np.asarray(grad_out, dtype=np.float64)
    N, S, M, D = value.shape
    Lq, L, K = loc.shape[1], loc.shape[3], loc.shape[4]
    full = pairs is None
    pn, pq, pm = _pairs_all(N, Lq, M) if full else (np.asarray(p, dtype=np.int64) for p in pairs)
    P = len(pn)
    grad_value = np.zeros((N, S, M, D), dtype=np.float64) if with_grad_value else None
    grad_loc = np.zeros((P, L, K, 2), dtype=np.float64)
    grad_attn = np.zeros((P, L, K), dtype=np.float64)
    for c0 in range(0, P, chunk):
        n, q, m = pn[c0:c0 + chunk], pq[c0:c0 + chunk], pm[c0:c0 + chunk]
        G = grad_out[n, q, m, :]
        for l in range(L):
            H, W = int(spatial_shapes[l, 0]), int(spatial_shapes[l, 1])
            s0 = int(level_start[l])
            for k in range(K):
                A = np.asarray(attn[n, q, m, l, k], dtype=np.float64)
                a, b, inside, V, rows, oks = _bilinear_terms(
                    value, n, m, loc[n, q, m, l, k, 0], loc[n, q, m, l, k, 1], H, W, s0, round_coords)
                w = ((1 - b) * (1 - a), (1 - b) * a, b * (1 - a), b * a)
                samp = sum(wc[:, None] * Vc for wc, Vc in zip(w, V))
                # out is linear in A: d out / d A = the bilinear sample.
                grad_attn[c0:c0 + chunk, l, k] = np.where(inside, (G * samp).sum(1), 0.0)
                # d sample / d x and d / d y of the bilinear form (right-derivative, R4).
                dsdx = (1 - b)[:, None] * (V[1] - V[0]) + b[:, None] * (V[3] - V[2])
                dsdy = (1 - a)[:, None] * (V[2] - V[0]) + a[:, None] * (V[3] - V[1])
                grad_loc[c0:c0 + chunk, l, k, 0] = np.where(inside, A * W * (G * dsdx).sum(1), 0.0)
                grad_loc[c0:c0 + chunk, l, k, 1] = np.where(inside, A * H * (G * dsdy).sum(1), 0.0)
                if with_grad_value:
                    # out is linear in the value map: each in-map corner receives A * w_c * G.
                    for wc, row, ok in zip(w, rows, oks):
                        sel = ok & inside
                        np.add.at(grad_value, (n[sel], row[sel], m[sel]),
                                  (A * wc)[sel, None] * G[sel])
    if full:
        grad_loc = grad_loc.reshape(N, Lq, M, L, K, 2)
        grad_attn = grad_attn.reshape(N, Lq, M, L, K)
    return grad_value, grad_loc, grad_attn


def msda_grad_value_rows(value, spatial_shapes, level_start, loc, attn, grad_out, rows,
                         round_coords=True, chunk=1 << 16):
    """grad_value at the listed (n[R], s[R], m[R]) rows only ([R, D]), summing
    every sample corner that lands on them. Scans all points once; used where the
    full scatter would be too slow."""
    spatial_shapes, level_start = _check(value, spatial_shapes, level_start, loc, attn)
    value = np.asarray(value, dtype=np.float64)
    N, S, M, D = value.shape
    Lq, L, K = loc.shape[1], loc.shape[3], loc.shape[4]
    rn, rs, rm = (np.asarray(r, dtype=np.int64) for r in rows)
    keys = (rn * S + rs) * M + rm
    order = np.argsort(keys, kind="stable")
    skeys = keys[order]
    res = np.zeros((len(keys), D), dtype=np.float64)
    pn, pq, pm = _pairs_all(N, Lq, M)
    for c0 in range(0, len(pn), chunk):
        n, q, m = pn[c0:c0 + chunk], pq[c0:c0 + chunk], pm[c0:c0 + chunk]
        for l in range(L):
            H, W = int(spatial_shapes[l, 0]), int(spatial_shapes[l, 1])
            s0 = int(level_start[l])
            for k in range(K):
                px, py = loc[n, q, m, l, k, 0], loc[n, q, m, l, k, 1]
                x = pixel_coordinate(px, W, round_coords)
                y = pixel_coordinate(py, H, round_coords)
                inside = (x >= -1.0) & (x < W) & (y >= -1.0) & (y < H)
                x0 = np.floor(np.where(inside, x, 0.0))
                y0 = np.floor(np.where(inside, y, 0.0))
                a = np.where(inside, x, 0.0) - x0
                b = np.where(inside, y, 0.0) - y0
                A = np.asarray(attn[n, q, m, l, k], dtype=np.float64)
                w = ((1 - b) * (1 - a), (1 - b) * a, b * (1 - a), b * a)
                for (dy, dx), wc in zip(_CORNERS, w):
                    i = (y0 + dy).astype(np.int64)
                    j = (x0 + dx).astype(np.int64)
                    ok = inside & (i >= 0) & (i < H) & (j >= 0) & (j < W)
                    key = (n * S + s0 + np.where(ok, i * W + j, 0)) * M + m
                    pos = np.searchsorted(skeys, key)
                    hit = ok & (pos < len(skeys))
                    hit[hit] = skeys[pos[hit]] == key[hit]
                    if not hit.any():
                        continue
                    contrib = (A * wc)[hit, None] * np.asarray(grad_out[n[hit], q[hit], m[hit], :], dtype=np.float64)
                    # Duplicate requested rows share one slot; spread back below.
                    np.add.at(res, order[pos[hit]], contrib)
    # Rows requested twice: copy the accumulated value to every duplicate.
    first = np.searchsorted(skeys, keys)
    return res[order[first]]


# --- the step before the sampling core ------------------------------------------------------
#
# Page "Deformable DETR", section "Deformable attention module": one linear
# projection of the query gives 2MK offset channels and MK logits, and the
# logits go through a softmax; section "Multi-scale deformable attention": the
# weights are normalised jointly over the L*K samples of a head and the
# sampling location is phi_l(p_hat) + offset, i.e. the reference point in
# level-l pixels plus an offset in level-l pixels. Section "Variants"
# (iterative bounding box refinement): with a box as reference, the offsets
# are scaled by the box's width and height around its centre.
#
# Reading R11 (arithmetic of the location, which the pages leave open): the
# location is formed in binary32, for points as fl(ref + fl(offset / size))
# with size = W_l for x and H_l for y, and for boxes as one fused
# multiply-add fl(centre + offset * box_size). It then goes through the same
# index-coordinate rule as a given location (R1, R3).


def softmax_weights(logits):
    """Softmax over the last two axes (L*K samples of one (n, q, m)), float64."""
    z = np.asarray(logits, dtype=np.float64)
    shape = z.shape
    z = z.reshape(shape[:-2] + (-1,))
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).reshape(shape)


def fused_locations(ref, offsets, spatial_shapes, exact=False):
    """Normalised locations [N,Lq,M,L,K,2] from reference points ([N,Lq,2]) with
    offsets in pixels of each level, or from boxes ([N,Lq,4] = cx, cy, w, h)
    with offsets in units of the box size (reading R11). ``exact=True`` forms
    them in float64 without binary32 rounding (for finite differences)."""
    ref = np.asarray(ref)
    off = np.asarray(offsets)
    ss = np.asarray(spatial_shapes, dtype=np.int64)
    L = ss.shape[0]
    size = np.stack([ss[:, 1], ss[:, 0]], axis=-1)  # (W_l, H_l) per level
    if exact:
        off = off.astype(np.float64)
        r = ref.astype(np.float64)
        if r.shape[-1] == 2:
            return r[:, :, None, None, None, :] + off / size.reshape(1, 1, 1, L, 1, 2)
        return r[:, :, None, None, None, :2] + off * r[:, :, None, None, None, 2:]
    off = off.astype(np.float32)
    r = ref.astype(np.float32)
    if r.shape[-1] == 2:
        step = (off / size.reshape(1, 1, 1, L, 1, 2).astype(np.float32)).astype(np.float32)
        return (r[:, :, None, None, None, :] + step).astype(np.float32)
    # one rounding of centre + offset * size: the float64 product of two
    # binary32 numbers is exact, so only the sum is inexact
    c = r[:, :, None, None, None, :2].astype(np.float64)
    wh = r[:, :, None, None, None, 2:].astype(np.float64)
    return _round_sum_to_f32(np.broadcast_to(c, off.shape), off.astype(np.float64) * wh)


def _round_sum_to_f32(a, b):
    """binary32 nearest (ties to even) of the exact sum of float64 arrays a + b.

    Rounding the float64 sum to binary32 rounds twice; the two differ only when
    the float64 sum s is exactly halfway between two binary32 numbers while the
    exact sum is not. Knuth's TwoSum gives the exact error e = (a + b) - s, and
    its sign then decides the halfway case. A non-finite operand gives the
    non-finite sum (its error term is NaN and the halfway test false)."""
    with np.errstate(invalid="ignore"):
        s = a + b
        bv = s - a
        e = (a - (s - bv)) + (b - bv)
        r = s.astype(np.float32)
        r64 = r.astype(np.float64)
        other = np.where(r64 > s, np.nextafter(r, np.float32(-np.inf)), np.nextafter(r, np.float32(np.inf)))
        halfway = (r64 + other.astype(np.float64)) * 0.5 == s
        # at a halfway s, the exact sum lies on the side of `other` when e points there
        toward_other = np.sign(e) == np.sign(other.astype(np.float64) - s)
    return np.where(halfway & (e != 0) & toward_other, other, r).astype(np.float32)


def msda_fused_forward(value, spatial_shapes, level_start, ref, offsets, logits, **kw):
    """out from the raw step before the core: locations from (ref, offsets),
    weights = softmax(logits); then the sampling core (with deformable groups
    when offsets has fewer heads than value, reading R12)."""
    loc = fused_locations(ref, offsets, spatial_shapes, exact=kw.pop("exact_locations", False))
    core = msda_forward if np.shape(offsets)[2] == np.shape(value)[2] else msda_grouped_forward
    return core(value, spatial_shapes, level_start, loc, softmax_weights(logits), **kw)


def msda_fused_backward(value, spatial_shapes, level_start, ref, offsets, logits, grad_out, queries=None,
                        **kw):
    """(grad_value, grad_offsets, grad_logits, grad_ref) by the chain rule through
    the softmax (dA_i/dz_j = A_i (delta_ij - A_j)) and the location formula
    (d loc / d offset = 1/size for points, box size for boxes; d loc / d ref =
    identity on the centre, offset on the box size). The rounding of R11 is
    taken to have derivative 1.

    ``queries=(n, q)`` restricts the result to the listed queries (all M heads
    of each): grad_value is then None and the other three are [Q, M, L, K, 2],
    [Q, M, L, K] and [Q, ref_dim]."""
    exact = kw.pop("exact_locations", False)
    loc = fused_locations(ref, offsets, spatial_shapes, exact=exact)
    A = softmax_weights(logits)
    off = np.asarray(offsets, dtype=np.float64)
    ref64 = np.asarray(ref, dtype=np.float64)
    if queries is None:
        core = msda_backward if off.shape[2] == np.shape(value)[2] else msda_grouped_backward
        gv, gl, ga = core(value, spatial_shapes, level_start, loc, A, grad_out, **kw)
    else:
        qn, qq = (np.asarray(a, dtype=np.int64) for a in queries)
        Q, M = len(qn), off.shape[2]
        pairs = (np.repeat(qn, M), np.repeat(qq, M), np.tile(np.arange(M), Q))
        gv, gl, ga = msda_backward(value, spatial_shapes, level_start, loc, A, grad_out, pairs=pairs,
                                   with_grad_value=False, **kw)
        gl = gl.reshape((Q,) + off.shape[2:])
        ga = ga.reshape((Q,) + off.shape[2:5])
        A, off, ref64 = A[qn, qq], off[qn, qq], ref64[qn, qq]
    # from here on the arrays are [..., M, L, K(, 2)] behind the query axes
    s = (A * ga).sum(axis=(-2, -1), keepdims=True)
    grad_logits = A * (ga - s)
    ss = np.asarray(spatial_shapes, dtype=np.int64)
    L = ss.shape[0]
    heads_levels_points = (-4, -3, -2)
    if ref64.shape[-1] == 2:
        size = np.stack([ss[:, 1], ss[:, 0]], axis=-1).reshape(L, 1, 2)  # (W_l, H_l)
        grad_off = gl / size
        grad_ref = gl.sum(axis=heads_levels_points)
    else:
        wh = ref64[..., None, None, None, 2:]
        grad_off = gl * wh
        # a sample outside the map (a non-finite location included, reading R2)
        # is absent from the sum: its term is zero, not 0 * offset (NaN when the
        # offset is infinite or NaN)
        with np.errstate(invalid="ignore"):
            size_terms = np.where(gl == 0.0, 0.0, gl * off)
        grad_ref = np.concatenate([gl.sum(axis=heads_levels_points),
                                   size_terms.sum(axis=heads_levels_points)], axis=-1)
    return gv, grad_off, grad_logits, grad_ref


# --- deformable groups ------------------------------------------------------------------------
#
# Page "Deformable Attention" (glossary), on heads and groups: heads are
# gathered into fewer deformable groups that share one set of sampled keys
# while keeping their own projections. Reading R12: G groups of M/G consecutive
# heads; group g = m // (M/G) supplies the sampling locations and the weights of
# head m; each head still reads its own value channels.

def _heads_from_groups(a, M):
    G = a.shape[2]
    if M % G:
        raise ValueError(f"groups ({G}) must divide heads ({M})")
    return np.repeat(np.asarray(a), M // G, axis=2)


def msda_grouped_forward(value, spatial_shapes, level_start, loc, attn, **kw):
    """out[n,q,m,:] with loc [N,Lq,G,L,K,2] and attn [N,Lq,G,L,K] shared by the
    M/G heads of each group: every head samples with its group's locations."""
    M = np.asarray(value).shape[2]
    return msda_forward(value, spatial_shapes, level_start, _heads_from_groups(loc, M),
                        _heads_from_groups(attn, M), **kw)


def msda_grouped_backward(value, spatial_shapes, level_start, loc, attn, grad_out, **kw):
    """(grad_value, grad_loc [N,Lq,G,L,K,2], grad_attn [N,Lq,G,L,K]): a group's
    location and weight feed all its heads, so their gradients are the sums of
    the per-head gradients over the group's heads."""
    M = np.asarray(value).shape[2]
    G = np.asarray(loc).shape[2]
    gv, gl, ga = msda_backward(value, spatial_shapes, level_start, _heads_from_groups(loc, M),
                               _heads_from_groups(attn, M), grad_out, **kw)
    N, Lq = gl.shape[:2]
    gl = gl.reshape((N, Lq, G, M // G) + gl.shape[3:]).sum(axis=3)
    ga = ga.reshape((N, Lq, G, M // G) + ga.shape[3:]).sum(axis=3)
    return gv, gl, ga
