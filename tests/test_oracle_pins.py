"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test ties one part of the oracle to something it does not compute itself:
the worked example printed on page "Deformable DETR Samples Sparse Points",
closed forms, invariants of the equation, a dense brute force written without
floor or padding logic, a library bilinear sampler, finite differences and exact
rational arithmetic.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (fused_locations, msda_backward, msda_forward, msda_fused_backward,
                    msda_fused_forward, msda_grad_value_rows, msda_grouped_backward,
                    msda_grouped_forward, pixel_coordinate, softmax_weights)
from tests.dense_reference import (dense_forward_backward, exact_index_coordinate,
                                   round_fraction_to_f32)
from workloads import init_pattern_workload, level_starts, uniform_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _single(value_hw, loc_xy, weights, M=1, D=1):
    """Helper: one image, one query, one level, K = len(weights) samples."""
    H, W = value_hw.shape[:2]
    value = value_hw.reshape(1, H * W, M, D)
    K = len(weights)
    loc = np.asarray(loc_xy, dtype=np.float32).reshape(1, 1, M, 1, K, 2)
    attn = np.asarray(weights, dtype=np.float32).reshape(1, 1, M, 1, K)
    return value, np.array([[H, W]]), np.array([0]), loc, attn


# --- P1: the printed worked example -------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        return json.load(f)


def test_worked_example_offsets_add_up():
    g = _golden()
    ref = np.array(g["reference_point"])
    np.testing.assert_allclose(ref + np.array(g["offsets"]), np.array(g["locations"]), atol=1e-12)
    np.testing.assert_allclose(np.array(g["weights"]) * np.array(g["sampled_values"]),
                               g["products"], atol=1e-12)


def test_worked_example_pixel_centres():
    """The page's four samples fall next to the 2x2 pixel block around (14,14) of the
    28x28 map; reading those pixels at their centres with the page's weights blends
    their values to the printed 0.70."""
    g = _golden()
    H, W = g["map_hw"]
    rng = np.random.default_rng(0)
    vmap = rng.uniform(-1, 1, (H, W))
    pix = [(14, 14), (13, 14), (13, 13), (14, 13)]  # (x, y) nearest pixel of each printed location
    for (x, y), v in zip(pix, g["sampled_values"]):
        vmap[y, x] = v
    # nearest-pixel claim: each printed location is within one pixel of the chosen centre
    for (x, y), (lx, ly) in zip(pix, g["locations"]):
        assert abs(lx * W - 0.5 - x) <= 0.5 + 1e-9 and abs(ly * H - 0.5 - y) <= 0.5 + 1e-9
    loc = [((x + 0.5) / W, (y + 0.5) / H) for x, y in pix]
    out = msda_forward(*_single(vmap, loc, g["weights"]))
    assert abs(out[0, 0, 0, 0] - g["blend"]) < 1e-6  # weights are float32 inputs


def test_worked_example_page_locations():
    """At the page's own fractional locations: on a map that holds a bilinear surface
    f = c0 + c1 x + c2 y + c3 xy (pixel coordinates), bilinear interpolation is exact,
    so choosing c with f(sample_k) = printed value_k makes the blend exactly 0.70."""
    g = _golden()
    H, W = g["map_hw"]
    xs = [exact_index_coordinate(lx, W) for lx, _ in g["locations"]]
    ys = [exact_index_coordinate(ly, H) for _, ly in g["locations"]]
    Amat = np.array([[1.0, x, y, x * y] for x, y in zip(xs, ys)])
    c = np.linalg.solve(Amat, np.array(g["sampled_values"]))
    ii, jj = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    vmap = c[0] + c[1] * jj + c[2] * ii + c[3] * jj * ii
    out = msda_forward(*_single(vmap, g["locations"], g["weights"]))
    w32 = np.asarray(g["weights"], dtype=np.float32).astype(np.float64)
    expect = float(np.dot(w32, g["sampled_values"]))
    assert abs(expect - g["blend"]) < 1e-7
    assert abs(out[0, 0, 0, 0] - expect) < 1e-10


# --- R3: the single binary32 rounding of the index coordinate -------------------------------

def test_pixel_coordinate_is_one_correct_rounding():
    rng = np.random.default_rng(11)
    locs = np.concatenate([
        rng.uniform(-0.2, 1.2, 4000),
        # adversarial: locations whose index coordinate is within an ulp of an integer
        ((np.arange(-3, 170) + 0.5) / 167.0),
        np.nextafter(((np.arange(-3, 170) + 0.5) / 167.0).astype(np.float32), np.float32(2)),
        np.nextafter(((np.arange(-3, 170) + 0.5) / 167.0).astype(np.float32), np.float32(-2)),
    ]).astype(np.float32)
    for size in (13, 16, 21, 42, 84, 100, 167):
        got = pixel_coordinate(locs, size)
        for lv, gv in zip(locs[::7], got[::7]):
            ex = Fraction(float(lv)) * size - Fraction(1, 2)
            if ex == 0 or abs(ex) < Fraction(1, 2 ** 100):
                continue
            assert gv == round_fraction_to_f32(ex)


# --- P2: constant maps ----------------------------------------------------------------------

def _tent_mass(t, n):
    """In-map share of a unit tent centred at index coordinate t on an axis of n pixels."""
    return np.clip(np.minimum(t + 1.0, n - t), 0.0, 1.0)


def test_constant_map_inside_returns_constant():
    w = uniform_workload(N=2, shapes=((7, 9), (4, 5)), Lq=11, M=3, D=4, K=3, seed=21, lo=0.2, hi=0.8)
    w.value[:] = 0.625
    out = msda_forward(w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)
    expect = 0.625 * w.attn.astype(np.float64).sum(axis=(3, 4))
    np.testing.assert_allclose(out, np.broadcast_to(expect[..., None], out.shape), rtol=0, atol=1e-12)


def test_constant_map_border_mass_closed_form():
    w = uniform_workload(N=1, shapes=((6, 10), (3, 4)), Lq=40, M=2, D=2, K=4, seed=22, lo=-0.4, hi=1.4)
    w.value[:] = -1.5
    out = msda_forward(w.value, w.spatial_shapes, w.level_start, w.loc, w.attn, round_coords=False)
    expect = np.zeros(out.shape[:3])
    for l, (H, W) in enumerate(w.spatial_shapes):
        x = w.loc[:, :, :, l, :, 0].astype(np.float64) * W - 0.5
        y = w.loc[:, :, :, l, :, 1].astype(np.float64) * H - 0.5
        expect += (w.attn[:, :, :, l, :] * _tent_mass(x, W) * _tent_mass(y, H)).sum(-1)
    np.testing.assert_allclose(out, -1.5 * np.broadcast_to(expect[..., None], out.shape), atol=1e-12)


# --- P3: pixel-centre reads ----------------------------------------------------------------

def test_pixel_centres_read_exact_pixels():
    rng = np.random.default_rng(3)
    H, W, M, D, K = 16, 8, 2, 3, 5
    value = rng.standard_normal((1, H * W, M, D))
    ii = rng.integers(0, H, (1, 1, M, 1, K))
    jj = rng.integers(0, W, (1, 1, M, 1, K))
    loc = np.stack([(jj + 0.5) / W, (ii + 0.5) / H], axis=-1).astype(np.float32)
    attn = rng.uniform(0, 1, (1, 1, M, 1, K)).astype(np.float32)
    out = msda_forward(value, [[H, W]], [0], loc, attn)
    for m in range(M):
        expect = sum(attn[0, 0, m, 0, k] * value[0, ii[0, 0, m, 0, k] * W + jj[0, 0, m, 0, k], m]
                     for k in range(K))
        np.testing.assert_allclose(out[0, 0, m], expect, atol=1e-14)


# --- P4: border closed forms -----------------------------------------------------------------

def test_border_closed_forms():
    rng = np.random.default_rng(4)
    H, W = 8, 16
    vmap = rng.standard_normal((H, W))
    i = 5
    cases = [((0.0, 0.0), 0.25 * vmap[0, 0]),
             ((1.0, 1.0), 0.25 * vmap[H - 1, W - 1]),
             ((0.0, (i + 0.5) / H), 0.5 * vmap[i, 0]),
             ((1.0, (i + 0.5) / H), 0.5 * vmap[i, W - 1]),
             ((-2.0 / W, 0.5), 0.0),          # x = -2.5: beyond one pixel outside
             ((0.5, 1.0 + 1.0 / H), 0.0),     # y = H + 0.5
             ((1.0 + 0.5 / W, 0.5), 0.0)]     # x = W exactly: outside by the half-open rule
    for (lx, ly), expect in cases:
        args = _single(vmap, [(lx, ly)], [0.8])
        out = msda_forward(*args)
        assert abs(out[0, 0, 0, 0] - 0.8 * expect) < 1e-7, (lx, ly)
        gv, gl, ga = msda_backward(*args, grad_out=np.ones((1, 1, 1, 1)))
        if expect == 0.0:
            assert np.all(gv == 0) and np.all(gl == 0) and np.all(ga == 0)


# --- P5: dense-grid brute force ----------------------------------------------------------------

@pytest.mark.parametrize("seed", [31, 32])
def test_dense_bruteforce_forward_backward(seed):
    w = uniform_workload(N=2, shapes=((5, 7), (3, 4), (2, 2)), Lq=6, M=3, D=4, K=3, seed=seed,
                         lo=-0.15, hi=1.15, with_grad=True)
    args = (w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)
    out, gv_d, gl_d, ga_d = dense_forward_backward(*args, grad_out=w.grad_out)
    np.testing.assert_allclose(msda_forward(*args), out, atol=1e-13)
    gv, gl, ga = msda_backward(*args, grad_out=w.grad_out)
    np.testing.assert_allclose(gv, gv_d, atol=1e-12)
    np.testing.assert_allclose(ga, ga_d, atol=1e-12)
    np.testing.assert_allclose(gl, gl_d, atol=1e-10)


def test_dense_bruteforce_on_kinks():
    """P10: the compass initialisation puts every sample on a pixel centre, where the
    location gradient jumps; the oracle must give the right-derivative there."""
    w = init_pattern_workload(N=1, shape=(8, 8), M=8, D=3, K=2, seed=7)
    w = _subset_queries(w, np.arange(0, 64, 5))
    args = (w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)
    x = w.loc[..., 0].astype(np.float64) * 8 - 0.5
    assert np.all(x == np.round(x))  # every sample exactly on a kink
    out, gv_d, gl_d, ga_d = dense_forward_backward(*args, grad_out=w.grad_out)
    gv, gl, ga = msda_backward(*args, grad_out=w.grad_out)
    np.testing.assert_allclose(msda_forward(*args), out, atol=1e-13)
    np.testing.assert_allclose(gl, gl_d, atol=1e-11)
    np.testing.assert_allclose(gv, gv_d, atol=1e-12)
    np.testing.assert_allclose(ga, ga_d, atol=1e-12)
    # and the right-derivative is what a forward difference sees
    h = 2.0 ** -20
    for axis in (0, 1):
        lp = w.loc.astype(np.float64).copy()
        lp[..., axis] += h
        fd = ((msda_forward(w.value, w.spatial_shapes, w.level_start, lp, w.attn, round_coords=False)
               - out) * w.grad_out).sum()
        np.testing.assert_allclose(fd / h, gl[..., axis].sum(), rtol=1e-6, atol=1e-8)


def _subset_queries(w, qs):
    w.loc = np.ascontiguousarray(w.loc[:, qs])
    w.attn = np.ascontiguousarray(w.attn[:, qs])
    w.grad_out = np.ascontiguousarray(w.grad_out[:, qs])
    return w


# --- P6: a library bilinear sampler ----------------------------------------------------------------

def test_single_sample_matches_torch_grid_sample():
    """L=1, K=1, A=1 is a plain bilinear sample (the deformable-convolution special
    case on page "Deformable DETR"); compare with torch's CPU grid_sample in float64,
    zero padding, align_corners=False, grid = 2*loc - 1."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    H, W, D, P = 6, 9, 3, 200
    vmap = rng.standard_normal((H, W, D))
    loc = rng.uniform(-0.2, 1.2, (P, 2)).astype(np.float32)
    x = loc[:, 0].astype(np.float64) * W - 0.5
    y = loc[:, 1].astype(np.float64) * H - 0.5
    off_kink = (np.abs(x - np.round(x)) > 1e-4) & (np.abs(y - np.round(y)) > 1e-4)
    value = vmap.reshape(1, H * W, 1, D)
    locs = loc.reshape(1, P, 1, 1, 1, 2)
    attn = np.ones((1, P, 1, 1, 1), dtype=np.float32)
    G = rng.standard_normal((1, P, 1, D))
    out = msda_forward(value, [[H, W]], [0], locs, attn, round_coords=False)
    gv, gl, _ = msda_backward(value, [[H, W]], [0], locs, attn, G, round_coords=False)
    inp = torch.tensor(vmap.transpose(2, 0, 1)[None], dtype=torch.float64, requires_grad=True)
    grid = torch.tensor(2.0 * loc.astype(np.float64) - 1.0, dtype=torch.float64).reshape(1, 1, P, 2)
    grid.requires_grad_(True)
    ref = torch.nn.functional.grid_sample(inp, grid, mode="bilinear", padding_mode="zeros",
                                          align_corners=False)  # [1, D, 1, P]
    np.testing.assert_allclose(out[0, :, 0, :], ref[0, :, 0, :].T.detach().numpy(), atol=1e-12)
    (ref[0, :, 0, :].T * torch.tensor(G[0, :, 0, :])).sum().backward()
    np.testing.assert_allclose(gv.reshape(H, W, D), inp.grad[0].numpy().transpose(1, 2, 0), atol=1e-12)
    g_grid = grid.grad.numpy().reshape(P, 2)
    np.testing.assert_allclose(gl.reshape(P, 2)[off_kink], 2.0 * g_grid[off_kink], atol=1e-10)


# --- P7: finite differences ----------------------------------------------------------------------

def test_finite_differences():
    w = uniform_workload(N=1, shapes=((6, 8), (3, 5)), Lq=5, M=2, D=3, K=2, seed=41,
                         lo=-0.1, hi=1.1, with_grad=True)
    loc = w.loc.astype(np.float64)
    args = (w.value, w.spatial_shapes, w.level_start)
    G = w.grad_out.astype(np.float64)
    gv, gl, ga = msda_backward(*args, loc, w.attn, G, round_coords=False)

    def f(value=w.value, loc=loc, attn=w.attn):
        return (msda_forward(value, w.spatial_shapes, w.level_start, loc, attn, round_coords=False) * G).sum()

    rng = np.random.default_rng(0)
    # value and attn: the output is linear in each, so any step is exact up to rounding
    for _ in range(10):
        idx = tuple(rng.integers(0, s) for s in w.value.shape)
        v2 = w.value.astype(np.float64).copy()
        v2[idx] += 0.5
        assert abs((f(value=v2) - f()) / 0.5 - gv[idx]) < 1e-10
        idx = tuple(rng.integers(0, s) for s in w.attn.shape)
        a2 = w.attn.astype(np.float64).copy()
        a2[idx] += 0.5
        assert abs((f(attn=a2) - f()) / 0.5 - ga[idx]) < 1e-10
    # loc: central differences away from kinks
    checked = 0
    for idx in np.ndindex(*loc.shape):
        l = idx[3]
        size = w.spatial_shapes[l][1 - idx[5]]  # x uses W, y uses H
        t = loc[idx] * size - 0.5
        if abs(t - np.round(t)) < 1e-4:
            continue
        h = 1e-6 / size
        lp, lm = loc.copy(), loc.copy()
        lp[idx] += h
        lm[idx] -= h
        fd = (f(loc=lp) - f(loc=lm)) / (2 * h)
        assert abs(fd - gl[idx]) < 1e-6 * max(1.0, abs(gl[idx])), (idx, fd, gl[idx])
        checked += 1
    assert checked > 50


# --- P8: adjoint identities ----------------------------------------------------------------------

def test_adjoint_identities():
    w = uniform_workload(N=2, shapes=((9, 11), (5, 6)), Lq=30, M=4, D=5, K=3, seed=51,
                         lo=-0.1, hi=1.1, with_grad=True)
    args = (w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)
    out = msda_forward(*args)
    gv, gl, ga = msda_backward(*args, grad_out=w.grad_out)
    lhs = (w.grad_out.astype(np.float64) * out).sum()
    assert abs(lhs - (gv * w.value).sum()) < 1e-10 * max(1, abs(lhs))
    assert abs(lhs - (ga * w.attn).sum()) < 1e-10 * max(1, abs(lhs))


# --- P9: invariants --------------------------------------------------------------------------------

def test_invariants_heads_levels_batch():
    w = uniform_workload(N=3, shapes=((6, 7), (3, 4)), Lq=9, M=4, D=3, K=2, seed=61, lo=-0.1, hi=1.1)
    args = (w.value, w.spatial_shapes, w.level_start)
    out = msda_forward(*args, w.loc, w.attn)
    # head permutation equivariance
    perm = np.array([2, 0, 3, 1])
    outp = msda_forward(w.value[:, :, perm], w.spatial_shapes, w.level_start, w.loc[:, :, perm],
                        w.attn[:, :, perm])
    np.testing.assert_allclose(outp, out[:, :, perm], atol=1e-14)
    # level additivity
    acc = 0
    for l in range(2):
        a = np.zeros_like(w.attn)
        a[:, :, :, l] = w.attn[:, :, :, l]
        acc = acc + msda_forward(*args, w.loc, a)
    np.testing.assert_allclose(acc, out, atol=1e-13)
    # batch independence
    out1 = msda_forward(w.value[1:2], w.spatial_shapes, w.level_start, w.loc[1:2], w.attn[1:2])
    np.testing.assert_allclose(out1, out[1:2], atol=1e-14)


def test_transpose_and_translation():
    rng = np.random.default_rng(71)
    H, W, M, D, K, Lq = 8, 16, 2, 3, 4, 7  # non-square, powers of two: exact coordinates
    vmap = rng.standard_normal((H, W, M, D))
    # locations on a 1/1024 lattice keep every coordinate exact in binary32
    loc = (rng.integers(-50, 1074, (1, Lq, M, 1, K, 2)) / 1024.0).astype(np.float32)
    attn = rng.uniform(0, 1, (1, Lq, M, 1, K)).astype(np.float32)
    out = msda_forward(vmap.reshape(1, H * W, M, D), [[H, W]], [0], loc, attn)
    # transposed map with swapped location components
    vt = vmap.transpose(1, 0, 2, 3).reshape(1, W * H, M, D)
    outt = msda_forward(vt, [[W, H]], [0], loc[..., ::-1].copy(), attn)
    np.testing.assert_allclose(outt, out, atol=1e-14)
    # translation: shift the map one pixel right (zero column enters on the left) and the
    # locations by one pixel; samples that stay clear of the new border are unchanged
    vs = np.zeros((H, W + 1, M, D))
    vs[:, 1:] = vmap
    loc_s = loc.astype(np.float64).copy()
    loc_s[..., 0] = (loc_s[..., 0] * W + 1.0) / (W + 1)
    outs = msda_forward(vs.reshape(1, H * (W + 1), M, D), [[H, W + 1]], [0], loc_s, attn,
                        round_coords=False)
    np.testing.assert_allclose(outs, out, atol=1e-12)


# --- helpers used at full size agree with the full computation -------------------------------------

def test_pair_subset_and_row_subset_agree_with_full():
    w = uniform_workload(N=2, shapes=((7, 9), (4, 5)), Lq=13, M=3, D=4, K=3, seed=81, lo=-0.1, hi=1.1,
                         with_grad=True)
    args = (w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)
    out = msda_forward(*args)
    gv, gl, ga = msda_backward(*args, grad_out=w.grad_out)
    rng = np.random.default_rng(1)
    pn, pq, pm = rng.integers(0, 2, 20), rng.integers(0, 13, 20), rng.integers(0, 3, 20)
    np.testing.assert_allclose(msda_forward(*args, pairs=(pn, pq, pm)), out[pn, pq, pm], atol=1e-14)
    _, gl_p, ga_p = msda_backward(*args, grad_out=w.grad_out, pairs=(pn, pq, pm), with_grad_value=False)
    np.testing.assert_allclose(gl_p, gl[pn, pq, pm], atol=1e-14)
    np.testing.assert_allclose(ga_p, ga[pn, pq, pm], atol=1e-14)
    S = w.value.shape[1]
    rn, rs, rm = rng.integers(0, 2, 30), rng.integers(0, S, 30), rng.integers(0, 3, 30)
    rn[1], rs[1], rm[1] = rn[0], rs[0], rm[0]  # a duplicate request
    got = msda_grad_value_rows(*args, w.grad_out, (rn, rs, rm))
    np.testing.assert_allclose(got, gv[rn, rs, rm], atol=1e-13)


def test_level_starts_layout():
    starts, S = level_starts(((100, 167), (50, 84), (25, 42), (13, 21)))
    assert list(starts) == [0, 16700, 20900, 21950] and S == 22223


# --- the fused step before the core (softmax of logits, locations from references) -------------

def test_softmax_weights_match_library_softmax():
    scipy_special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(91)
    z = rng.standard_normal((2, 5, 3, 4, 2)) * 3
    A = softmax_weights(z)
    ref = scipy_special.softmax(z.reshape(2, 5, 3, 8), axis=-1).reshape(z.shape)
    np.testing.assert_allclose(A, ref, atol=1e-15)
    np.testing.assert_allclose(A.sum(axis=(-2, -1)), 1.0, atol=1e-14)
    np.testing.assert_allclose(softmax_weights(z + 7.0), A, atol=1e-15)


def test_fused_locations_closed_forms():
    shapes = np.array([[8, 16], [4, 8]])
    # reference at a pixel centre of level 0 plus an integer pixel offset lands on
    # a pixel centre of that level
    ref = np.array([[[(5 + 0.5) / 16, (2 + 0.5) / 8]]], dtype=np.float32)
    off = np.zeros((1, 1, 1, 2, 1, 2), dtype=np.float32)
    off[0, 0, 0, 0, 0] = (3.0, -1.0)
    loc = fused_locations(ref, off, shapes)
    assert loc[0, 0, 0, 0, 0, 0] * 16 - 0.5 == 8.0 and loc[0, 0, 0, 0, 0, 1] * 8 - 0.5 == 1.0
    # a zero offset reads the reference point itself at every level
    np.testing.assert_array_equal(loc[0, 0, 0, 1, 0], ref[0, 0])
    # boxes: zero offsets give the centre, offset (1, -1) moves by (w, -h)
    box = np.array([[[0.5, 0.25, 0.125, 0.5]]], dtype=np.float32)
    offb = np.zeros((1, 1, 1, 1, 2, 2), dtype=np.float32)
    offb[0, 0, 0, 0, 1] = (1.0, -1.0)
    locb = fused_locations(box, offb, shapes[:1])
    np.testing.assert_array_equal(locb[0, 0, 0, 0, 0], [0.5, 0.25])
    np.testing.assert_array_equal(locb[0, 0, 0, 0, 1], [0.625, -0.25])


@pytest.mark.parametrize("ref_dim", [2, 4])
def test_fused_backward_finite_differences(ref_dim):
    rng = np.random.default_rng(95 + ref_dim)
    shapes = np.array([[6, 8], [3, 5]])
    starts = np.array([0, 48])
    N, Lq, M, D, L, K = 1, 4, 2, 3, 2, 2
    value = rng.standard_normal((N, 63, M, D))
    if ref_dim == 2:
        ref = rng.uniform(0.1, 0.9, (N, Lq, 2))
        off = rng.standard_normal((N, Lq, M, L, K, 2)) * 1.5
    else:
        ref = np.concatenate([rng.uniform(0.3, 0.7, (N, Lq, 2)), rng.uniform(0.1, 0.4, (N, Lq, 2))], -1)
        off = rng.uniform(-0.5, 0.5, (N, Lq, M, L, K, 2))
    logits = rng.standard_normal((N, Lq, M, L, K))
    G = rng.standard_normal((N, Lq, M, D))
    kw = dict(round_coords=False, exact_locations=True)
    _, g_off, g_log, g_ref = msda_fused_backward(value, shapes, starts, ref, off, logits, G, **kw)

    def f(ref=ref, off=off, logits=logits):
        return (msda_fused_forward(value, shapes, starts, ref, off, logits, **kw) * G).sum()

    h = 1e-6
    for idx in [(0, 1, 0, 1, 0), (0, 3, 1, 0, 1), (0, 0, 1, 1, 1)]:
        zp, zm = logits.copy(), logits.copy()
        zp[idx] += h
        zm[idx] -= h
        assert abs((f(logits=zp) - f(logits=zm)) / (2 * h) - g_log[idx]) < 1e-6
    checked = 0
    for idx in np.ndindex(*off.shape):
        op, om = off.copy(), off.copy()
        op[idx] += h
        om[idx] -= h
        fd = (f(off=op) - f(off=om)) / (2 * h)
        if abs(fd - g_off[idx]) > 1e-5 * max(1.0, abs(fd)):
            # central differences straddle a kink of the bilinear read
            x = fused_locations(ref, off, shapes, exact=True)[idx] * shapes[idx[3]][1 - idx[5]] - 0.5
            assert abs(x - np.round(x)) < 1e-4, (idx, fd, g_off[idx])
        else:
            checked += 1
    assert checked > 40
    for idx in np.ndindex(*ref.shape):
        rp, rm = ref.copy(), ref.copy()
        rp[idx] += h
        rm[idx] -= h
        fd = (f(ref=rp) - f(ref=rm)) / (2 * h)
        assert abs(fd - g_ref[idx]) < 1e-4 * max(1.0, abs(fd)), (idx, fd, g_ref[idx])


def test_box_locations_are_one_rounding_of_the_fused_multiply_add():
    """Reading R11 for boxes: loc = nearest binary32 of centre + offset * size,
    checked against exact rationals, including inputs where rounding the
    float64 sum to binary32 would round twice the wrong way."""
    rng = np.random.default_rng(97)
    xs, ys = [], []
    # centre 1, size * offset just above 2^-24: the exact sum lies just above
    # the binary32 halfway point 1 + 2^-24, its float64 rounding on it
    for x in rng.uniform(1.0, 2.0, 20000).astype(np.float32):
        y = np.float32(2.0 ** -24 / float(x))
        while Fraction(float(x)) * Fraction(float(y)) <= Fraction(1, 2 ** 24):
            y = np.nextafter(y, np.float32(1))
        ex = 1 + Fraction(float(x)) * Fraction(float(y))
        if float(ex) == 1 + 2.0 ** -24:
            xs.append(x)
            ys.append(y)
        if len(xs) == 16:
            break
    assert len(xs) == 16
    n = len(xs)
    box = np.zeros((1, n, 4), dtype=np.float32)
    box[0, :, 0] = 1.0
    box[0, :, 1] = rng.uniform(-1, 1, n)
    box[0, :, 2] = ys
    box[0, :, 3] = rng.uniform(0.01, 1, n)
    off = np.zeros((1, n, 1, 1, 1, 2), dtype=np.float32)
    off[0, :, 0, 0, 0, 0] = xs
    off[0, :, 0, 0, 0, 1] = rng.uniform(-3, 3, n)
    # plus random boxes
    box2 = rng.uniform(0.0, 1.0, (1, 64, 4)).astype(np.float32)
    off2 = (rng.standard_normal((1, 64, 1, 1, 1, 2)) * 2).astype(np.float32)
    shapes = np.array([[4, 4]])
    for b, o in ((box, off), (box2, off2)):
        got = fused_locations(b, o, shapes)
        for q in range(b.shape[1]):
            for c in range(2):
                ex = Fraction(float(b[0, q, c])) + Fraction(float(o[0, q, 0, 0, 0, c])) * Fraction(float(b[0, q, 2 + c]))
                assert got[0, q, 0, 0, 0, c] == round_fraction_to_f32(ex), (q, c)
    # the halfway cases do round up, away from the float64 sum's tie
    assert np.all(fused_locations(box, off, shapes)[0, :, 0, 0, 0, 0] == np.float32(1 + 2.0 ** -23))


@pytest.mark.parametrize("ref_dim", [2, 4])
def test_fused_backward_query_subset_agrees_with_full(ref_dim):
    rng = np.random.default_rng(99 + ref_dim)
    shapes = np.array([[6, 8], [3, 5]])
    starts = np.array([0, 48])
    N, Lq, M, D, L, K = 2, 5, 3, 4, 2, 2
    value = rng.standard_normal((N, 63, M, D))
    ref = rng.uniform(0.2, 0.8, (N, Lq, ref_dim)).astype(np.float32)
    off = (rng.standard_normal((N, Lq, M, L, K, 2)) * (1.5 if ref_dim == 2 else 0.3)).astype(np.float32)
    logits = rng.standard_normal((N, Lq, M, L, K)).astype(np.float32)
    G = rng.standard_normal((N, Lq, M, D))
    _, go, gz, gr = msda_fused_backward(value, shapes, starts, ref, off, logits, G)
    qn, qq = np.array([1, 0, 1]), np.array([4, 2, 0])
    gv, go_s, gz_s, gr_s = msda_fused_backward(value, shapes, starts, ref, off, logits, G, queries=(qn, qq))
    assert gv is None
    np.testing.assert_allclose(go_s, go[qn, qq], rtol=0, atol=1e-12)
    np.testing.assert_allclose(gz_s, gz[qn, qq], rtol=0, atol=1e-12)
    np.testing.assert_allclose(gr_s, gr[qn, qq], rtol=0, atol=1e-12)


@pytest.mark.parametrize("ref_dim", [2, 4])
def test_fused_non_finite_offsets_act_as_far_outside(ref_dim):
    """Reading R2 for formed locations: an offset that is NaN or infinite puts
    its sample outside every level, so every result equals the one with that
    offset replaced by a finite offset far outside the map (its weight still
    enters the head's softmax); its own offset gradient is zero."""
    rng = np.random.default_rng(111 + ref_dim)
    shapes = np.array([[6, 8], [3, 5]])
    starts = np.array([0, 48])
    N, Lq, M, D, L, K = 2, 4, 2, 3, 2, 3
    value = rng.standard_normal((N, 63, M, D))
    ref = rng.uniform(0.3, 0.7, (N, Lq, ref_dim)).astype(np.float32)
    if ref_dim == 4:
        ref[..., 2:] = rng.uniform(0.1, 0.3, (N, Lq, 2))
    off = (rng.standard_normal((N, Lq, M, L, K, 2)) * (1.5 if ref_dim == 2 else 0.3)).astype(np.float32)
    logits = rng.standard_normal((N, Lq, M, L, K)).astype(np.float32)
    G = rng.standard_normal((N, Lq, M, D))
    bad, far = off.copy(), off.copy()
    for (n, q, m, l, k, c), v in zip([(0, 1, 0, 0, 2, 0), (1, 3, 1, 1, 0, 1), (0, 0, 1, 1, 1, 0)],
                                     [np.nan, np.inf, -np.inf]):
        bad[n, q, m, l, k, c] = v
        # far outside: 1e4 level pixels (points) or 1e4 box sizes (boxes) away
        far[n, q, m, l, k, c] = 1e4 if v != -np.inf else -1e4
    out_b = msda_fused_forward(value, shapes, starts, ref, bad, logits)
    out_f = msda_fused_forward(value, shapes, starts, ref, far, logits)
    np.testing.assert_array_equal(out_b, out_f)
    res_b = msda_fused_backward(value, shapes, starts, ref, bad, logits, G)
    res_f = msda_fused_backward(value, shapes, starts, ref, far, logits, G)
    for a, b in zip(res_b, res_f):
        assert np.all(np.isfinite(a))
        np.testing.assert_array_equal(a, b)
    assert res_b[1][0, 1, 0, 0, 2].tolist() == [0.0, 0.0]


# --- deformable groups (reading R12) ---------------------------------------------------------

def test_groups_of_one_head_are_the_core():
    w = uniform_workload(N=1, shapes=((6, 7), (3, 4)), Lq=9, M=3, D=4, K=2, seed=120, with_grad=True)
    args = (w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)
    np.testing.assert_array_equal(msda_grouped_forward(*args), msda_forward(*args))
    for a, b in zip(msda_grouped_backward(*args, w.grad_out), msda_backward(*args, w.grad_out)):
        np.testing.assert_array_equal(a, b)


def test_grouped_heads_share_their_group_samples():
    """With equal value channels in every head of a group, the heads of the group
    return equal outputs; with the group's channels split across heads, the
    heads' outputs add up to the core's output on the summed channels."""
    rng = np.random.default_rng(121)
    shapes = np.array([[5, 6], [3, 3]])
    starts = np.array([0, 30])
    N, Lq, M, G, D, L, K = 2, 7, 6, 2, 3, 2, 3
    base = rng.standard_normal((N, 39, G, D))
    value = np.repeat(base, M // G, axis=2)
    loc = rng.uniform(-0.1, 1.1, (N, Lq, G, L, K, 2))
    attn = rng.uniform(0, 1, (N, Lq, G, L, K))
    out = msda_grouped_forward(value, shapes, starts, loc, attn).reshape(N, Lq, G, M // G, D)
    for h in range(1, M // G):
        np.testing.assert_allclose(out[:, :, :, h], out[:, :, :, 0], atol=1e-12)
    np.testing.assert_allclose(out[:, :, :, 0], msda_forward(base, shapes, starts, loc, attn), atol=1e-12)
    split = rng.standard_normal((N, 39, M, D))
    tot = split.reshape(N, 39, G, M // G, D).sum(axis=3)
    o2 = msda_grouped_forward(split, shapes, starts, loc, attn).reshape(N, Lq, G, M // G, D).sum(axis=3)
    np.testing.assert_allclose(o2, msda_forward(tot, shapes, starts, loc, attn), atol=1e-12)


def test_grouped_backward_finite_differences_and_adjoint():
    rng = np.random.default_rng(122)
    shapes = np.array([[6, 8], [3, 5]])
    starts = np.array([0, 48])
    N, Lq, M, G, D, L, K = 1, 4, 4, 2, 3, 2, 2
    value = rng.standard_normal((N, 63, M, D))
    loc = rng.uniform(0.05, 0.95, (N, Lq, G, L, K, 2))
    attn = rng.uniform(0, 1, (N, Lq, G, L, K))
    Gr = rng.standard_normal((N, Lq, M, D))
    kw = dict(round_coords=False)
    gv, gl, ga = msda_grouped_backward(value, shapes, starts, loc, attn, Gr, **kw)

    def f(loc=loc, attn=attn):
        return (msda_grouped_forward(value, shapes, starts, loc, attn, **kw) * Gr).sum()

    h = 1e-6
    for idx in [(0, 0, 0, 0, 0), (0, 3, 1, 1, 1), (0, 2, 1, 0, 1)]:
        ap, am = attn.copy(), attn.copy()
        ap[idx] += h
        am[idx] -= h
        assert abs((f(attn=ap) - f(attn=am)) / (2 * h) - ga[idx]) < 1e-6
        for c in range(2):
            lp, lm = loc.copy(), loc.copy()
            lp[idx + (c,)] += h
            lm[idx + (c,)] -= h
            fd = (f(loc=lp) - f(loc=lm)) / (2 * h)
            assert abs(fd - gl[idx + (c,)]) < 1e-4 * max(1.0, abs(fd)), (idx, c, fd, gl[idx + (c,)])
    # out is linear in value: <G, out> = <grad_value, value>
    assert abs(f() - (gv * value).sum()) < 1e-9 * max(1.0, abs(f()))
