"""Parity of the fused entry points (softmax of logits and location formation
inside the kernels) with the fp64 oracle, through the C ABI.

Tolerances follow the sampling core's: out, grad_value and grad_logits
max-abs <= 1e-5 (float32 arithmetic; bf16 out within one bf16 ulp); offset
gradients in pixel units of their level (points: they already are; boxes:
divided by (w * W_l, h * H_l)) max-abs <= 1e-5. grad_ref sums grad_loc over the
M*L*K samples of a query, so its bound is the sum of those samples' bounds:
1e-5 * sum W_l (x) or H_l (y) for the centre, and that sum weighted by |offset|
for the box size.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import msda_fused_backward, msda_fused_forward, msda_grad_value_rows  # noqa: E402
from oracle import fused_locations, softmax_weights  # noqa: E402
from tests.gpu_util import (assert_f32, assert_normwise, bf16_ulp, fused_device_inputs,  # noqa: E402
                            fused_pixel_offsets, fused_ref_bound, max_abs, note, to_f64)
import scale_deformable_attention_msda_amd as msda  # noqa: E402
from workloads import COCO_LEVELS, fused_workload  # noqa: E402

pytestmark = pytest.mark.gpu

SMALL_LEVELS = ((20, 34), (10, 17), (5, 9), (3, 5))


def _oracle_args(w):
    return (w.value, w.spatial_shapes, w.level_start, w.ref, w.offsets, w.logits)


def _check_out(w, got, ref):
    if w.dtype == "f32":
        assert_f32("out", got, ref)
        return
    assert_normwise("out", got, ref)
    bad = np.abs(got - ref) > bf16_ulp(ref) + 1e-5
    assert not bad.any(), f"{bad.sum()} bf16 outputs beyond one ulp; worst {max_abs(got, ref):.3e}"


def _check_grads(w, got, ref, ref_rows, off_rows, check_gv=True):
    gv, go, gz, gr = got
    rgv, rgo, rgz, rgr = ref
    if check_gv:
        assert_f32("grad_value", gv, rgv)
    assert_f32("grad_logits", gz, rgz)
    assert_f32("grad_offsets (pixel units)", fused_pixel_offsets(w, go, ref_rows), fused_pixel_offsets(w, rgo, ref_rows))
    if gr is not None:
        assert np.all(np.isfinite(gr)), "grad_ref: non-finite values"
        excess = np.abs(np.asarray(gr, np.float64) - rgr) - fused_ref_bound(w, off_rows)
        assert excess.max() <= 0, f"grad_ref beyond its bound by {excess.max():.3e}"


def _gpu_fused_backward(w, **kw):
    value, ref, off, logits, g = fused_device_inputs(w)
    res = msda.msda_fused_backward(value, w.spatial_shapes, w.level_start, ref, off, logits, g, **kw)
    torch.cuda.synchronize()
    return tuple(None if t is None else to_f64(t) for t in res)


# ------------------------------------------------------------------ forward

@pytest.mark.parametrize("kind,ref_dim,dtype", [("encoder", 2, "f32"), ("encoder", 2, "bf16")])
def test_fused_forward_encoder_small_maps_full(kind, ref_dim, dtype):
    w = fused_workload(kind, N=2, shapes=SMALL_LEVELS, ref_dim=ref_dim, dtype=dtype, seed=31)
    note(f"fused forward {kind} ref_dim={ref_dim} {dtype} small maps")
    value, ref, off, logits, _ = fused_device_inputs(w)
    out = to_f64(msda.msda_fused_forward(value, w.spatial_shapes, w.level_start, ref, off, logits))
    torch.cuda.synchronize()
    _check_out(w, out, msda_fused_forward(*_oracle_args(w)))


@pytest.mark.parametrize("ref_dim,dtype", [(2, "bf16"), (4, "bf16"), (2, "f32"), (4, "f32")])
def test_fused_forward_decoder_full_config(ref_dim, dtype):
    w = fused_workload("decoder", N=2, Lq=300, ref_dim=ref_dim, dtype=dtype, seed=32 + ref_dim)
    note(f"fused forward decoder N=2 Lq=300 COCO levels ref_dim={ref_dim} {dtype}")
    value, ref, off, logits, _ = fused_device_inputs(w)
    out = to_f64(msda.msda_fused_forward(value, w.spatial_shapes, w.level_start, ref, off, logits))
    torch.cuda.synchronize()
    _check_out(w, out, msda_fused_forward(*_oracle_args(w)))


# ----------------------------------------------------------------- backward

@pytest.mark.parametrize("K", [4, 8])
def test_fused_backward_encoder_small_maps_full(K):
    w = fused_workload("encoder", N=2, shapes=SMALL_LEVELS, K=K, seed=40 + K, with_grad=True)
    note(f"fused backward encoder points K={K} f32 small maps")
    got = _gpu_fused_backward(w)
    ref = msda_fused_backward(*_oracle_args(w), w.grad_out)
    _check_grads(w, got, ref, w.ref, w.offsets)


@pytest.mark.parametrize("L,K,kind,ref_dim", [(4, 16, "encoder", 2), (2, 2, "encoder", 2), (1, 2, "encoder", 2),
                                               (4, 4, "decoder", 4)])
def test_fused_backward_dense_route_point_counts(L, K, kind, ref_dim):
    """The tile-sorted route, where the counting pass forms each sample's
    location and softmax weight itself (L*K a power of two up to 64: a pair's
    logits in segments of 2 to 64 lanes, a whole wave at 64), for reference
    points and for boxes (300 box queries on small maps)."""
    shapes = SMALL_LEVELS[:L]
    kw = dict(Lq=300) if kind == "decoder" else {}
    w = fused_workload(kind, N=2, shapes=shapes, K=K, ref_dim=ref_dim, seed=45 + L + K, with_grad=True, **kw)
    tiles = sum(((h + 7) // 8) * ((wd + 7) // 8) for h, wd in shapes)
    assert w.dims["Lq"] * L * K >= 32 * tiles  # the dense route
    note(f"fused backward dense route {kind} ref_dim={ref_dim} L={L} K={K}")
    got = _gpu_fused_backward(w)
    ref = msda_fused_backward(*_oracle_args(w), w.grad_out)
    _check_grads(w, got, ref, w.ref, w.offsets)


@pytest.mark.parametrize("ref_dim,dtype", [(2, "f32"), (4, "f32"), (4, "bf16")])
def test_fused_backward_decoder_full_config(ref_dim, dtype):
    w = fused_workload("decoder", N=2, Lq=300, ref_dim=ref_dim, dtype=dtype, seed=50 + ref_dim, with_grad=True)
    note(f"fused backward decoder N=2 Lq=300 ref_dim={ref_dim} {dtype}")
    got = _gpu_fused_backward(w)
    ref = msda_fused_backward(*_oracle_args(w), w.grad_out)
    # bf16 inputs are exact values and the arithmetic is float32: same bar
    _check_grads(w, got, ref, w.ref, w.offsets)


@pytest.mark.parametrize("ref_dim,dtype", [(2, "f32"), (4, "f32"), (2, "bf16")])
def test_fused_hot_shapes_with_odd_point_counts(ref_dim, dtype):
    """40000 pairs of D=32 heads select the launch shapes whose sample
    pass batches two samples' corner loads per lane; L*K = 9 leaves the last
    batch of each chunk half empty and takes the softmax from per-pair
    statistics (L*K not a power of two)."""
    w = fused_workload("decoder", N=1, shapes=((24, 40), (12, 20), (6, 10)), Lq=5000, M=8, D=32, K=3,
                       ref_dim=ref_dim, dtype=dtype, seed=110 + ref_dim, with_grad=True)
    note(f"fused hot launch shapes with L*K=9, ref_dim={ref_dim}, {dtype}, 40000 pairs")
    value, ref_t, off, logits, _ = fused_device_inputs(w)
    out = to_f64(msda.msda_fused_forward(value, w.spatial_shapes, w.level_start, ref_t, off, logits))
    _check_out(w, out, msda_fused_forward(*_oracle_args(w)))
    got = _gpu_fused_backward(w)
    ref = msda_fused_backward(*_oracle_args(w), w.grad_out)
    _check_grads(w, got, ref, w.ref, w.offsets)


def test_fused_backward_encoder_full_size_sampled():
    w = fused_workload("encoder", N=2, shapes=COCO_LEVELS, K=4, seed=60, with_grad=True)
    d = w.dims
    note("fused backward encoder full size N=2 S=Lq=22223 M=8 D=32 K=4 f32")
    value, ref, off, logits, g = fused_device_inputs(w)
    gv, go, gz, gr = msda.msda_fused_backward(value, w.spatial_shapes, w.level_start, ref, off, logits, g)
    out = msda.msda_fused_forward(value, w.spatial_shapes, w.level_start, ref, off, logits)
    torch.cuda.synchronize()
    rng = np.random.default_rng(61)
    qn = rng.integers(0, d["N"], 800)
    qq = rng.integers(0, d["Lq"], 800)
    qn[0], qq[0], qn[1], qq[1] = 0, 0, d["N"] - 1, d["Lq"] - 1
    _, rgo, rgz, rgr = msda_fused_backward(*_oracle_args(w), w.grad_out, queries=(qn, qq))
    idx = (torch.as_tensor(qn), torch.as_tensor(qq))
    _check_grads(w, (None, to_f64(go[idx]), to_f64(gz[idx]), to_f64(gr[idx])), (None, rgo, rgz, rgr),
                 w.ref[qn, qq], w.offsets[qn, qq], check_gv=False)
    # grad_value rows, through the oracle's core with the oracle's own locations and weights
    rs = rng.integers(0, d["S"], 300)
    rm = rng.integers(0, d["M"], 300)
    rn = rng.integers(0, d["N"], 300)
    loc = fused_locations(w.ref, w.offsets, w.spatial_shapes)
    A = softmax_weights(w.logits)
    rgv = msda_grad_value_rows(w.value, w.spatial_shapes, w.level_start, loc, A, w.grad_out, (rn, rs, rm))
    assert_f32("grad_value", to_f64(gv[torch.as_tensor(rn), torch.as_tensor(rs), torch.as_tensor(rm)]), rgv)
    # adjoint identity over the whole tensors: <G, out> = <grad_value, value>
    lhs = float((g.double() * out.double()).sum())
    rv = float((gv.double() * value.double()).sum())
    scale = float((g.double().abs() * out.double().abs()).sum())
    assert abs(lhs - rv) <= 1e-6 * scale, (lhs, rv, scale)
    # the logit gradients of one head sum to zero (softmax is shift-invariant)
    assert float(gz.double().sum(dim=(-2, -1)).abs().max()) <= 1e-5


def test_fused_backward_without_grad_ref_and_determinism():
    w = fused_workload("decoder", N=2, Lq=300, ref_dim=4, dtype="f32", seed=70, with_grad=True)
    note("fused backward, grad_ref skipped vs computed, repeated calls")
    a = _gpu_fused_backward(w)
    b = _gpu_fused_backward(w, need_grad_ref=False)
    assert b[3] is None
    # grad_offsets, grad_logits and grad_ref do not depend on the order of work
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[2], b[2])
    c = _gpu_fused_backward(w)
    np.testing.assert_array_equal(a[3], c[3])
    assert max_abs(a[0], b[0]) <= 1e-6


@pytest.mark.parametrize("L,K,D,dtype", [(16, 16, 8, "f32"), (3, 5, 5, "f32"), (2, 3, 100, "f32"),
                                         (2, 4, 6, "bf16"), (1, 1, 64, "f32")])
def test_fused_shapes(L, K, D, dtype):
    shapes = [(9, 13), (5, 7), (3, 4), (2, 2)] * 4
    w = fused_workload("decoder", N=1, shapes=shapes[:L], Lq=37, M=3, D=D, K=K, ref_dim=4 if L % 2 else 2,
                       dtype=dtype, seed=80 + L + K, with_grad=True)
    note(f"fused shapes L={L} K={K} D={D} {dtype}")
    value, ref, off, logits, _ = fused_device_inputs(w)
    out = to_f64(msda.msda_fused_forward(value, w.spatial_shapes, w.level_start, ref, off, logits))
    torch.cuda.synchronize()
    _check_out(w, out, msda_fused_forward(*_oracle_args(w)))
    got = _gpu_fused_backward(w)
    _check_grads(w, got, msda_fused_backward(*_oracle_args(w), w.grad_out), w.ref, w.offsets)


def test_fused_nan_logit_poisons_only_its_head():
    w = fused_workload("decoder", N=1, shapes=((6, 8), (3, 4)), Lq=5, M=2, D=8, K=3, seed=90)
    w.logits[0, 2, 1, 0, 1] = np.nan
    note("fused forward with one NaN logit")
    value, ref, off, logits, _ = fused_device_inputs(w)
    out = to_f64(msda.msda_fused_forward(value, w.spatial_shapes, w.level_start, ref, off, logits))
    torch.cuda.synchronize()
    ref_out = msda_fused_forward(*_oracle_args(w))
    assert np.array_equal(np.isnan(out), np.isnan(ref_out))
    assert np.isnan(out[0, 2, 1]).all() and np.isfinite(np.delete(out.reshape(-1, 8), 5, axis=0)).all()
    keep = ~np.isnan(ref_out)
    assert_f32("out", out[keep], ref_out[keep])


@pytest.mark.parametrize("ref_dim", [2, 4])
def test_fused_non_finite_offsets(ref_dim):
    """NaN and infinite offsets give non-finite locations, which lie outside
    every level: those samples add nothing and get zero offset gradients, while
    their weights still take part in the head's softmax (the oracle receives the
    same offsets)."""
    w = fused_workload("decoder", N=2, shapes=((12, 16), (6, 8)), Lq=30, M=4, D=8, K=3, ref_dim=ref_dim,
                       seed=96 + ref_dim, with_grad=True)
    rng = np.random.default_rng(97)
    flat = w.offsets.reshape(-1, 2)
    pick = rng.random(flat.shape[0]) < 0.15
    bad = np.array([np.nan, np.inf, -np.inf], np.float32)
    flat[pick, rng.integers(0, 2, size=int(pick.sum()))] = bad[rng.integers(0, 3, size=int(pick.sum()))]
    note(f"fused forward and backward with non-finite offsets, ref_dim={ref_dim}")
    value, ref_t, off, logits, g = fused_device_inputs(w)
    out = to_f64(msda.msda_fused_forward(value, w.spatial_shapes, w.level_start, ref_t, off, logits))
    gv, go, gz, gr = (to_f64(t) for t in msda.msda_fused_backward(value, w.spatial_shapes, w.level_start, ref_t,
                                                                    off, logits, g))
    torch.cuda.synchronize()
    for t in (out, gv, go, gz, gr):
        assert np.all(np.isfinite(t))
    assert not go.reshape(-1, 2)[pick].any()
    _check_out(w, out, msda_fused_forward(*_oracle_args(w)))
    finite = np.isfinite(w.offsets).all(axis=-1, keepdims=True)
    rgv, rgo, rgz, rgr = msda_fused_backward(*_oracle_args(w), w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_logits", gz, rgz)
    assert_f32("grad_offsets (pixel units)", fused_pixel_offsets(w, np.where(finite, go, 0.0), w.ref),
               fused_pixel_offsets(w, np.where(finite, rgo, 0.0), w.ref))
    excess = np.abs(gr - rgr) - fused_ref_bound(w, np.where(finite, w.offsets, 0.0))
    assert excess.max() <= 0, f"grad_ref beyond its bound by {excess.max():.3e}"


def test_fused_autograd_wrapper():
    w = fused_workload("decoder", N=1, shapes=((6, 8), (3, 4)), Lq=10, M=2, D=8, K=2, ref_dim=4, seed=95,
                       with_grad=True)
    value, ref, off, logits, g = fused_device_inputs(w)
    for t in (value, ref, off, logits):
        t.requires_grad_(True)
    note("fused autograd wrapper")
    out = msda.msda_fused_sample(value, w.spatial_shapes, w.level_start, ref, off, logits)
    out.backward(g)
    gv, go, gz, gr = msda.msda_fused_backward(value.detach(), w.spatial_shapes, w.level_start, ref.detach(),
                                              off.detach(), logits.detach(), g)
    torch.cuda.synchronize()
    assert torch.allclose(value.grad, gv, atol=1e-6)
    assert torch.equal(off.grad, go) and torch.equal(logits.grad, gz) and torch.equal(ref.grad, gr)
