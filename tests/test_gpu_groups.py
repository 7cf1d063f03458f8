"""Parity of the deformable-group entry points with the fp64 oracle, through
the C ABI. Tolerances as for the sampling core: float32 max-abs <= 1e-5 (the
location gradient in pixel units of its level), bf16 outputs within one bf16
ulp. A group's location and weight gradients sum over its M/G heads and are
still held to the per-head 1e-5 (their measured errors stay below it); only the
reference gradient, a sum over a query's samples, takes the sum of their
per-sample bounds."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import (msda_backward, msda_forward, msda_fused_backward, msda_fused_forward,  # noqa: E402
                    msda_grouped_backward, msda_grouped_forward)
from tests.gpu_util import (assert_f32, assert_grad_loc, assert_normwise, bf16_ulp, device_inputs,  # noqa: E402
                            max_abs, note, to_f64)
import scale_deformable_attention_msda_amd as msda  # noqa: E402
from workloads import decoder_workload, encoder_workload, fused_workload  # noqa: E402

pytestmark = pytest.mark.gpu

SMALL_LEVELS = ((20, 34), (10, 17), (5, 9), (3, 5))


def _args(w):
    return (w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)


def _check_out(w, got, ref):
    if w.dtype == "f32":
        assert_f32("out", got, ref)
    else:
        assert_normwise("out", got, ref)
        bad = np.abs(got - ref) > bf16_ulp(ref) + 1e-5
        assert not bad.any(), f"{bad.sum()} bf16 outputs beyond one ulp; worst {max_abs(got, ref):.3e}"


@pytest.mark.parametrize("G,dtype", [(2, "f32"), (1, "f32"), (4, "bf16")])
def test_grouped_forward_small_maps_full(G, dtype):
    w = encoder_workload(N=2, shapes=SMALL_LEVELS, M=8, D=32, K=4, dtype=dtype, seed=130 + G, groups=G)
    note(f"grouped forward encoder small maps G={G} {dtype}")
    value, loc, attn, _ = device_inputs(w)
    out = to_f64(msda.msda_grouped_forward(value, w.spatial_shapes, w.level_start, loc, attn))
    torch.cuda.synchronize()
    _check_out(w, out, msda_grouped_forward(*_args(w)))


@pytest.mark.parametrize("G,K", [(2, 4), (4, 8), (1, 4)])
def test_grouped_backward_small_maps_full(G, K):
    w = encoder_workload(N=2, shapes=SMALL_LEVELS, M=8, D=32, K=K, seed=140 + G + K, groups=G, with_grad=True)
    note(f"grouped backward encoder small maps G={G} K={K} f32")
    value, loc, attn, g = device_inputs(w)
    gv, gl, ga = (to_f64(t) for t in msda.msda_grouped_backward(value, w.spatial_shapes, w.level_start, loc,
                                                                  attn, g))
    torch.cuda.synchronize()
    rgv, rgl, rga = msda_grouped_backward(*_args(w), w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga, atol=1e-5)
    assert_grad_loc(gl, rgl, w.spatial_shapes, atol=1e-5)


@pytest.mark.parametrize("G,dtype", [(2, "bf16"), (1, "f32")])
def test_grouped_decoder_full_config(G, dtype):
    w = decoder_workload(N=2, Lq=300, M=8, D=32, K=4, dtype=dtype, seed=150 + G, groups=G, with_grad=True)
    note(f"grouped decoder N=2 Lq=300 G={G} {dtype} forward and backward")
    value, loc, attn, g = device_inputs(w)
    out = to_f64(msda.msda_grouped_forward(value, w.spatial_shapes, w.level_start, loc, attn))
    gv, gl, ga = (to_f64(t) for t in msda.msda_grouped_backward(value, w.spatial_shapes, w.level_start, loc,
                                                                  attn, g))
    torch.cuda.synchronize()
    _check_out(w, out, msda_grouped_forward(*_args(w)))
    rgv, rgl, rga = msda_grouped_backward(*_args(w), w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga, atol=1e-5)
    assert_grad_loc(gl, rgl, w.spatial_shapes, atol=1e-5)


def test_groups_equal_to_heads_match_the_core_bitwise():
    w = encoder_workload(N=1, shapes=SMALL_LEVELS, M=8, D=32, K=4, seed=160, with_grad=True)
    note("grouped entry points with G = M against the core entry points")
    value, loc, attn, g = device_inputs(w)
    a = msda.msda_grouped_forward(value, w.spatial_shapes, w.level_start, loc, attn)
    b = msda.msda_forward(value, w.spatial_shapes, w.level_start, loc, attn)
    _, gl1, ga1 = msda.msda_grouped_backward(value, w.spatial_shapes, w.level_start, loc, attn, g)
    _, gl2, ga2 = msda.msda_backward(value, w.spatial_shapes, w.level_start, loc, attn, g)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(gl1, gl2) and torch.equal(ga1, ga2)
    assert_f32("out", to_f64(a), msda_forward(*_args(w)))
    _, rgl, rga = msda_backward(*_args(w), w.grad_out, with_grad_value=False)
    assert_f32("grad_attn", to_f64(ga1), rga)


@pytest.mark.parametrize("kind,ref_dim,G", [("encoder", 2, 2), ("decoder", 4, 4)])
def test_fused_inputs_with_groups(kind, ref_dim, G):
    shapes = SMALL_LEVELS if kind == "encoder" else ((20, 34), (10, 17), (5, 9), (3, 5))
    w = fused_workload(kind, N=2, shapes=shapes, Lq=60, M=8, D=32, K=4, ref_dim=ref_dim, seed=170 + G,
                       groups=G, with_grad=True)
    note(f"fused inputs with groups: {kind} ref_dim={ref_dim} G={G}")
    dev = "cuda:0"
    value = torch.from_numpy(w.value).to(dev)
    ref, off, z, g = (torch.from_numpy(a).to(dev) for a in (w.ref, w.offsets, w.logits, w.grad_out))
    out = to_f64(msda.msda_fused_forward(value, w.spatial_shapes, w.level_start, ref, off, z))
    gv, go, gz, gr = (to_f64(t) for t in msda.msda_fused_backward(value, w.spatial_shapes, w.level_start, ref,
                                                                    off, z, g))
    torch.cuda.synchronize()
    args = (w.value, w.spatial_shapes, w.level_start, w.ref, w.offsets, w.logits)
    assert_f32("out", out, msda_fused_forward(*args))
    rgv, rgo, rgz, rgr = msda_fused_backward(*args, w.grad_out)
    heads = 8 // G
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_logits", gz, rgz, atol=1e-5)
    if ref_dim == 2:
        assert_f32("grad_offsets", go, rgo, atol=1e-5)
    else:
        ss = w.spatial_shapes
        size = np.stack([ss[:, 1], ss[:, 0]], axis=-1).reshape(-1, 1, 2).astype(np.float64)
        box = w.ref.astype(np.float64)[:, :, None, None, None, 2:]
        assert_f32("grad_offsets (pixel units)", go / (size * box), rgo / (size * box), atol=1e-5)
    # a query's reference gradient sums its G*L*K samples (bound: their pixel bounds in normalised units)
    bound = 1e-5 * heads * G * w.dims["K"] * float(ss_sum(w)) * (1 + (ref_dim == 4) * float(np.abs(w.offsets).max()))
    assert max_abs(gr, rgr) <= bound, (max_abs(gr, rgr), bound)


def ss_sum(w):
    return np.maximum(w.spatial_shapes[:, 0], w.spatial_shapes[:, 1]).sum()


def test_grouped_autograd_wrapper_matches_entry_points():
    w = decoder_workload(N=2, shapes=((12, 20), (6, 10)), Lq=40, M=8, D=16, K=3, dtype="f32", seed=190,
                         groups=2, with_grad=True)
    value, loc, attn, g = device_inputs(w)
    value.requires_grad_(True)
    loc.requires_grad_(True)
    attn.requires_grad_(True)
    note("grouped autograd wrapper, G=2")
    out = msda.msda_grouped_sample(value, w.spatial_shapes, w.level_start, loc, attn)
    out.backward(g)
    gv, gl, ga = msda.msda_grouped_backward(value.detach(), w.spatial_shapes, w.level_start, loc.detach(),
                                            attn.detach(), g)
    ref_out = msda.msda_grouped_forward(value.detach(), w.spatial_shapes, w.level_start, loc.detach(),
                                        attn.detach())
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), ref_out)
    assert torch.allclose(value.grad, gv, atol=1e-6)
    assert torch.equal(loc.grad, gl) and torch.equal(attn.grad, ga)
    _check_out(w, to_f64(out.detach()), msda_grouped_forward(*_args(w)))
