"""Seeded sweep of small random problems through the C ABI against the fp64
oracle: 1 to 5 levels (1x1 maps included), 1 to 8 points, odd and even channel
counts, queries from a handful to a few hundred (so both grad_value routes,
per-sample atomics and the tile sort, occur), float32 and bfloat16 values.
Each case runs the forward and the backward and compares every output
element, at the bars of the other parity tests. The same draw of sizes also
drives the fused entry points (reference points or boxes, random deformable
groups) and the grouped core; location, offset and logit gradients of a group
sum over its M/G heads and are held to the per-head 1e-5; the reference
gradient of a query sums all its samples and takes the sum of their bounds."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import (msda_backward, msda_forward, msda_fused_backward, msda_fused_forward,  # noqa: E402
                    msda_grouped_backward, msda_grouped_forward)
from tests.gpu_util import (assert_f32, assert_grad_loc, assert_normwise, bf16_ulp, device_inputs,  # noqa: E402
                            fused_device_inputs, fused_pixel_offsets, fused_ref_bound, gpu_backward,
                            gpu_forward, max_abs, note, to_f64)
import scale_deformable_attention_msda_amd as msda  # noqa: E402
from workloads import decoder_workload, fused_workload, uniform_workload  # noqa: E402

CHANNELS = (1, 2, 3, 4, 5, 7, 8, 12, 16, 24, 31, 32, 33, 48, 64, 96)


def _cases(count=32, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        L = int(rng.integers(1, 6))
        shapes = tuple((int(rng.integers(1, 25)), int(rng.integers(1, 25))) for _ in range(L))
        K = int(rng.integers(1, 9))
        cases.append(dict(N=int(rng.integers(1, 4)), shapes=shapes, M=int(rng.integers(1, 9)),
                          D=int(rng.choice(CHANNELS)), K=K, Lq=int(rng.integers(1, 300)),
                          dtype="bf16" if rng.random() < 0.3 else "f32", seed=5000 + i))
    return cases


CASES = _cases()


def _with_groups(cases, seed):
    """Each case with a deformable group count G drawn from the divisors of M."""
    rng = np.random.default_rng(seed)
    out = []
    for c in cases:
        divs = [g for g in range(1, c["M"] + 1) if c["M"] % g == 0]
        out.append(dict(c, G=int(rng.choice(divs)), ref_dim=int(rng.choice([2, 4]))))
    return out


FUSED_CASES = _with_groups(_cases(16, seed=2025), seed=7)
GROUPED_CASES = [{k: v for k, v in c.items() if k != "ref_dim"} for c in _with_groups(_cases(12, seed=2026), seed=8)]


def _case_id(c):
    extra = (f"-G{c['G']}" if "G" in c else "") + (f"-ref{c['ref_dim']}" if "ref_dim" in c else "")
    return f"N{c['N']}-L{len(c['shapes'])}-M{c['M']}-D{c['D']}-K{c['K']}-Lq{c['Lq']}-{c['dtype']}{extra}"


def _check_out(dtype, out, ref):
    if dtype == "f32":
        assert_f32("out", out, ref)
    else:
        assert_normwise("out", out, ref)
        slack = bf16_ulp(ref) + 1e-5
        assert not (np.abs(out - ref) > slack).any(), f"bf16 out beyond one ulp: {max_abs(out, ref):.3e}"


def _tiles(shapes):
    return sum(((h + 7) // 8) * ((w + 7) // 8) for h, w in shapes)


def test_sweep_covers_both_grad_value_routes():
    """The sweep holds problems on each side of the route threshold (fewer
    than 32 samples per tile and head go to per-sample atomics)."""
    dense = [c["Lq"] * len(c["shapes"]) * c["K"] >= 32 * _tiles(c["shapes"]) for c in CASES]
    assert any(dense) and not all(dense)


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_random_problem(case):
    w = uniform_workload(N=case["N"], shapes=case["shapes"], Lq=case["Lq"], M=case["M"], D=case["D"],
                         K=case["K"], dtype=case["dtype"], seed=case["seed"], lo=-0.2, hi=1.2,
                         with_grad=True)
    note(f"sweep case {case}")
    args = (w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)
    _check_out(case["dtype"], to_f64(gpu_forward(w)), msda_forward(*args))
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*args, w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)
    assert_grad_loc(gl, rgl, w.spatial_shapes)


@pytest.mark.gpu
@pytest.mark.parametrize("case", FUSED_CASES, ids=_case_id)
def test_random_fused_problem(case):
    """Raw offsets and logits (reference points: N(0, 2) pixel offsets; boxes:
    N(0, 0.25) box-unit offsets) with G deformable groups."""
    G = case["G"]
    w = fused_workload("decoder", N=case["N"], shapes=case["shapes"], Lq=case["Lq"], M=case["M"], D=case["D"],
                       K=case["K"], dtype=case["dtype"], seed=case["seed"], ref_dim=case["ref_dim"],
                       groups=None if G == case["M"] else G, with_grad=True)
    note(f"fused sweep case {case}")
    value, ref_t, off, logits, g = fused_device_inputs(w)
    out = to_f64(msda.msda_fused_forward(value, w.spatial_shapes, w.level_start, ref_t, off, logits))
    gv, go, gz, gr = (to_f64(t) for t in msda.msda_fused_backward(value, w.spatial_shapes, w.level_start,
                                                                    ref_t, off, logits, g))
    torch.cuda.synchronize()
    args = (w.value, w.spatial_shapes, w.level_start, w.ref, w.offsets, w.logits)
    _check_out(case["dtype"], out, msda_fused_forward(*args))
    rgv, rgo, rgz, rgr = msda_fused_backward(*args, w.grad_out)
    heads = case["M"] // G
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_logits", gz, rgz, atol=1e-5)
    assert_f32("grad_offsets (pixel units)", fused_pixel_offsets(w, go, w.ref), fused_pixel_offsets(w, rgo, w.ref),
               atol=1e-5)
    assert np.all(np.isfinite(gr))
    excess = np.abs(gr - rgr) - heads * fused_ref_bound(w, w.offsets)
    assert excess.max() <= 0, f"grad_ref beyond its bound by {excess.max():.3e}"


@pytest.mark.gpu
@pytest.mark.parametrize("case", GROUPED_CASES, ids=_case_id)
def test_random_grouped_problem(case):
    """Locations and weights shared by the M/G heads of each group (decoder
    recipe: uniform reference points plus N(0, 4) pixel offsets)."""
    G = case["G"]
    w = decoder_workload(N=case["N"], shapes=case["shapes"], Lq=case["Lq"], M=case["M"], D=case["D"],
                         K=case["K"], dtype=case["dtype"], seed=case["seed"], groups=G, with_grad=True)
    note(f"grouped sweep case {case}")
    value, loc, attn, g = device_inputs(w)
    out = to_f64(msda.msda_grouped_forward(value, w.spatial_shapes, w.level_start, loc, attn))
    gv, gl, ga = (to_f64(t) for t in msda.msda_grouped_backward(value, w.spatial_shapes, w.level_start, loc,
                                                                  attn, g))
    torch.cuda.synchronize()
    args = (w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)
    _check_out(case["dtype"], out, msda_grouped_forward(*args))
    rgv, rgl, rga = msda_grouped_backward(*args, w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga, atol=1e-5)
    assert_grad_loc(gl, rgl, w.spatial_shapes, atol=1e-5)
