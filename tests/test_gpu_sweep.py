"""Seeded sweep of small random problems through the C ABI against the fp64
oracle: 1 to 5 levels (1x1 maps included), 1 to 8 points, odd and even channel
counts, queries from a handful to a few hundred (so both grad_value routes,
per-sample atomics and the tile sort, occur), float32 and bfloat16 values.
Each case runs the forward and the backward and compares every output
element, at the bars of the other parity tests."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import msda_backward, msda_forward  # noqa: E402
from tests.gpu_util import (assert_f32, assert_grad_loc, assert_normwise, bf16_ulp,  # noqa: E402
                            gpu_backward, gpu_forward, max_abs, note, to_f64)
from workloads import uniform_workload  # noqa: E402

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


def _tiles(shapes):
    return sum(((h + 7) // 8) * ((w + 7) // 8) for h, w in shapes)


def test_sweep_covers_both_grad_value_routes():
    """The sweep holds problems on each side of the route threshold (fewer
    than 32 samples per tile and head go to per-sample atomics)."""
    dense = [c["Lq"] * len(c["shapes"]) * c["K"] >= 32 * _tiles(c["shapes"]) for c in CASES]
    assert any(dense) and not all(dense)


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=lambda c: (f"N{c['N']}-L{len(c['shapes'])}-M{c['M']}-D{c['D']}"
                                                      f"-K{c['K']}-Lq{c['Lq']}-{c['dtype']}"))
def test_random_problem(case):
    w = uniform_workload(N=case["N"], shapes=case["shapes"], Lq=case["Lq"], M=case["M"], D=case["D"],
                         K=case["K"], dtype=case["dtype"], seed=case["seed"], lo=-0.2, hi=1.2,
                         with_grad=True)
    note(f"sweep case {case}")
    args = (w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)
    out = to_f64(gpu_forward(w))
    ref = msda_forward(*args)
    if case["dtype"] == "f32":
        assert_f32("out", out, ref)
    else:
        assert_normwise("out", out, ref)
        slack = bf16_ulp(ref) + 1e-5
        assert not (np.abs(out - ref) > slack).any(), f"bf16 out beyond one ulp: {max_abs(out, ref):.3e}"
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*args, w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)
    assert_grad_loc(gl, rgl, w.spatial_shapes)
