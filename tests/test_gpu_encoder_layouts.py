"""Encoder-layout forwards (every pixel of every level is a query, Lq = S),
element by element against the fp64 oracle, beyond the standard encoder
shapes: mid-sized maps spanning many workgroups, far offsets (N(0, 12 px), so
a workgroup's samples scatter over much of each level), levels listed coarse to
fine, one-pixel and one-row levels, several images, other channel counts and
point counts. The result must not depend on the query count either: the same
problem with one more query gives the same bits for the shared queries.

Tolerances as everywhere: fp32 max-abs <= 1e-5; bf16 outputs normwise <= 2e-2
and within one bf16 ulp elementwise."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import msda_forward  # noqa: E402
from tests.gpu_util import assert_bf16_out, assert_f32, device_inputs, note, to_f64  # noqa: E402
import scale_deformable_attention_msda_amd as msda  # noqa: E402
from workloads import encoder_workload  # noqa: E402

pytestmark = pytest.mark.gpu

SMALL_LEVELS = ((20, 34), (10, 17), (5, 9), (3, 5))
MID_LEVELS = ((64, 96), (32, 48), (16, 24), (8, 12))


def _check(w, label):
    note(f"encoder-layout forward: {label} N={w.dims['N']} S={w.dims['S']} M={w.dims['M']} D={w.dims['D']} "
         f"K={w.dims['K']} {w.dtype}")
    value, loc, attn, _ = device_inputs(w)
    ss, ls = w.spatial_shapes, w.level_start
    out = msda.msda_forward(value, ss, ls, loc, attn)
    # one more query (a copy of the first): the shared queries' bits do not change
    loc2 = torch.cat([loc, loc[:, :1]], dim=1).contiguous()
    attn2 = torch.cat([attn, attn[:, :1]], dim=1).contiguous()
    out2 = msda.msda_forward(value, ss, ls, loc2, attn2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2[:, :-1]), f"{label}: result depends on the query count"
    ref = msda_forward(w.value, ss, ls, w.loc, w.attn)
    if w.dtype == "bf16":
        assert_bf16_out(to_f64(out), ref)
    else:
        assert_f32("out", to_f64(out), ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_encoder_offsets_small_and_mid_maps(dtype):
    _check(encoder_workload(N=2, shapes=SMALL_LEVELS, M=8, D=32, K=4, dtype=dtype, seed=1201), "small maps")
    _check(encoder_workload(N=1, shapes=MID_LEVELS, M=8, D=32, K=4, dtype=dtype, seed=1202), "mid maps")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_far_offsets(dtype):
    _check(encoder_workload(N=1, shapes=MID_LEVELS, M=4, D=32, K=4, dtype=dtype, seed=1203, offset_px=12.0),
           "far offsets")


def test_level_order_and_tiny_levels():
    _check(encoder_workload(N=1, shapes=((5, 9), (20, 34), (1, 1), (10, 17)), M=4, D=32, K=4, seed=1204),
           "levels out of order with a 1x1 level")
    _check(encoder_workload(N=3, shapes=((1, 7), (3, 2)), M=2, D=32, K=3, seed=1205), "tiny levels, K=3")


@pytest.mark.parametrize("D,dtype", [(16, "f32"), (64, "bf16"), (32, "f32")])
def test_channel_counts_and_points(D, dtype):
    _check(encoder_workload(N=1, shapes=SMALL_LEVELS, M=4, D=D, K=8 if D == 32 else 4, dtype=dtype, seed=1206),
           f"D={D}")


def test_three_image_launch_matches_per_image_launches():
    """Three mid-sized encoder images in one fp32 launch (6120 workgroups; with
    the extra query of _check, a ragged last workgroup) against the oracle, and
    bit for bit against each image launched on its own (2040 workgroups): a
    query's result does not depend on the batch it is launched with."""
    w = encoder_workload(N=3, shapes=MID_LEVELS, M=8, D=32, K=4, seed=1207)
    _check(w, "three images in one launch")
    value, loc, attn, _ = device_inputs(w)
    ss, ls = w.spatial_shapes, w.level_start
    out = msda.msda_forward(value, ss, ls, loc, attn)
    singles = [msda.msda_forward(value[n:n + 1].contiguous(), ss, ls, loc[n:n + 1].contiguous(),
                                 attn[n:n + 1].contiguous()) for n in range(3)]
    torch.cuda.synchronize()
    for n in range(3):
        assert torch.equal(out[n:n + 1], singles[n]), f"image {n}"
