"""The encoder forward with value windows staged in LDS (launches where every
pixel is a query, Lq = S, and the levels cover every row of value), element by
element against the fp64 oracle, and bit for bit against the plain forward
(the same problem with one extra query, which takes the plain path): the two
compute the same weights and sum in the same order.

Cases: ordinary encoder offsets (every corner inside its tile's window), far
offsets (windows cut to their capacity, so a share of the samples read their
rows from global memory), levels listed coarse to fine, single-pixel levels,
several images, and the channel counts the window path takes (fp32 D = 16 and
32, bf16 D = 32 and 64).

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
# 8x8 tiles of the finest level: 8 x 12 of them, several pyramid tiles deep
MID_LEVELS = ((64, 96), (32, 48), (16, 24), (8, 12))


def _window_and_plain(w):
    """Forward through the window path (Lq = S) and through the plain path (the
    same queries plus one more, so Lq = S + 1), on the same device inputs."""
    value, loc, attn, _ = device_inputs(w)
    ss, ls = w.spatial_shapes, w.level_start
    out = msda.msda_forward(value, ss, ls, loc, attn)
    loc2 = torch.cat([loc, loc[:, :1]], dim=1).contiguous()
    attn2 = torch.cat([attn, attn[:, :1]], dim=1).contiguous()
    out2 = msda.msda_forward(value, ss, ls, loc2, attn2)
    torch.cuda.synchronize()
    return out, out2[:, :-1]


def _check(w, label):
    note(f"window forward: {label} N={w.dims['N']} S={w.dims['S']} M={w.dims['M']} D={w.dims['D']} "
         f"K={w.dims['K']} {w.dtype}")
    out, plain = _window_and_plain(w)
    assert torch.equal(out, plain), f"{label}: window and plain forward differ"
    ref = msda_forward(w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)
    if w.dtype == "bf16":
        assert_bf16_out(to_f64(out), ref)
    else:
        assert_f32("out", to_f64(out), ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_window_forward_encoder_offsets(dtype):
    _check(encoder_workload(N=2, shapes=SMALL_LEVELS, M=8, D=32, K=4, dtype=dtype, seed=1201), "small maps")
    _check(encoder_workload(N=1, shapes=MID_LEVELS, M=8, D=32, K=4, dtype=dtype, seed=1202), "mid maps")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_window_forward_far_offsets_read_outside_the_window(dtype):
    # N(0, 12 px) offsets: an 8x8 tile's corners span ~80 px, far beyond a window's
    # capacity, so windows are cut and many samples take the global-memory rows
    _check(encoder_workload(N=1, shapes=MID_LEVELS, M=4, D=32, K=4, dtype=dtype, seed=1203, offset_px=12.0),
           "far offsets")


def test_window_forward_level_order_and_tiny_levels():
    # finest level not first; one-pixel and one-row levels
    _check(encoder_workload(N=1, shapes=((5, 9), (20, 34), (1, 1), (10, 17)), M=4, D=32, K=4, seed=1204),
           "levels out of order with a 1x1 level")
    _check(encoder_workload(N=3, shapes=((1, 7), (3, 2)), M=2, D=32, K=3, seed=1205), "tiny levels, K=3")


@pytest.mark.parametrize("D,dtype", [(16, "f32"), (64, "bf16"), (32, "f32")])
def test_window_forward_channel_counts_and_points(D, dtype):
    _check(encoder_workload(N=1, shapes=SMALL_LEVELS, M=4, D=D, K=8 if D == 32 else 4, dtype=dtype, seed=1206),
           f"D={D}")


def test_window_forward_full_size_encoder_matches_plain():
    # the encoder workload at its real size: bit-identical to the plain forward
    w = encoder_workload(N=1, M=8, D=32, K=4, seed=2)
    note("window forward: full encoder shape vs plain path")
    out, plain = _window_and_plain(w)
    assert torch.equal(out, plain)
