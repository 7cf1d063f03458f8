"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances: float32 paths max-abs <= 1e-5 on out, grad_value and grad_attn;
grad_loc is compared in pixel units of its level (grad_loc_x / W_l,
grad_loc_y / H_l) at max-abs <= 1e-5, since at W_l = 167 one float32 ulp of the
raw gradient is already above 1e-5. bfloat16 outputs: normwise
max|gpu - oracle| / max|oracle| <= 2e-2, and additionally within one bf16 ulp
(+1e-5) elementwise, since the fp32 sum is rounded once to bf16.
"""
import dataclasses
import os
import subprocess

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import (fused_locations, msda_backward, msda_forward, msda_fused_backward,  # noqa: E402
                    msda_grad_value_rows, softmax_weights)
from tests.gpu_util import (assert_bf16_out, assert_f32, assert_grad_loc, assert_normwise, bf16_ulp,  # noqa: E402
                            device_inputs, gpu_backward, gpu_forward, max_abs, note, sample_pairs,
                            sample_rows, to_f64)
import scale_deformable_attention_msda_amd as msda  # noqa: E402
from workloads import (config_workload, decoder_workload, encoder_workload,  # noqa: E402
                       init_pattern_workload, uniform_workload)

pytestmark = pytest.mark.gpu

# Encoder-style maps small enough for the full oracle: 4 levels, S = 910 (ragged
# tiles: 910*8 pairs is not a multiple of the 32 pairs of a workgroup).
SMALL_LEVELS = ((20, 34), (10, 17), (5, 9), (3, 5))


def _oracle_args(w):
    return (w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)


def _check_bf16_out(got, ref):
    assert_bf16_out(got, ref)


# ------------------------------------------------------------ full elementwise parity

def test_tiny_forward_full():
    w = config_workload("tiny_fwd")
    note("tiny_fwd forward N=1 16x16 M=2 D=8 K=4 Lq=32 f32")
    out = to_f64(gpu_forward(w))
    assert_f32("out", out, msda_forward(*_oracle_args(w)))


def test_encoder_forward_small_maps_full():
    w = encoder_workload(N=2, shapes=SMALL_LEVELS, M=8, D=32, K=4, seed=12)
    note("encoder forward small maps N=2 S=910 M=8 D=32 K=4 f32")
    out = to_f64(gpu_forward(w))
    assert_f32("out", out, msda_forward(*_oracle_args(w)))


def test_decoder_bf16_forward_full_config():
    w = config_workload("decoder_fwd_bf16")
    note("decoder_fwd_bf16 full config N=2 Lq=300 COCO levels bf16")
    out = to_f64(gpu_forward(w))
    _check_bf16_out(out, msda_forward(*_oracle_args(w)))


def test_batched_encoder_bf16_small_maps_full():
    w = encoder_workload(N=3, shapes=SMALL_LEVELS, M=8, D=32, K=4, dtype="bf16", seed=14)
    note("batched encoder bf16 small maps N=3")
    out = to_f64(gpu_forward(w))
    _check_bf16_out(out, msda_forward(*_oracle_args(w)))


@pytest.mark.parametrize("K", [4, 8])
def test_encoder_backward_small_maps_full(K):
    w = encoder_workload(N=2, shapes=SMALL_LEVELS, M=8, D=32, K=K, seed=15 + K, with_grad=True)
    note(f"encoder backward small maps N=2 K={K} f32")
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*_oracle_args(w), w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)
    assert_grad_loc(gl, rgl, w.spatial_shapes)


def test_bf16_backward_small_maps_full():
    w = encoder_workload(N=2, shapes=SMALL_LEVELS, M=8, D=32, K=4, dtype="bf16", seed=19,
                         with_grad=True)
    note("encoder backward bf16 value/grad_out, fp32 gradients")
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*_oracle_args(w), w.grad_out)
    # inputs are exact bf16 values; the arithmetic is fp32, so the fp32 bar applies
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)
    assert_grad_loc(gl, rgl, w.spatial_shapes)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decoder_backward_full_config(dtype):
    """Decoder-sized launch (few samples per value tile): grad_value comes from
    per-sample atomics instead of the tile sort."""
    w = config_workload("decoder_fwd_bf16", dtype=dtype, with_grad=True)
    note(f"decoder backward full config N=2 Lq=300 COCO levels {dtype}")
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*_oracle_args(w), w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)
    assert_grad_loc(gl, rgl, w.spatial_shapes)


# ----------------------------------------------------- full-size configs, sampled outputs

def test_encoder_forward_full_size_sampled():
    w = config_workload("encoder_fwd")
    note("encoder_fwd full size N=1 S=Lq=22223 M=8 D=32 K=4 f32")
    out = gpu_forward(w)
    n, q, m = sample_pairs(w, 6000, seed=1)
    got = to_f64(out[torch.as_tensor(n), torch.as_tensor(q), torch.as_tensor(m)])
    assert_f32("out", got, msda_forward(*_oracle_args(w), pairs=(n, q, m)))
    # determinism: a second call is bitwise identical
    out2 = gpu_forward(w)
    assert torch.equal(out, out2)


def test_batched_encoder_bf16_full_size_sampled():
    w = config_workload("batched_encoder_fwd_bf16")
    note("batched_encoder_fwd_bf16 full size N=8 bf16")
    out = gpu_forward(w)
    n, q, m = sample_pairs(w, 6000, seed=2)
    got = to_f64(out[torch.as_tensor(n), torch.as_tensor(q), torch.as_tensor(m)])
    _check_bf16_out(got, msda_forward(*_oracle_args(w), pairs=(n, q, m)))


@pytest.mark.parametrize("name", ["encoder_bwd", "encoder_bwd_k8", "encoder_bwd_n4"])
def test_encoder_backward_full_size_sampled(name):
    # encoder_bwd_n4: four images give ~2700 split tiles, more than the scan's
    # LDS table holds, so their work items take its other path
    if name == "encoder_bwd_n4":
        w = encoder_workload(N=4, M=8, D=32, K=4, seed=9, with_grad=True)
    else:
        w = config_workload(name)
    note(f"{name} full size N={w.dims['N']} S=Lq=22223 M=8 D=32 K={w.dims['K']} f32")
    value, loc, attn, grad_out = device_inputs(w)
    gv, gl, ga = msda.msda_backward(value, w.spatial_shapes, w.level_start, loc, attn, grad_out)
    out = msda.msda_forward(value, w.spatial_shapes, w.level_start, loc, attn)
    torch.cuda.synchronize()
    n, q, m = sample_pairs(w, 3000, seed=3)
    idx = (torch.as_tensor(n), torch.as_tensor(q), torch.as_tensor(m))
    _, rgl, rga = msda_backward(*_oracle_args(w), w.grad_out, pairs=(n, q, m), with_grad_value=False)
    assert_f32("grad_attn", to_f64(ga[idx]), rga)
    assert_grad_loc(to_f64(gl[idx]), rgl, w.spatial_shapes)
    rn, rs, rm = sample_rows(w, 400, seed=4)
    rgv = msda_grad_value_rows(*_oracle_args(w), w.grad_out, (rn, rs, rm))
    assert_f32("grad_value", to_f64(gv[torch.as_tensor(rn), torch.as_tensor(rs), torch.as_tensor(rm)]), rgv)
    # adjoint identities over the whole tensors: <G,out> = <grad_value,V> = <grad_attn,A>
    lhs = float((grad_out.double() * out.double()).sum())
    rv = float((gv.double() * value.double()).sum())
    ra = float((ga.double() * attn.double()).sum())
    scale = float((grad_out.double().abs() * out.double().abs()).sum())
    assert abs(lhs - rv) <= 1e-6 * scale and abs(lhs - ra) <= 1e-6 * scale, (lhs, rv, ra, scale)


# ------------------------------------------------------------------------ edge cases

@pytest.mark.parametrize("D,dtype", [(5, "f32"), (12, "f32"), (64, "f32"), (100, "f32"),
                                     (1024, "f32"), (6, "bf16"), (8, "bf16"), (40, "bf16"),
                                     (1024, "bf16")])
def test_channel_counts(D, dtype):
    w = uniform_workload(N=2, shapes=((7, 9), (4, 5)), Lq=19, M=3, D=D, K=3, dtype=dtype,
                         seed=100 + D, with_grad=True)
    note(f"channel count D={D} {dtype}")
    out = to_f64(gpu_forward(w))
    ref = msda_forward(*_oracle_args(w))
    if dtype == "f32":
        assert_f32("out", out, ref)
    else:
        _check_bf16_out(out, ref)
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*_oracle_args(w), w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)
    assert_grad_loc(gl, rgl, w.spatial_shapes)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_pixel_levels(dtype):
    """Levels of one pixel (its centre at normalised (0.5, 0.5)), beside a small
    one: every sample inside interpolates towards the zero padding on both axes."""
    w = uniform_workload(N=2, shapes=((1, 1), (2, 3), (1, 1)), Lq=37, M=3, D=8, K=5, dtype=dtype,
                         seed=750, lo=-0.6, hi=1.6, with_grad=True)
    note(f"single-pixel levels, {dtype}")
    out = to_f64(gpu_forward(w))
    ref = msda_forward(*_oracle_args(w))
    if dtype == "f32":
        assert_f32("out", out, ref)
    else:
        _check_bf16_out(out, ref)
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*_oracle_args(w), w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)
    assert_grad_loc(gl, rgl, w.spatial_shapes)


def test_max_levels_and_points():
    shapes = tuple((2 + (l % 5), 3 + (l % 4)) for l in range(16))
    w = uniform_workload(N=1, shapes=shapes, Lq=9, M=2, D=8, K=16, seed=200, with_grad=True)
    note("L=16 K=16 (several descriptor chunks per workgroup)")
    assert_f32("out", to_f64(gpu_forward(w)), msda_forward(*_oracle_args(w)))
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*_oracle_args(w), w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)
    assert_grad_loc(gl, rgl, w.spatial_shapes)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hot_shapes_with_odd_point_counts(dtype):
    """D=32 with 16-byte lanes and enough pairs (40000) for the launch shapes
    that batch several samples' corner loads per lane (three in the bf16
    forward, two in the backward's sample pass), with L*K = 9 samples per
    head, so the last batch of every chunk is partly empty."""
    w = uniform_workload(N=1, shapes=((24, 40), (12, 20), (6, 10)), Lq=5000, M=8, D=32, K=3,
                         dtype=dtype, seed=300, with_grad=True)
    note(f"hot launch shapes with L*K=9, {dtype}, 40000 pairs")
    out = to_f64(gpu_forward(w))
    ref = msda_forward(*_oracle_args(w))
    if dtype == "f32":
        assert_f32("out", out, ref)
    else:
        _check_bf16_out(out, ref)
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*_oracle_args(w), w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)
    assert_grad_loc(gl, rgl, w.spatial_shapes)


def test_large_map_counts_tiles_in_global_memory():
    """A 400x400 level has 2500 8x8 tiles per (image, head), more than the
    binning passes count in LDS, so they count and place entries with one
    global atomic each; 24000 queries of 4 points keep the launch on the
    sorted (dense) grad_value path."""
    w = uniform_workload(N=1, shapes=((400, 400),), Lq=24000, M=2, D=8, K=4, seed=310, with_grad=True)
    note("one 400x400 level: 2500 tiles per (image, head), dense backward")
    assert_f32("out", to_f64(gpu_forward(w)), msda_forward(*_oracle_args(w)))
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*_oracle_args(w), w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)
    assert_grad_loc(gl, rgl, w.spatial_shapes)


@pytest.mark.parametrize("kind,dtype", [("dense", "f32"), ("dense", "bf16"), ("sparse", "f32")])
def test_non_finite_locations_contribute_nothing(kind, dtype):
    """A location with a NaN, infinite or overflowing coordinate lies outside
    every level: its sample adds nothing to out and gets zero grad_loc and
    grad_attn, exactly as a location far outside the map (the oracle's input
    here). Both grad_value routes: the sorted one (dense) and the atomic one."""
    if kind == "dense":
        w = encoder_workload(N=2, shapes=SMALL_LEVELS, M=8, D=32, K=4, dtype=dtype, seed=720,
                             with_grad=True)
    else:  # 40 queries x 16 samples stay below 32 samples per tile: per-sample atomics
        w = decoder_workload(N=2, shapes=SMALL_LEVELS, Lq=40, dtype=dtype, seed=721, with_grad=True)
    rng = np.random.default_rng(722)
    flat = w.loc.reshape(-1, 2)
    pick = rng.random(flat.shape[0]) < 0.1
    bad = np.array([np.nan, np.inf, -np.inf, 3e38, -3e38], np.float32)
    vals = bad[rng.integers(0, len(bad), size=(int(pick.sum()), 2))]
    one = rng.random(len(vals)) < 0.5  # half keep one finite coordinate
    axis = rng.integers(0, 2, size=len(vals))
    vals[one, axis[one]] = flat[pick][one, axis[one]]
    gpu_loc = flat.copy()
    gpu_loc[pick] = vals
    far = flat.copy()
    far[pick] = -5.0
    wg = dataclasses.replace(w, loc=gpu_loc.reshape(w.loc.shape))
    wo = dataclasses.replace(w, loc=far.reshape(w.loc.shape))
    note(f"non-finite locations ({int(pick.sum())} samples), {kind} backward, {dtype}")
    out = gpu_forward(wg)
    gv, gl, ga = gpu_backward(wg)
    for t in (out, gv, gl, ga):
        assert bool(torch.isfinite(t).all())
    ref = msda_forward(*_oracle_args(wo))
    if dtype == "f32":
        assert_f32("out", to_f64(out), ref)
    else:
        _check_bf16_out(to_f64(out), ref)
    rgv, rgl, rga = msda_backward(*_oracle_args(wo), wo.grad_out)
    assert_f32("grad_value", to_f64(gv), rgv)
    assert_f32("grad_attn", to_f64(ga), rga)
    assert_grad_loc(to_f64(gl), rgl, w.spatial_shapes)
    assert not to_f64(gl).reshape(-1, 2)[pick].any() and not to_f64(ga).reshape(-1)[pick].any()


def test_elongated_levels():
    """A 1x20000 and a 20000x1 level: 2500 one-row (one-column) tiles each, so
    the tiles are counted in global memory, coordinates reach 2e4, and 20000
    queries of 8 samples keep the sorted grad_value route."""
    w = uniform_workload(N=1, shapes=((1, 20000), (20000, 1)), Lq=20000, M=1, D=4, K=4, seed=760,
                         with_grad=True)
    note("elongated levels 1x20000 and 20000x1, dense backward")
    assert_f32("out", to_f64(gpu_forward(w)), msda_forward(*_oracle_args(w)))
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*_oracle_args(w), w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)
    assert_grad_loc(gl, rgl, w.spatial_shapes)


def test_native_program_through_the_c_abi():
    """tests/c/abi_device.cpp (built with the library): plain HIP buffers and
    a stream of its own, no torch, forward and backward through the C ABI,
    checked against closed forms (constant map, adjoint identity)."""
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_device")
    assert os.path.exists(exe), f"{exe} is missing: __graft_entry__.build() compiles it"
    note("native C++ program through the C ABI (hipMalloc buffers, own stream)")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout + res.stderr


def test_empty_problems():
    w = uniform_workload(N=1, shapes=((4, 4),), Lq=3, M=2, D=4, K=2, seed=300, with_grad=True)
    note("empty problems: Lq = 0 and N = 0")
    value, loc, attn, grad_out = device_inputs(w)
    out = msda.msda_forward(value, w.spatial_shapes, w.level_start, loc[:, :0].contiguous(),
                            attn[:, :0].contiguous())
    assert out.shape == (1, 0, 2, 4)
    gv = torch.full_like(value, float("nan"))
    msda.msda_backward(value, w.spatial_shapes, w.level_start, loc[:, :0].contiguous(),
                       attn[:, :0].contiguous(), grad_out[:, :0].contiguous(), grad_value=gv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(gv).item() == 0  # zeroed even with no queries
    out0 = msda.msda_forward(value[:0], w.spatial_shapes, w.level_start, loc[:0], attn[:0])
    assert out0.shape == (0, 3, 2, 4)


def test_samples_outside_and_nan():
    w = uniform_workload(N=1, shapes=((6, 7), (3, 3)), Lq=40, M=2, D=4, K=4, seed=400, lo=-1.0,
                         hi=2.0, with_grad=True)
    w.loc[0, :5] = np.nan
    w.loc[0, 5:10, :, :, :, 0] = 5.0      # far right of every level
    w.loc[0, 10:12, :, :, :, 1] = -0.75   # far above
    note("samples outside the map and NaN locations")
    out = to_f64(gpu_forward(w))
    ref = msda_forward(*_oracle_args(w))
    assert np.all(ref[0, :12] == 0)
    assert_f32("out", out, ref)
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*_oracle_args(w), w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)
    assert_grad_loc(gl, rgl, w.spatial_shapes)
    assert np.all(gl[0, :12] == 0) and np.all(ga[0, :12] == 0)


def test_kinks_follow_the_right_derivative():
    w = init_pattern_workload(N=2, shape=(16, 16), M=8, D=4, K=3, seed=500)
    note("compass initialisation: every sample on a pixel centre")
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*_oracle_args(w), w.grad_out)
    assert_grad_loc(gl, rgl, w.spatial_shapes)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)


def test_worked_example_on_gpu():
    """The printed example (page "Deformable DETR Samples Sparse Points"): the
    weighted blend of the four samples is 0.70; same construction as the oracle pin
    (a bilinear surface through the printed values at the printed locations)."""
    import json
    import os
    from tests.dense_reference import exact_index_coordinate
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))
    H, W = g["map_hw"]
    xs = [exact_index_coordinate(lx, W) for lx, _ in g["locations"]]
    ys = [exact_index_coordinate(ly, H) for _, ly in g["locations"]]
    c = np.linalg.solve(np.array([[1.0, x, y, x * y] for x, y in zip(xs, ys)]), g["sampled_values"])
    ii, jj = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    vmap = (c[0] + c[1] * jj + c[2] * ii + c[3] * jj * ii).astype(np.float32)
    value = torch.from_numpy(vmap.reshape(1, H * W, 1, 1)).cuda()
    loc = torch.tensor(g["locations"], dtype=torch.float32).reshape(1, 1, 1, 1, 4, 2).cuda()
    attn = torch.tensor(g["weights"], dtype=torch.float32).reshape(1, 1, 1, 1, 4).cuda()
    note("worked example on GPU")
    out = msda.msda_forward(value, [[H, W]], [0], loc, attn)
    # the fp32 map stores c-surface values to ~1e-7 relative (|f| <= ~200 on the map)
    assert abs(out.item() - g["blend"]) < 1e-4


def test_guard_zones_untouched():
    w = uniform_workload(N=1, shapes=((9, 11), (5, 6)), Lq=37, M=4, D=8, K=3, seed=600,
                         with_grad=True)
    value, loc, attn, grad_out = device_inputs(w)
    d = w.dims
    G = 4096
    note("guard zones around every output")

    def guarded(n):
        buf = torch.full((n + 2 * G,), 12345.0, dtype=torch.float32, device="cuda")
        return buf, buf[G:G + n]

    ob, out = guarded(d["N"] * d["Lq"] * d["M"] * d["D"])
    msda.msda_forward(value, w.spatial_shapes, w.level_start, loc, attn,
                      out=out.view(d["N"], d["Lq"], d["M"], d["D"]))
    vb, gv = guarded(value.numel())
    lb, gl = guarded(loc.numel())
    ab, ga = guarded(attn.numel())
    msda.msda_backward(value, w.spatial_shapes, w.level_start, loc, attn, grad_out,
                       grad_value=gv.view(value.shape), grad_loc=gl.view(loc.shape),
                       grad_attn=ga.view(attn.shape))
    torch.cuda.synchronize()
    for buf in (ob, vb, lb, ab):
        assert torch.all(buf[:G] == 12345.0) and torch.all(buf[-G:] == 12345.0)
    assert_f32("out", to_f64(out).reshape(d["N"], d["Lq"], d["M"], d["D"]),
               msda_forward(*_oracle_args(w)))


def test_unaligned_value_and_stream():
    """A value view starting 4 bytes past an allocation takes narrower accesses and
    must give the same result; a side stream is honoured."""
    w = uniform_workload(N=1, shapes=((8, 8),), Lq=21, M=2, D=8, K=4, seed=700)
    value, loc, attn, _ = device_inputs(w)
    flat = torch.empty(value.numel() + 1, dtype=torch.float32, device="cuda")
    flat[1:] = value.reshape(-1)
    shifted = flat[1:].view(value.shape)
    assert shifted.data_ptr() % 16 != 0
    note("unaligned value view on a side stream")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = msda.msda_forward(shifted, w.spatial_shapes, w.level_start, loc, attn)
    s.synchronize()
    assert_f32("out", to_f64(out), msda_forward(*_oracle_args(w)))
    with pytest.raises(msda.MSDAError):
        bad = torch.empty(loc.numel() + 1, dtype=torch.float32, device="cuda")[1:].view(loc.shape)
        msda.msda_forward(value, w.spatial_shapes, w.level_start, bad, attn)


def test_explicit_stream_handle():
    """A raw stream handle (or a torch stream) passed as ``stream`` is used in
    place of torch's current stream, for the forward and the backward (its
    workspace comes from torch)."""
    w = uniform_workload(N=1, shapes=((9, 7), (4, 5)), Lq=33, M=2, D=8, K=3, seed=710,
                         with_grad=True)
    value, loc, attn, grad_out = device_inputs(w)
    d = w.dims
    need = msda.msda_backward_workspace_size(w.spatial_shapes, w.level_start, d["N"], d["S"], d["M"],
                                             d["D"], d["L"], d["Lq"], d["K"])
    torch.cuda.synchronize()
    note("explicit stream handle: forward and backward queued behind matmuls")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):  # keeps the side stream busy for a few milliseconds
        a = torch.randn(2048, 2048, device="cuda")
        for _ in range(8):
            a = torch.mm(a, a) * (1.0 / 64)
    out = msda.msda_forward(value, w.spatial_shapes, w.level_start, loc, attn, stream=s.cuda_stream)
    gv, gl, ga = msda.msda_backward(value, w.spatial_shapes, w.level_start, loc, attn, grad_out,
                                    stream=s.cuda_stream)
    out_s = msda.msda_forward(value, w.spatial_shapes, w.level_start, loc, attn, stream=s)  # a torch stream
    # Memory the backward's workspace came from must not be handed out again while the
    # side stream has not reached it: fill same-sized blocks on the current stream.
    junk = [torch.full((max(need, 1),), 255, dtype=torch.uint8, device="cuda") for _ in range(4)]
    s.synchronize()
    del junk
    assert_f32("out", to_f64(out), msda_forward(*_oracle_args(w)))
    assert torch.equal(out, out_s)
    rv, rl, ra = msda_backward(*_oracle_args(w), w.grad_out)
    assert_f32("grad_value", to_f64(gv), rv)
    assert_grad_loc(to_f64(gl), rl, w.spatial_shapes)
    assert_f32("grad_attn", to_f64(ga), ra)


def test_autograd_wrapper_matches_entry_points():
    w = uniform_workload(N=1, shapes=((6, 8), (3, 4)), Lq=10, M=2, D=8, K=2, seed=800,
                         with_grad=True)
    value, loc, attn, grad_out = device_inputs(w)
    value.requires_grad_(True)
    loc.requires_grad_(True)
    attn.requires_grad_(True)
    note("autograd wrapper")
    out = msda.msda_sample(value, w.spatial_shapes, w.level_start, loc, attn)
    out.backward(grad_out)
    gv, gl, ga = msda.msda_backward(value.detach(), w.spatial_shapes, w.level_start, loc.detach(),
                                    attn.detach(), grad_out)
    torch.cuda.synchronize()
    assert torch.allclose(value.grad, gv, atol=1e-6)
    assert torch.equal(loc.grad, gl) and torch.equal(attn.grad, ga)


def test_crowded_tile_is_split():
    """Thousands of samples on one 8x8 tile: its grad_value work is split over
    several workgroups whose partial sums are combined."""
    w = uniform_workload(N=1, shapes=((4, 5),), Lq=1500, M=2, D=32, K=4, seed=900, lo=0.0, hi=1.0,
                         with_grad=True)
    note("crowded tile: 6000 samples per head on a 4x5 map")
    gv, gl, ga = (to_f64(t) for t in gpu_backward(w))
    rgv, rgl, rga = msda_backward(*_oracle_args(w), w.grad_out)
    assert_f32("grad_value", gv, rgv)
    assert_f32("grad_attn", ga, rga)
    assert_grad_loc(gl, rgl, w.spatial_shapes)


def test_levels_with_gaps():
    """level_start may leave rows of value outside every level; their gradient is 0."""
    rng = np.random.default_rng(950)
    shapes = np.array([[5, 6], [3, 3]], dtype=np.int64)
    starts = np.array([2, 40], dtype=np.int64)
    S, M, D, Lq, K = 52, 2, 8, 11, 3
    value = rng.standard_normal((1, S, M, D)).astype(np.float32)
    loc = rng.uniform(-0.1, 1.1, (1, Lq, M, 2, K, 2)).astype(np.float32)
    attn = rng.uniform(0, 1, (1, Lq, M, 2, K)).astype(np.float32)
    G = rng.standard_normal((1, Lq, M, D)).astype(np.float32)
    note("levels with gaps in value's rows")
    args = [torch.from_numpy(a).cuda() for a in (value, loc, attn, G)]
    out = msda.msda_forward(args[0], shapes, starts, args[1], args[2])
    gv = torch.full_like(args[0], float("nan"))
    gv, gl, ga = msda.msda_backward(args[0], shapes, starts, args[1], args[2], args[3], grad_value=gv)
    torch.cuda.synchronize()
    assert_f32("out", to_f64(out), msda_forward(value, shapes, starts, loc, attn))
    rgv, rgl, rga = msda_backward(value, shapes, starts, loc, attn, G)
    assert_f32("grad_value", to_f64(gv), rgv)
    assert_f32("grad_attn", to_f64(ga), rga)
    assert_grad_loc(to_f64(gl), rgl, shapes)


def test_graph_capture_of_decoder_layers():
    """Six decoder layers' sampling (forward and backward, bf16 values) captured
    in one HIP graph through the C ABI and replayed; every replay, with eager
    work and synchronisation in between, must equal the eager results."""
    w = config_workload("decoder_fwd_bf16", with_grad=True)
    value, loc, attn, grad_out = device_inputs(w)
    ss, ls = w.spatial_shapes, w.level_start
    d = w.dims
    gen = torch.Generator(device="cuda").manual_seed(5)
    layers = []
    for _ in range(6):
        l_loc = (loc + 0.01 * torch.randn(loc.shape, device="cuda", generator=gen)).contiguous()
        l_attn = torch.softmax(torch.randn(attn.shape[:3] + (d["L"] * d["K"],), device="cuda", generator=gen),
                               -1).reshape(attn.shape).contiguous()
        layers.append((l_loc, l_attn))
    ws_bytes = msda.msda_backward_workspace_size(ss, ls, d["N"], d["S"], d["M"], d["D"], d["L"], d["Lq"],
                                                 d["K"], msda.MSDA_BF16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    outs = [torch.empty((d["N"], d["Lq"], d["M"], d["D"]), dtype=torch.bfloat16, device="cuda") for _ in range(6)]
    gvs = [torch.empty(value.shape, dtype=torch.float32, device="cuda") for _ in range(6)]
    gls = [torch.empty(loc.shape, dtype=torch.float32, device="cuda") for _ in range(6)]
    gas = [torch.empty(attn.shape, dtype=torch.float32, device="cuda") for _ in range(6)]

    def run():
        for i, (l_loc, l_attn) in enumerate(layers):
            msda.msda_forward(value, ss, ls, l_loc, l_attn, out=outs[i])
            msda.msda_backward(value, ss, ls, l_loc, l_attn, grad_out, grad_value=gvs[i], grad_loc=gls[i],
                               grad_attn=gas[i], workspace=ws)

    note("graph capture: 6 decoder layers forward+backward, bf16")
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs + gvs + gls + gas]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        for t in outs + gvs + gls + gas:
            t.fill_(float("nan"))
        _ = (torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outs + gvs + gls + gas
        for k, (a, b) in enumerate(zip(got, ref)):
            if k < 6 or k >= 18:  # forward outputs and grad_attn are deterministic
                assert torch.equal(a, b), (rep, k)
            else:
                assert torch.allclose(a, b, rtol=0, atol=1e-5), (rep, k)


def test_graph_capture_of_the_dense_backward():
    """The tile-sorted backward (counters cleared by a fill kernel, count, scan,
    scatter, grad_value items with split-tile atomics) captured in a HIP graph:
    each replay, with new inputs copied into the captured buffers, eager work
    and synchronisation in between, matches the oracle for those inputs."""
    wls = [encoder_workload(N=2, shapes=SMALL_LEVELS, M=8, D=32, K=4, seed=730 + i, with_grad=True)
           for i in range(2)]
    d = wls[0].dims
    ss, ls = wls[0].spatial_shapes, wls[0].level_start
    tiles = sum(((h + 7) // 8) * ((w_ + 7) // 8) for h, w_ in SMALL_LEVELS)
    assert d["Lq"] * d["L"] * d["K"] >= 32 * tiles  # the dense route
    refs = [msda_backward(*_oracle_args(w), w.grad_out) for w in wls]
    value, loc, attn, grad_out = device_inputs(wls[0])
    gv, gl, ga = torch.empty_like(value), torch.empty_like(loc), torch.empty_like(attn)
    ws = torch.empty(msda.msda_backward_workspace_size(ss, ls, d["N"], d["S"], d["M"], d["D"], d["L"], d["Lq"],
                                                       d["K"]), dtype=torch.uint8, device="cuda")

    def run():
        msda.msda_backward(value, ss, ls, loc, attn, grad_out, grad_value=gv, grad_loc=gl, grad_attn=ga,
                           workspace=ws)

    note("graph capture: dense encoder backward, small maps, f32")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        w = wls[rep % 2]
        for dst, src in ((value, w.value), (loc, w.loc), (attn, w.attn), (grad_out, w.grad_out)):
            dst.copy_(torch.from_numpy(src))
        for t in (gv, gl, ga):
            t.fill_(float("nan"))
        _ = (torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rgv, rgl, rga = refs[rep % 2]
        assert_f32("grad_value", to_f64(gv), rgv)
        assert_f32("grad_attn", to_f64(ga), rga)
        assert_grad_loc(to_f64(gl), rgl, w.spatial_shapes)


def test_concurrent_calls_from_host_threads():
    """The library keeps no state between calls: four host threads, each with
    its own stream and problem (dense and sparse grad_value routes), call the
    forward and the backward at the same time; every result matches the oracle."""
    import threading

    wls = [encoder_workload(N=1, shapes=SMALL_LEVELS, M=8, D=32, K=4, seed=740 + i, with_grad=True)
           if i % 2 == 0 else
           decoder_workload(N=2, shapes=SMALL_LEVELS, Lq=30, dtype="f32", seed=740 + i, with_grad=True)
           for i in range(4)]
    refs = [(msda_forward(*_oracle_args(w)), msda_backward(*_oracle_args(w), w.grad_out)) for w in wls]
    inputs = [device_inputs(w) for w in wls]
    torch.cuda.synchronize()
    results, errors = [None] * 4, []

    def worker(i):
        try:
            value, loc, attn, grad_out = inputs[i]
            w = wls[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    out = msda.msda_forward(value, w.spatial_shapes, w.level_start, loc, attn)
                    grads = msda.msda_backward(value, w.spatial_shapes, w.level_start, loc, attn, grad_out)
            s.synchronize()
            results[i] = (out, grads)
        except Exception as e:  # reported by the main thread
            errors.append((i, repr(e)))

    note("concurrent calls: 4 host threads, own streams")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i, w in enumerate(wls):
        out, (gv, gl, ga) = results[i]
        ref_out, (rgv, rgl, rga) = refs[i]
        assert_f32("out", to_f64(out), ref_out)
        assert_f32("grad_value", to_f64(gv), rgv)
        assert_f32("grad_attn", to_f64(ga), rga)
        assert_grad_loc(to_f64(gl), rgl, w.spatial_shapes)


def test_batch_split_across_launches():
    """Images whose value slice exceeds 2^27 elements run one launch per image;
    every pointer (value, loc, attn, ref, outputs and gradients) is offset per
    launch and the workspace is reused. One level of 1449x1449 pixels, M=2,
    D=32: 134.4 M elements per image, so N=3 takes three launches."""
    rng = np.random.default_rng(990)
    N, H, W, M, D, K, Lq = 3, 1449, 1449, 2, 32, 4, 150
    S = H * W
    shapes = np.array([[H, W]], dtype=np.int64)
    starts = np.array([0], dtype=np.int64)
    value = rng.standard_normal((N, S, M, D), dtype=np.float32)
    loc = rng.uniform(-0.05, 1.05, (N, Lq, M, 1, K, 2)).astype(np.float32)
    attn = rng.uniform(0, 1, (N, Lq, M, 1, K)).astype(np.float32)
    G = rng.standard_normal((N, Lq, M, D), dtype=np.float32)
    note("batch split: N=3 images of 1449x1449 x M=2 x D=32, one launch per image")
    dv = torch.from_numpy(value).cuda()
    dl, da, dg = (torch.from_numpy(a).cuda() for a in (loc, attn, G))
    out = msda.msda_forward(dv, shapes, starts, dl, da)
    gv, gl, ga = msda.msda_backward(dv, shapes, starts, dl, da, dg)
    torch.cuda.synchronize()
    n = np.repeat(np.arange(N), 40)
    q = np.tile(np.linspace(0, Lq - 1, 40).astype(np.int64), N)
    m = np.tile(np.arange(40) % M, N)
    idx = (torch.as_tensor(n), torch.as_tensor(q), torch.as_tensor(m))
    assert_f32("out", to_f64(out[idx]), msda_forward(value, shapes, starts, loc, attn, pairs=(n, q, m)))
    _, rgl, rga = msda_backward(value, shapes, starts, loc, attn, G, pairs=(n, q, m), with_grad_value=False)
    assert_f32("grad_attn", to_f64(ga[idx]), rga)
    assert_grad_loc(to_f64(gl[idx]), rgl, shapes)
    # grad_value rows: ones that samples touch (corner pixels of sampled pairs) and random ones
    px = np.clip((loc[n, q, m, 0, 0, 0] * W - 0.5).astype(np.int64), 0, W - 1)
    py = np.clip((loc[n, q, m, 0, 0, 1] * H - 0.5).astype(np.int64), 0, H - 1)
    rs = np.concatenate([py * W + px, rng.integers(0, S, 60)])
    rn = np.concatenate([n, rng.integers(0, N, 60)])
    rm = np.concatenate([m, rng.integers(0, M, 60)])
    rgv = msda_grad_value_rows(value, shapes, starts, loc, attn, G, (rn, rs, rm))
    assert np.abs(rgv).max() > 0
    assert_f32("grad_value", to_f64(gv[torch.as_tensor(rn), torch.as_tensor(rs), torch.as_tensor(rm)]), rgv)
    # the fused entry points split the same way (ref and grad_ref offset per launch)
    ref = rng.uniform(0.2, 0.8, (N, Lq, 4)).astype(np.float32)
    ref[..., 2:] = rng.uniform(0.05, 0.3, (N, Lq, 2))
    off = rng.standard_normal((N, Lq, M, 1, K, 2)).astype(np.float32) * 0.3
    z = rng.standard_normal((N, Lq, M, 1, K)).astype(np.float32)
    dref, doff, dz = (torch.from_numpy(a).cuda() for a in (ref, off, z))
    fout = msda.msda_fused_forward(dv, shapes, starts, dref, doff, dz)
    _, fgo, fgz, fgr = msda.msda_fused_backward(dv, shapes, starts, dref, doff, dz, dg)
    torch.cuda.synchronize()
    floc = fused_locations(ref, off, shapes)
    fA = softmax_weights(z)
    assert_f32("fused out", to_f64(fout[idx]), msda_forward(value, shapes, starts, floc, fA, pairs=(n, q, m)))
    qn, qq = np.arange(N).repeat(3), np.tile(np.array([0, Lq // 2, Lq - 1]), N)
    _, rgo, rgz, rgr = msda_fused_backward(value, shapes, starts, ref, off, z, G, queries=(qn, qq))
    qi = (torch.as_tensor(qn), torch.as_tensor(qq))
    assert_f32("fused grad_logits", to_f64(fgz[qi]), rgz)
    scale = (np.float64(W) * ref[qn, qq, 2:][:, None, None, None, :])  # box size * W_l: pixel units
    assert_f32("fused grad_offsets (pixel units)", to_f64(fgo[qi]) / scale, rgo / scale)
    bound = 1e-5 * M * K * W * (1 + np.abs(off).max())
    assert max_abs(to_f64(fgr[qi]), rgr) <= bound
