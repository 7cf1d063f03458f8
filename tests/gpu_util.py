"""Helpers of the GPU parity tests: move workloads to the device, run the HIP
path through the binding, and compare with the fp64 oracle."""
import os
import sys

import numpy as np
import torch

import scale_deformable_attention_msda_amd as msda


def note(msg):
    """Name the case on stdout before a GPU step, so a failing run says which one it was."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def device_inputs(w, device="cuda:0"):
    if w.dtype == "bf16":
        value = torch.from_numpy(w.value_bits.view(np.int16).copy()).view(torch.bfloat16).to(device)
    else:
        value = torch.from_numpy(w.value).to(device)
    loc = torch.from_numpy(w.loc).to(device)
    attn = torch.from_numpy(w.attn).to(device)
    grad_out = None
    if w.grad_out is not None:
        if w.dtype == "bf16":
            grad_out = torch.from_numpy(w.grad_out_bits.view(np.int16).copy()).view(torch.bfloat16).to(device)
        else:
            grad_out = torch.from_numpy(w.grad_out).to(device)
    return value, loc, attn, grad_out


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def gpu_forward(w, device="cuda:0"):
    value, loc, attn, _ = device_inputs(w, device)
    out = msda.msda_forward(value, w.spatial_shapes, w.level_start, loc, attn)
    torch.cuda.synchronize()
    return out


def gpu_backward(w, device="cuda:0"):
    value, loc, attn, grad_out = device_inputs(w, device)
    gv, gl, ga = msda.msda_backward(value, w.spatial_shapes, w.level_start, loc, attn, grad_out)
    torch.cuda.synchronize()
    return gv, gl, ga


# every parity comparison of the session: (test, quantity, error, raw or None,
# max |g - r| / max(1, |r|)); summarised at the end of the run (conftest.py)
ERRORS = []


def _record(name, err, raw, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rel = float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref)))) if ref.size else 0.0
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    ERRORS.append((test, name, err, raw, rel))


def max_abs(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)))) if np.size(ref) else 0.0


def assert_f32(name, got, ref, atol=1e-5):
    err = max_abs(got, ref)
    _record(name, err, None, got, ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert err <= atol, f"{name}: max-abs error {err:.3e} > {atol:.1e}"
    return err


def grad_loc_pixels(gl, spatial_shapes, level_axis=-3):
    """grad_loc divided by (W_l, H_l): the location gradient in pixel units of its level."""
    gl = np.asarray(gl, np.float64)
    L = spatial_shapes.shape[0]
    scale = np.ones((L, 1, 2))
    scale[:, 0, 0] = spatial_shapes[:, 1]
    scale[:, 0, 1] = spatial_shapes[:, 0]
    return gl / scale


def assert_grad_loc(got, ref, spatial_shapes, atol=1e-5):
    """max-abs in pixel units; the raw error is reported alongside."""
    e_px = max_abs(grad_loc_pixels(got, spatial_shapes), grad_loc_pixels(ref, spatial_shapes))
    e_raw = max_abs(got, ref)
    _record("grad_loc (pixel units)", e_px, e_raw, got, ref)
    assert np.all(np.isfinite(got)), "grad_loc: non-finite values"
    assert e_px <= atol, f"grad_loc: max-abs (pixel units) {e_px:.3e} > {atol:.1e}; raw {e_raw:.3e}"
    return e_px, e_raw


def assert_normwise(name, got, ref, rtol=2e-2):
    ref = np.asarray(ref, np.float64)
    err = max_abs(got, ref) / max(float(np.max(np.abs(ref))), 1e-30)
    _record(name + " (normwise)", err, max_abs(got, ref), got, ref)
    assert err <= rtol, f"{name}: normwise error {err:.3e} > {rtol:.1e}"
    return err


def assert_bf16_out(got, ref):
    """bf16 output: normwise bound, and within one bf16 ulp (+1e-5) elementwise,
    since the float32 sum is rounded once to bf16."""
    assert_normwise("out", got, ref)
    slack = bf16_ulp(ref) + 1e-5
    bad = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)) > slack
    assert not bad.any(), f"{bad.sum()} bf16 outputs beyond one ulp; worst {max_abs(got, ref):.3e}"


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def sample_pairs(w, count, seed):
    d = w.dims
    rng = np.random.default_rng(seed)
    n = rng.integers(0, d["N"], count)
    q = rng.integers(0, d["Lq"], count)
    m = rng.integers(0, d["M"], count)
    # always include the very first and very last pair (tile edges, ragged tail)
    n[0], q[0], m[0] = 0, 0, 0
    n[1], q[1], m[1] = d["N"] - 1, d["Lq"] - 1, d["M"] - 1
    return n, q, m


def sample_rows(w, count, seed):
    d = w.dims
    rng = np.random.default_rng(seed)
    n = rng.integers(0, d["N"], count)
    s = rng.integers(0, d["S"], count)
    m = rng.integers(0, d["M"], count)
    # include rows of the coarsest level, where many samples pile up
    s0 = int(w.level_start[-1])
    s[: count // 4] = rng.integers(s0, d["S"], count // 4)
    n[-1], s[-1], m[-1] = d["N"] - 1, d["S"] - 1, d["M"] - 1
    return n, s, m


# ---------------------------------------------------------------- fused inputs

def fused_device_inputs(w, device="cuda:0"):
    if w.dtype == "bf16":
        value = torch.from_numpy(w.value_bits.view(np.int16).copy()).view(torch.bfloat16).to(device)
    else:
        value = torch.from_numpy(w.value).to(device)
    ref = torch.from_numpy(w.ref).to(device)
    off = torch.from_numpy(w.offsets).to(device)
    logits = torch.from_numpy(w.logits).to(device)
    g = None
    if w.grad_out is not None:
        if w.dtype == "bf16":
            g = torch.from_numpy(w.grad_out_bits.view(np.int16).copy()).view(torch.bfloat16).to(device)
        else:
            g = torch.from_numpy(w.grad_out).to(device)
    return value, ref, off, logits, g


def fused_pixel_offsets(w, g_off, ref_rows):
    """Offset gradients in pixel units of their level: points are already; boxes
    are divided by (w * W_l, h * H_l). ref_rows: the reference rows [..., ref_dim]
    matching g_off's leading axes."""
    g_off = np.asarray(g_off, np.float64)
    if w.ref.shape[-1] == 2:
        return g_off
    ss = w.spatial_shapes
    size = np.stack([ss[:, 1], ss[:, 0]], axis=-1).reshape(-1, 1, 2).astype(np.float64)  # [L,1,2]
    box = np.asarray(ref_rows, np.float64)[..., None, None, None, 2:]
    return g_off / (size * box)


def fused_ref_bound(w, off_rows):
    """Per-element bound of grad_ref [..., ref_dim] for queries with offsets off_rows [..., M, L, K, 2]."""
    ss = w.spatial_shapes
    size = np.stack([ss[:, 1], ss[:, 0]], axis=-1).reshape(-1, 1, 2).astype(np.float64)  # (W_l, H_l)
    off_rows = np.asarray(off_rows, np.float64)
    centre = 1e-5 * np.broadcast_to(size, off_rows.shape).sum(axis=(-4, -3, -2))
    if w.ref.shape[-1] == 2:
        return centre
    return np.concatenate([centre, 1e-5 * (size * np.abs(off_rows)).sum(axis=(-4, -3, -2))], axis=-1)
