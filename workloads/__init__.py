"""Seeded synthetic inputs for the multi-scale deformable attention sampling core.

This module only draws inputs. It holds none of the sampling arithmetic (no
coordinate transform, no bilinear read, no weighted sum): the HIP library and the
fp64 oracle both receive what it returns and compute independently.

What the inputs stand in for. The method runs on multi-scale feature maps of
COCO images (page "Deformable DETR", sections "Encoder" and "Hyperparameters":
L=4 levels at strides 8/16/32/64, C=256 channels, M=8 heads, K=4 points,
300 object queries). No dataset or trained weight is available, so every input
is synthetic, with those shapes:

* An 800x1333 image gives the level maps 100x167, 50x84, 25x42, 13x21.
* Encoder queries are the pixels of the maps themselves; each query's reference
  point is its own pixel centre in normalised image coordinates (page
  "Deformable DETR", section "Encoder"). Offsets are Gaussian, in pixels of the
  sampled level, converted to normalised units by dividing by that level's
  width/height.
* Decoder reference points are uniform in [0,1]^2 (section "Decoder" predicts
  them with a sigmoid; no trained projection exists here).
* Attention weights are a softmax of N(0,1) logits taken jointly over the L*K
  samples of one (query, head), so they sum to 1 per head (section
  "Multi-scale deformable attention").

The softmax and the reference-plus-offset locations above only draw the
sampling core's inputs, following the workloads' stated recipe. The fused entry
points (the step in front of the core) are instead given the raw draws (logits,
reference points or boxes, offsets) from ``fused_workload``; the kernels and the
oracle each form weights and locations from them on their own, and neither
calls anything here to do so.

Draw order with ``np.random.default_rng(seed)``: value -> reference points ->
offsets -> logits -> grad_out. Values are drawn in float64 and cast to float32;
bf16 values are float32 rounded to nearest-even and kept as raw uint16 bits,
with ``value`` holding their exact float32 upcast.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

# The four encoder levels of an 800x1333 image at strides 8, 16, 32, 64.
COCO_LEVELS = ((100, 167), (50, 84), (25, 42), (13, 21))


def level_starts(shapes):
    """Row offset of each level in the flattened S axis (levels concatenated,
    finest first, each level row-major over (y, x))."""
    starts, s = [], 0
    for h, w in shapes:
        starts.append(s)
        s += h * w
    return np.asarray(starts, dtype=np.int64), s


def bf16_bits_from_f32(x):
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bits.

    Works in uint32 in place: for every non-NaN pattern (at most 0xFF800000)
    adding at most 0x8000 cannot wrap; NaN patterns are overwritten after."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32)
    t = u >> 16
    t &= 1
    t += 0x7FFF
    t += u
    t >>= 16
    bits = t.astype(np.uint16)
    bits[np.isnan(x32)] = 0x7FC0
    return bits


def f32_from_bf16_bits(bits):
    """Exact float32 value of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _softmax_lastaxis(logits):
    z = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


@dataclass
class Workload:
    """One synthetic problem. Shapes follow the library boundary:
    value [N,S,M,D], spatial_shapes [L,2] as (H,W), level_start [L],
    loc [N,Lq,M,L,K,2] as normalised (x,y), attn [N,Lq,M,L,K], grad_out [N,Lq,M,D]."""

    name: str
    dtype: str  # "f32" or "bf16": the element type of value / out / grad_out
    value: np.ndarray  # float32 (exact upcast when dtype == "bf16")
    spatial_shapes: np.ndarray  # int64 [L,2]
    level_start: np.ndarray  # int64 [L]
    loc: np.ndarray  # float32
    attn: np.ndarray  # float32
    grad_out: np.ndarray | None = None  # float32 (exact upcast when bf16)
    value_bits: np.ndarray | None = None  # uint16 when dtype == "bf16"
    grad_out_bits: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def dims(self):
        N, S, M, D = self.value.shape
        _, Lq, G, L, K, _ = self.loc.shape
        return dict(N=N, S=S, M=M, D=D, L=L, Lq=Lq, K=K, G=G)

    @property
    def points(self):
        d = self.dims
        return d["N"] * d["Lq"] * d["M"] * d["L"] * d["K"]

    def manifest(self):
        def h(a):
            return None if a is None else hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()

        return dict(name=self.name, dtype=self.dtype, dims=self.dims, points=self.points,
                    sha256=dict(value=h(self.value_bits if self.dtype == "bf16" else self.value),
                                loc=h(self.loc), attn=h(self.attn), grad_out=h(self.grad_out)),
                    **self.meta)


def _value(rng, shape, dist, dtype):
    if dist == "normal":
        v = rng.standard_normal(shape)
    elif dist == "uniform":
        v = rng.uniform(-1.0, 1.0, shape)
    else:
        raise ValueError(dist)
    v32 = v.astype(np.float32)
    if dtype == "bf16":
        bits = bf16_bits_from_f32(v32)
        return f32_from_bf16_bits(bits), bits
    return v32, None


def _grad_out(rng, shape, dtype):
    g32 = rng.standard_normal(shape).astype(np.float32)
    if dtype == "bf16":
        bits = bf16_bits_from_f32(g32)
        return f32_from_bf16_bits(bits), bits
    return g32, None


def _attn(rng, N, Lq, M, L, K):
    logits = rng.standard_normal((N, Lq, M, L * K))
    return _softmax_lastaxis(logits).reshape(N, Lq, M, L, K).astype(np.float32)


def encoder_workload(N=1, shapes=COCO_LEVELS, M=8, D=32, K=4, dtype="f32", seed=2,
                     offset_px=2.0, with_grad=False, name="encoder", groups=None):
    """Encoder-style input: every pixel of every level is a query (Lq = S, query
    q is flattened pixel q), its reference point is its pixel centre, and point k
    of head m at level l sits at that reference plus a N(0, offset_px) pixel
    offset per axis in level-l pixels. ``groups``: loc and attn carry that many
    deformable groups instead of M heads."""
    H = M if groups is None else groups
    shapes = tuple(tuple(int(v) for v in hw) for hw in shapes)
    L = len(shapes)
    starts, S = level_starts(shapes)
    Lq = S
    rng = np.random.default_rng(seed)
    value, value_bits = _value(rng, (N, S, M, D), "normal", dtype)
    # Reference point of each query pixel: its centre, normalised by its own level.
    ref = np.empty((Lq, 2), dtype=np.float64)
    for (h, w), s0 in zip(shapes, starts):
        yy, xx = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
        ref[s0:s0 + h * w, 0] = ((xx + 0.5) / w).ravel()
        ref[s0:s0 + h * w, 1] = ((yy + 0.5) / h).ravel()
    wh = np.asarray([[w, h] for h, w in shapes], dtype=np.float64)  # [L,2] as (W,H)
    off = rng.standard_normal((N, Lq, H, L, K, 2)) * offset_px
    loc = (ref[None, :, None, None, None, :] + off / wh[None, None, None, :, None, :]).astype(np.float32)
    attn = _attn(rng, N, Lq, H, L, K)
    g, g_bits = _grad_out(rng, (N, Lq, M, D), dtype) if with_grad else (None, None)
    return Workload(name, dtype, value, np.asarray(shapes, dtype=np.int64), starts, loc, attn,
                    g, value_bits, g_bits,
                    meta=dict(seed=seed, recipe=f"encoder queries=pixels, offsets N(0,{offset_px}px)"))


def decoder_workload(N=2, shapes=COCO_LEVELS, Lq=300, M=8, D=32, K=4, dtype="bf16", seed=3,
                     offset_px=4.0, with_grad=False, name="decoder", groups=None):
    """Decoder-style input: Lq object queries per image with reference points
    uniform in [0,1]^2, plus N(0, offset_px) pixel offsets per level.
    ``groups``: loc and attn carry that many deformable groups instead of M heads."""
    H = M if groups is None else groups
    shapes = tuple(tuple(int(v) for v in hw) for hw in shapes)
    L = len(shapes)
    starts, S = level_starts(shapes)
    rng = np.random.default_rng(seed)
    value, value_bits = _value(rng, (N, S, M, D), "normal", dtype)
    ref = rng.uniform(0.0, 1.0, (N, Lq, 2))
    wh = np.asarray([[w, h] for h, w in shapes], dtype=np.float64)
    off = rng.standard_normal((N, Lq, H, L, K, 2)) * offset_px
    loc = (ref[:, :, None, None, None, :] + off / wh[None, None, None, :, None, :]).astype(np.float32)
    attn = _attn(rng, N, Lq, H, L, K)
    g, g_bits = _grad_out(rng, (N, Lq, M, D), dtype) if with_grad else (None, None)
    return Workload(name, dtype, value, np.asarray(shapes, dtype=np.int64), starts, loc, attn,
                    g, value_bits, g_bits,
                    meta=dict(seed=seed, recipe=f"decoder refs U[0,1]^2, offsets N(0,{offset_px}px)"))


def uniform_workload(N=1, shapes=((16, 16),), Lq=32, M=2, D=8, K=4, dtype="f32", seed=1,
                     lo=-0.1, hi=1.1, with_grad=False, name="uniform"):
    """Locations drawn directly, uniform in [lo,hi]^2, so a share of the samples
    straddles or leaves the map border; value uniform in [-1,1]."""
    shapes = tuple(tuple(int(v) for v in hw) for hw in shapes)
    L = len(shapes)
    starts, S = level_starts(shapes)
    rng = np.random.default_rng(seed)
    value, value_bits = _value(rng, (N, S, M, D), "uniform", dtype)
    loc = rng.uniform(lo, hi, (N, Lq, M, L, K, 2)).astype(np.float32)
    attn = _attn(rng, N, Lq, M, L, K)
    g, g_bits = _grad_out(rng, (N, Lq, M, D), dtype) if with_grad else (None, None)
    return Workload(name, dtype, value, np.asarray(shapes, dtype=np.int64), starts, loc, attn,
                    g, value_bits, g_bits,
                    meta=dict(seed=seed, recipe=f"locations U[{lo},{hi}]^2"))


@dataclass
class FusedWorkload:
    """Raw predictions for the fused entry points: ref [N,Lq,2] reference points
    (normalised x, y) or [N,Lq,4] boxes (cx, cy, w, h); offsets [N,Lq,M,L,K,2]
    in level-l pixels (points) or in box units (boxes); logits [N,Lq,M,L,K];
    all float32. value / grad_out as in Workload."""

    name: str
    dtype: str
    value: np.ndarray
    spatial_shapes: np.ndarray
    level_start: np.ndarray
    ref: np.ndarray
    offsets: np.ndarray
    logits: np.ndarray
    grad_out: np.ndarray | None = None
    value_bits: np.ndarray | None = None
    grad_out_bits: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def dims(self):
        N, S, M, D = self.value.shape
        _, Lq, G, L, K, _ = self.offsets.shape
        return dict(N=N, S=S, M=M, D=D, L=L, Lq=Lq, K=K, G=G, ref_dim=self.ref.shape[-1])

    @property
    def points(self):
        d = self.dims
        return d["N"] * d["Lq"] * d["M"] * d["L"] * d["K"]


def fused_workload(kind="encoder", N=1, shapes=COCO_LEVELS, Lq=300, M=8, D=32, K=4, dtype="f32", seed=8,
                   ref_dim=2, offset_px=2.0, box_offset_sd=0.25, with_grad=False, name=None, groups=None):
    """Raw inputs of the step before the sampling core.

    kind "encoder": every pixel is a query (Lq = S) with its pixel centre as
    reference point (ref_dim 2) and N(0, offset_px) offsets in level pixels.
    kind "decoder": Lq queries per image; points uniform in [0,1]^2 with
    N(0, offset_px) pixel offsets, or (ref_dim 4) boxes with centres uniform in
    [0.05, 0.95]^2 and sizes uniform in [0.02, 0.6], offsets N(0, box_offset_sd)
    in box units. Logits are N(0,1). Draw order: value -> ref -> offsets ->
    logits -> grad_out."""
    shapes = tuple(tuple(int(v) for v in hw) for hw in shapes)
    L = len(shapes)
    starts, S = level_starts(shapes)
    rng = np.random.default_rng(seed)
    value, value_bits = _value(rng, (N, S, M, D), "normal", dtype)
    if kind == "encoder":
        if ref_dim != 2:
            raise ValueError("encoder queries use reference points")
        Lq = S
        ref = np.empty((Lq, 2), dtype=np.float64)
        for (h, w), s0 in zip(shapes, starts):
            yy, xx = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
            ref[s0:s0 + h * w, 0] = ((xx + 0.5) / w).ravel()
            ref[s0:s0 + h * w, 1] = ((yy + 0.5) / h).ravel()
        ref = np.broadcast_to(ref, (N, Lq, 2))
    elif ref_dim == 2:
        ref = rng.uniform(0.0, 1.0, (N, Lq, 2))
    elif ref_dim == 4:
        ref = np.concatenate([rng.uniform(0.05, 0.95, (N, Lq, 2)), rng.uniform(0.02, 0.6, (N, Lq, 2))], -1)
    else:
        raise ValueError(ref_dim)
    sd = offset_px if ref_dim == 2 else box_offset_sd
    H = M if groups is None else groups  # deformable groups, when given
    offsets = (rng.standard_normal((N, Lq, H, L, K, 2)) * sd).astype(np.float32)
    logits = rng.standard_normal((N, Lq, H, L, K)).astype(np.float32)
    g, g_bits = _grad_out(rng, (N, Lq, M, D), dtype) if with_grad else (None, None)
    return FusedWorkload(name or f"fused_{kind}_ref{ref_dim}", dtype, value, np.asarray(shapes, dtype=np.int64),
                         starts, np.ascontiguousarray(ref, dtype=np.float32), offsets, logits, g, value_bits,
                         g_bits, meta=dict(seed=seed, kind=kind, ref_dim=ref_dim))


# The five workloads the library is measured and checked on, plus the K=8
# backward variant (the glossary page "Deformable Attention" gives K as 4 or 8).
def config_workload(name, **override):
    if name == "tiny_fwd":
        kw = dict(N=1, shapes=((16, 16),), Lq=32, M=2, D=8, K=4, dtype="f32", seed=1)
        kw.update(override)
        return uniform_workload(name=name, **kw)
    if name == "encoder_fwd":
        kw = dict(N=1, M=8, D=32, K=4, dtype="f32", seed=2, offset_px=2.0)
        kw.update(override)
        return encoder_workload(name=name, **kw)
    if name == "decoder_fwd_bf16":
        kw = dict(N=2, Lq=300, M=8, D=32, K=4, dtype="bf16", seed=3, offset_px=4.0)
        kw.update(override)
        return decoder_workload(name=name, **kw)
    if name == "batched_encoder_fwd_bf16":
        kw = dict(N=8, M=8, D=32, K=4, dtype="bf16", seed=4, offset_px=2.0)
        kw.update(override)
        return encoder_workload(name=name, **kw)
    if name == "encoder_bwd":
        kw = dict(N=2, M=8, D=32, K=4, dtype="f32", seed=5, offset_px=2.0, with_grad=True)
        kw.update(override)
        return encoder_workload(name=name, **kw)
    if name == "encoder_bwd_k8":
        kw = dict(N=2, M=8, D=32, K=8, dtype="f32", seed=6, offset_px=2.0, with_grad=True)
        kw.update(override)
        return encoder_workload(name=name, **kw)
    raise KeyError(name)


CONFIG_NAMES = ("tiny_fwd", "encoder_fwd", "decoder_fwd_bf16", "batched_encoder_fwd_bf16",
                "encoder_bwd", "encoder_bwd_k8")


def init_pattern_workload(N=1, shape=(16, 16), M=8, D=4, K=2, seed=7, name="init_pattern"):
    """Structured input after the initialisation on page "Deformable DETR"
    (section "Hyperparameters", Initialization): reference points at pixel
    centres, head m's point k offset by k+1 pixels in the m-th of the eight
    compass directions, equal weights 1/(L*K). On a single power-of-two level
    every sample lands exactly on a pixel centre, where the location gradient
    of bilinear interpolation is discontinuous."""
    h, w = shape
    starts, S = level_starts((shape,))
    rng = np.random.default_rng(seed)
    value, _ = _value(rng, (N, S, M, D), "normal", "f32")
    dirs = [(-1, -1), (-1, 0), (-1, 1), (0, -1), (0, 1), (1, -1), (1, 0), (1, 1)]
    yy, xx = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    cx = (xx.ravel() + 0.5)
    cy = (yy.ravel() + 0.5)
    loc = np.empty((N, S, M, 1, K, 2), dtype=np.float64)
    for m in range(M):
        dx, dy = dirs[m % 8]
        for k in range(K):
            loc[:, :, m, 0, k, 0] = (cx + dx * (k + 1)) / w
            loc[:, :, m, 0, k, 1] = (cy + dy * (k + 1)) / h
    attn = np.full((N, S, M, 1, K), 1.0 / K, dtype=np.float32)
    g, _ = _grad_out(rng, (N, S, M, D), "f32")
    return Workload(name, "f32", value, np.asarray([shape], dtype=np.int64), starts,
                    loc.astype(np.float32), attn, g, meta=dict(seed=seed, recipe="init compass pattern"))
