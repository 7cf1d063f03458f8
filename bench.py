#!/usr/bin/env python3
"""Throughput of the MSDA sampling core (forward + backward) on one MI355X.

One step = msda_forward then msda_backward on the encoder-shape workload: one
800x1333 image's four levels 100x167, 50x84, 25x42, 13x21 (S = Lq = 22223),
M=8 heads, D=32 channels per head (C=256), K=4 points, fp32, every pixel a
query with N(0, 2 px) offsets and softmax weights (synthetic stand-in for
COCO feature maps). Inputs are resident in HBM before timing. Several buffer
sets (inputs and outputs) are cycled so that no step finds its data in the
256 MB Infinity Cache left behind by the previous one.

Prints one JSON line: sampled points/s (N*Lq*M*L*K per step / wall time of
the timed steps, which carry no event markers), per-pass timings from HIP
events on the launch stream (each pass launched back to back between two
events), the HBM roofline of the dominant kernel and the fp64 CPU oracle's
rate on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
KERNEL_SRC = os.path.join(ROOT, "scale_deformable_attention_msda_amd", "csrc", "msda_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "msda_encoder_fwd_bwd_hbm_traffic.md")
TRACE_FILE = os.path.join(ROOT, "profiles", "msda_encoder_fwd_bwd_kernel_stats.md")


def kernel_source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source; None otherwise."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    out = {}
    for key in ("fwd", "bwd"):
        mm = re.search(rf"traffic_bytes_{key}:\s*([0-9.eE+]+)", text)
        if mm:
            out[key] = float(mm.group(1))
    return out or None


def traced_durations():
    """Average pass durations (us) from the committed rocprofv3 kernel-trace
    summary of this benchmark, if it was taken on the current kernel source:
    the forward kernel, and the sum of the backward's kernels per call."""
    if not os.path.exists(TRACE_FILE):
        return None
    text = open(TRACE_FILE).read()
    m = re.search(r"Kernel source sha256 \(first 16 hex\): `([0-9a-f]+)`", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    out = {}
    mm = re.search(r"Forward \(fwd_kernel\) average: ([0-9.]+) us", text)
    if mm:
        out["fwd"] = float(mm.group(1))
    mm = re.search(r"Backward \(sum of the averages of its \d+ kernels per call\): ([0-9.]+) us", text)
    if mm:
        out["bwd"] = float(mm.group(1))
    return out or None


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (no GPU call)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, seconds):
    """The fp64 oracle, as it stands, on the first P (n, q, m) pairs of the same
    workload: forward plus backward (grad_value scatter included)."""
    import numpy as np

    from oracle import msda_backward, msda_forward

    d = w.dims
    args = (w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)

    def run(P):
        idx = np.arange(P)
        n = idx // (d["Lq"] * d["M"])
        q = (idx // d["M"]) % d["Lq"]
        m = idx % d["M"]
        t0 = time.perf_counter()
        msda_forward(*args, pairs=(n, q, m))
        msda_backward(*args, w.grad_out, pairs=(n, q, m), with_grad_value=True)
        return time.perf_counter() - t0

    P = 2048
    t = run(P)
    P = int(min(d["N"] * d["Lq"] * d["M"], max(P, P * seconds / max(t, 1e-3))))
    # when the whole workload takes less than the budget, it is run again (at
    # most four passes) so that the timing covers about `seconds` of work
    t, passes = run(P), 1
    while t < seconds * (passes / (passes + 1)) and passes < 4:
        t += run(P)
        passes += 1
    pts = P * d["L"] * d["K"] * passes
    what = f"first {P} (n,q,m) pairs" if passes == 1 else f"all {P} (n,q,m) pairs, {passes} passes"
    return {"value": pts / t, "unit": "sampled points/s", "cores": 1, "kind": "oracle",
            "sample": f"{what} = {pts} points of the same workload, forward + "
                      f"backward in float64 NumPy, single-threaded ({t:.1f} s)",
            "host_cpus_available": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


_POOL_WORKLOAD = None


def _oracle_chunk(args):
    """Pool worker: forward + backward of the oracle on pairs [p0, p1) (the
    workload is drawn once per worker, outside the timed part)."""
    import numpy as np

    from oracle import msda_backward, msda_forward
    from workloads import config_workload

    global _POOL_WORKLOAD
    if _POOL_WORKLOAD is None:
        _POOL_WORKLOAD = config_workload("encoder_fwd", with_grad=True)
    w = _POOL_WORKLOAD
    p0, p1 = args
    d = w.dims
    idx = np.arange(p0, p1)
    pairs = (idx // (d["Lq"] * d["M"]), (idx // d["M"]) % d["Lq"], idx % d["M"])
    a = (w.value, w.spatial_shapes, w.level_start, w.loc, w.attn)
    t0 = time.perf_counter()
    msda_forward(*a, pairs=pairs)
    msda_backward(*a, w.grad_out, pairs=pairs, with_grad_value=True)
    return time.perf_counter() - t0


def cpu_baseline_pool(w):
    """The same oracle sharded over contiguous pair ranges of the whole workload
    in a process pool of one worker per available host CPU (spawned processes,
    each single-threaded NumPy); wall time of the pool."""
    import multiprocessing as mp

    d = w.dims
    cores = len(os.sched_getaffinity(0))
    total = d["N"] * d["Lq"] * d["M"]
    per = max(1, -(-total // cores))  # the whole workload, split evenly
    chunks = [(k * per, min(total, (k + 1) * per)) for k in range(cores) if k * per < total]
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in env:
        os.environ[k] = "1"
    try:
        with mp.get_context("spawn").Pool(len(chunks)) as pool:
            pool.map(_oracle_chunk, [(0, 64)] * len(chunks))  # imports and the workload, once per worker
            t0 = time.perf_counter()
            pool.map(_oracle_chunk, chunks)
            wall = time.perf_counter() - t0
    finally:
        for k, v in env.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    P = sum(b - a for a, b in chunks)
    pts = P * d["L"] * d["K"]
    return {"value": pts / wall, "unit": "sampled points/s", "cores": len(chunks), "kind": "oracle",
            "sample": f"first {P} (n,q,m) pairs = {pts} points, forward + backward, sharded over "
                      f"{len(chunks)} spawned single-threaded workers ({wall:.1f} s wall)",
            "cpu_model": cpu_model()}


def decoder_latency(msda, torch, dev, layers=6, reps=20):
    """Decoder cross-attention shape (N=2, Lq=300, bf16 values): per-layer time of
    forward+backward issued eagerly vs replayed from one captured HIP graph of
    `layers` layers (launch overhead is what separates them at this size)."""
    import numpy as np

    from workloads import config_workload

    w = config_workload("decoder_fwd_bf16", with_grad=True)
    d = w.dims
    value = torch.from_numpy(w.value_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    g = torch.from_numpy(w.grad_out_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    loc = torch.from_numpy(w.loc).to(dev)
    attn = torch.from_numpy(w.attn).to(dev)
    ss, ls = w.spatial_shapes, w.level_start
    out = torch.empty((d["N"], d["Lq"], d["M"], d["D"]), dtype=torch.bfloat16, device=dev)
    gv = torch.empty(value.shape, dtype=torch.float32, device=dev)
    gl = torch.empty_like(loc)
    ga = torch.empty_like(attn)
    ws = torch.empty(msda.msda_backward_workspace_size(ss, ls, d["N"], d["S"], d["M"], d["D"], d["L"],
                                                       d["Lq"], d["K"], msda.MSDA_BF16),
                     dtype=torch.uint8, device=dev)

    def run(fwd_only=False):
        for _ in range(layers):
            msda.msda_forward(value, ss, ls, loc, attn, out=out)
            if not fwd_only:
                msda.msda_backward(value, ss, ls, loc, attn, g, grad_value=gv, grad_loc=gl, grad_attn=ga,
                                   workspace=ws)

    res = {"workload": "decoder cross-attention: N=2, Lq=300, levels 100x167/50x84/25x42/13x21, M=8, "
                       "D=32, K=4, bf16 values", "layers": layers}
    for name, fwd_only in (("fwd", True), ("fwd_bwd", False)):
        run(fwd_only)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            run(fwd_only)
        torch.cuda.synchronize()
        eager = (time.perf_counter() - t0) / (reps * layers)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run(fwd_only)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run(fwd_only)
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        replay = (time.perf_counter() - t0) / (reps * layers)
        res[name] = {"eager_us_per_layer": round(eager * 1e6, 2), "graph_us_per_layer": round(replay * 1e6, 2)}
    return res


def time_launches(torch, fn, sets, steps):
    """Per-launch times of fn over the buffer sets, cycled. The mean comes from
    `steps` back-to-back launches with one event before the first and one after
    the last, so no event marker sits between launches (a marker costs the GPU
    ~4 us); the percentiles come from a second run with an event between
    consecutive launches, so each of those includes one marker. Returns
    (mean_ms, per_launch_ms array)."""
    import numpy as np

    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        fn(sets[i % len(sets)])
    b.record(stream)
    torch.cuda.synchronize()
    mean_ms = a.elapsed_time(b) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn(sets[i % len(sets)])
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return mean_ms, np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])


def copy_calibration(torch, dev):
    """One 256 MiB device-to-device copy from a source pushed out of the 256 MB
    Infinity Cache by a 1 GiB fill, so its reads and writes go to HBM: the
    known bytes that scale the FETCH_SIZE / WRITE_SIZE counters of a profiled
    run to bytes."""
    src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    flush = torch.zeros(256 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst, flush


def copy_ceiling(torch, dev, reps=5):
    """Measured stream-copy ceiling: a 512 MiB device-to-device copy whose source
    and destination (1 GiB together) exceed the 256 MB Infinity Cache, timed with
    HIP events; bytes read plus bytes written per second (median of reps)."""
    import numpy as np

    src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    nbytes = 2 * src.numel() * 4
    del src, dst
    return nbytes / (float(np.median(ms)) * 1e-3) / 1e9


def fused_passes(msda, torch, dev, steps, rotate):
    """The same encoder shape fed with raw predictions (reference points, pixel
    offsets, logits) through msda_fused_forward / msda_fused_backward, next to
    the unfused route: a torch softmax and location pass, then msda_forward."""
    import numpy as np

    from workloads import COCO_LEVELS, fused_workload

    w = fused_workload("encoder", N=1, shapes=COCO_LEVELS, K=4, seed=2, with_grad=True)
    d = w.dims
    ss, ls = w.spatial_shapes, w.level_start
    size = torch.tensor([[hw[1], hw[0]] for hw in ss.tolist()], dtype=torch.float32, device=dev)
    sets = []
    for _ in range(rotate):
        s = {"value": torch.from_numpy(w.value).to(dev), "ref": torch.from_numpy(w.ref).to(dev),
             "off": torch.from_numpy(w.offsets).to(dev), "logits": torch.from_numpy(w.logits).to(dev),
             "g": torch.from_numpy(w.grad_out).to(dev)}
        s["out"] = torch.empty((d["N"], d["Lq"], d["M"], d["D"]), dtype=torch.float32, device=dev)
        s["gv"] = torch.empty_like(s["value"])
        s["go"] = torch.empty_like(s["off"])
        s["gz"] = torch.empty_like(s["logits"])
        s["gr"] = torch.empty_like(s["ref"])
        s["ws"] = torch.empty(msda.msda_fused_backward_workspace_size(ss, ls, d["N"], d["S"], d["M"], d["D"],
                                                                      d["L"], d["Lq"], d["K"]),
                              dtype=torch.uint8, device=dev)
        sets.append(s)

    def fwd(s):
        msda.msda_fused_forward(s["value"], ss, ls, s["ref"], s["off"], s["logits"], out=s["out"])

    def bwd(s):
        msda.msda_fused_backward(s["value"], ss, ls, s["ref"], s["off"], s["logits"], s["g"], grad_value=s["gv"],
                                 grad_offsets=s["go"], grad_logits=s["gz"], grad_ref=s["gr"], workspace=s["ws"])

    def unfused_fwd(s):
        attn = torch.softmax(s["logits"].reshape(d["N"], d["Lq"], d["M"], -1), -1).reshape(s["logits"].shape)
        loc = s["ref"][:, :, None, None, None, :] + s["off"] / size[None, None, None, :, None, :]
        msda.msda_forward(s["value"], ss, ls, loc, attn, out=s["out"])

    # the unfused route's backward: weights and locations saved by its forward,
    # the core backward, then the softmax and location gradients as torch ops
    for st in sets:
        st["attn"] = torch.softmax(st["logits"].reshape(d["N"], d["Lq"], d["M"], -1), -1).reshape(
            st["logits"].shape).contiguous()
        st["loc"] = (st["ref"][:, :, None, None, None, :] + st["off"] / size[None, None, None, :, None, :]).contiguous()
        st["ws_core"] = torch.empty(msda.msda_backward_workspace_size(ss, ls, d["N"], d["S"], d["M"], d["D"], d["L"],
                                                                      d["Lq"], d["K"]), dtype=torch.uint8, device=dev)

    def unfused_bwd(s):
        gv, gl, ga = msda.msda_backward(s["value"], ss, ls, s["loc"], s["attn"], s["g"], grad_value=s["gv"],
                                        workspace=s["ws_core"])
        a = s["attn"]
        torch.mul(a, ga - (a * ga).sum(dim=(-2, -1), keepdim=True), out=s["gz"])
        torch.div(gl, size[None, None, None, :, None, :], out=s["go"])
        torch.sum(gl, dim=(2, 3, 4), out=s["gr"])

    res = {"workload": "encoder shape as above from raw inputs: reference points at pixel centres, "
                       "N(0,2px) offsets, N(0,1) logits"}
    for name, fn in (("fwd", fwd), ("bwd", bwd), ("unfused_fwd", unfused_fwd), ("unfused_bwd", unfused_bwd)):
        for i in range(3):
            fn(sets[i % rotate])
        mean_ms, ms = time_launches(torch, fn, sets[:rotate], steps)
        res[name] = {"us_mean": round(mean_ms * 1e3, 2), "us_median_with_marker": round(float(np.median(ms)) * 1e3, 2),
                     "points_per_s": w.points / (mean_ms * 1e-3)}
    return res


def grouped_passes(msda, torch, dev, steps, rotate, groups=(1, 2, 4)):
    """The encoder shape with G deformable groups (loc and attn shared by the
    M/G heads of a group): forward and backward per pass, per G."""
    import numpy as np

    from workloads import encoder_workload

    res = {"workload": "encoder shape as above, loc/attn per deformable group"}
    for G in groups:
        w = encoder_workload(N=1, M=8, D=32, K=4, seed=2, groups=G, with_grad=True)
        d = w.dims
        ss, ls = w.spatial_shapes, w.level_start
        sets = []
        for _ in range(rotate):
            s = {"value": torch.from_numpy(w.value).to(dev), "loc": torch.from_numpy(w.loc).to(dev),
                 "attn": torch.from_numpy(w.attn).to(dev), "g": torch.from_numpy(w.grad_out).to(dev)}
            s["out"] = torch.empty((d["N"], d["Lq"], d["M"], d["D"]), dtype=torch.float32, device=dev)
            s["gv"] = torch.empty_like(s["value"])
            s["gl"] = torch.empty_like(s["loc"])
            s["ga"] = torch.empty_like(s["attn"])
            sets.append(s)

        def fwd(s):
            msda.msda_grouped_forward(s["value"], ss, ls, s["loc"], s["attn"], out=s["out"])

        def bwd(s):
            msda.msda_grouped_backward(s["value"], ss, ls, s["loc"], s["attn"], s["g"], grad_value=s["gv"],
                                       grad_loc=s["gl"], grad_attn=s["ga"])

        entry = {}
        for name, fn in (("fwd", fwd), ("bwd", bwd)):
            for i in range(3):
                fn(sets[i % rotate])
            mean_ms, _ = time_launches(torch, fn, sets[:rotate], steps)
            entry[name + "_us_mean"] = round(mean_ms * 1e3, 2)
        entry["points_per_s_fwd_bwd"] = w.points / ((entry["fwd_us_mean"] + entry["bwd_us_mean"]) * 1e-6)
        res[f"G={G}"] = entry
        del sets
    return res


CONFIG_PASSES = (("batched_encoder_fwd_bf16", False, 2), ("encoder_bwd", True, 3), ("encoder_bwd_k8", True, 2),
                 ("encoder_bwd_bf16", True, 3))


def config_passes(msda, torch, dev, steps, only=None):
    """The other configurations of the workload table, timed the same way
    (HIP events around each call, buffer sets cycled so inputs come from HBM):
    batched encoder forward in bf16 (N=8), the encoder backward at N=2 with
    K=4 and K=8, and the same K=4 backward with bf16 value and grad_out.
    Algorithmic bytes: every input read once, every output written once,
    value counted in full (every row is sampled)."""
    import numpy as np

    from workloads import config_workload

    def dev_tensor(w, name):
        if w.dtype == "bf16":
            bits = getattr(w, name + "_bits")
            return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        return torch.from_numpy(getattr(w, name)).to(dev)

    res = {}
    for name, backward, rotate in CONFIG_PASSES:
        if only is not None and name != only:
            continue
        if name == "encoder_bwd_bf16":
            from workloads import encoder_workload
            w = encoder_workload(N=2, M=8, D=32, K=4, dtype="bf16", seed=5, with_grad=True,
                                 name="encoder_bwd_bf16")
        else:
            w = config_workload(name)
        d = w.dims
        ss, ls = w.spatial_shapes, w.level_start
        elem = 2 if w.dtype == "bf16" else 4
        pts = w.points
        vbytes = d["N"] * d["S"] * d["M"] * d["D"] * elem
        obytes = d["N"] * d["Lq"] * d["M"] * d["D"] * elem
        if backward:
            alg = vbytes + obytes + 12 * pts + d["N"] * d["S"] * d["M"] * d["D"] * 4 + 12 * pts
        else:
            alg = vbytes + 12 * pts + obytes
        sets = []
        for _ in range(rotate):
            s = {"value": dev_tensor(w, "value"), "loc": torch.from_numpy(w.loc).to(dev),
                 "attn": torch.from_numpy(w.attn).to(dev)}
            if backward:
                s["g"] = dev_tensor(w, "grad_out")
                s["gv"] = torch.empty(s["value"].shape, dtype=torch.float32, device=dev)
                s["gl"] = torch.empty_like(s["loc"])
                s["ga"] = torch.empty_like(s["attn"])
                s["ws"] = torch.empty(msda.msda_backward_workspace_size(ss, ls, d["N"], d["S"], d["M"], d["D"],
                                                                        d["L"], d["Lq"], d["K"]),
                                      dtype=torch.uint8, device=dev)
            else:
                s["out"] = torch.empty((d["N"], d["Lq"], d["M"], d["D"]), dtype=s["value"].dtype, device=dev)
            sets.append(s)

        def run(s):
            if backward:
                msda.msda_backward(s["value"], ss, ls, s["loc"], s["attn"], s["g"], grad_value=s["gv"],
                                   grad_loc=s["gl"], grad_attn=s["ga"], workspace=s["ws"])
            else:
                msda.msda_forward(s["value"], ss, ls, s["loc"], s["attn"], out=s["out"])

        for i in range(3):
            run(sets[i % rotate])
        mean_ms, ms = time_launches(torch, run, sets[:rotate], steps)
        t = mean_ms * 1e-3
        res[name] = {"workload": f"N={d['N']}, Lq={d['Lq']}, M={d['M']}, D={d['D']}, K={d['K']}, {w.dtype}, "
                                 f"{'backward' if backward else 'forward'}",
                     "us_mean": round(t * 1e6, 2), "us_median_with_marker": round(float(np.median(ms)) * 1e3, 2),
                     "points_per_s": pts / t, "alg_bytes": alg, "alg_GBps": round(alg / t / 1e9, 1),
                     "hbm_frac": round(alg / t / 1e9 / HBM_PEAK_GBPS, 4)}
        del sets
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotate", type=int, default=4, help="buffer sets cycled across steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--main-only", action="store_true",
                    help="time only the encoder forward + backward (no decoder, fused-input or group sections), "
                         "e.g. under a profiler")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (HBM counter calibration)")
    ap.add_argument("--only", default=None,
                    choices=["decoder_latency", "fused_inputs", "deformable_groups"] +
                    [c[0] for c in CONFIG_PASSES],
                    help="run only this secondary section or configuration and print its result "
                         "(e.g. under a profiler); no main step")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only: the sampling core needs no "
                                   "collective (batch or head sharding is exchange-free), so no "
                                   "multi-GPU figure is measured",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import scale_deformable_attention_msda_amd as msda
    from workloads import config_workload

    if args.only is not None:
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        if args.copy_calibration:
            copy_calibration(torch, dev)
        steps = min(args.steps, 20)
        if args.only == "decoder_latency":
            res = decoder_latency(msda, torch, dev)
        elif args.only == "fused_inputs":
            res = fused_passes(msda, torch, dev, min(args.steps, 30), args.rotate)
        elif args.only == "deformable_groups":
            res = grouped_passes(msda, torch, dev, steps, args.rotate)
        else:
            res = config_passes(msda, torch, dev, steps, only=args.only)[args.only]
        print(json.dumps({"section": args.only, "result": res}))
        return

    w = config_workload("encoder_fwd", with_grad=True)
    d = w.dims
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pts = w.points
    U = d["N"] * d["S"] * d["M"] * d["D"] * 4  # bytes of one fp32 value map
    assert d["Lq"] * d["M"] * d["D"] * 4 == U
    # algorithmic bytes: every input read once, every output written once
    # (value counted in full: in this encoder workload every row is sampled)
    b_fwd = U + U + U // 2 + U            # value, loc, attn, out
    b_bwd = U + U + U + U // 2 + U + U + U // 2  # value, grad_out, loc, attn | grad_value, grad_loc, grad_attn

    host = dict(value=torch.from_numpy(w.value), loc=torch.from_numpy(w.loc),
                attn=torch.from_numpy(w.attn), grad_out=torch.from_numpy(w.grad_out))
    sets = []
    for _ in range(args.rotate):
        s = {k: v.to(dev) for k, v in host.items()}
        s["out"] = torch.empty((d["N"], d["Lq"], d["M"], d["D"]), dtype=torch.float32, device=dev)
        s["gv"] = torch.empty_like(s["value"])
        s["gl"] = torch.empty_like(s["loc"])
        s["ga"] = torch.empty_like(s["attn"])
        s["ws"] = torch.empty(msda.msda_backward_workspace_size(
            w.spatial_shapes, w.level_start, d["N"], d["S"], d["M"], d["D"], d["L"], d["Lq"], d["K"]),
            dtype=torch.uint8, device=dev)
        sets.append(s)
    ss, ls = w.spatial_shapes, w.level_start

    def step(s):
        msda.msda_forward(s["value"], ss, ls, s["loc"], s["attn"], out=s["out"])
        msda.msda_backward(s["value"], ss, ls, s["loc"], s["attn"], s["grad_out"],
                           grad_value=s["gv"], grad_loc=s["gl"], grad_attn=s["ga"], workspace=s["ws"])

    if args.copy_calibration:
        copy_calibration(torch, dev)

    for i in range(args.warmup):
        step(sets[i % args.rotate])
    torch.cuda.synchronize()

    # The timed region: exactly `steps` forward + backward steps, nothing else
    # on the stream (no event markers between the passes).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % args.rotate])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = pts / (ms_per_step * 1e-3)

    # Per-pass breakdown: the same `steps` steps again, with an event between
    # the passes and between steps (2 per step, chained), so each pass is
    # timed where it runs in the step; each interval includes one marker.
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(args.steps):
        s = sets[i % args.rotate]
        msda.msda_forward(s["value"], ss, ls, s["loc"], s["attn"], out=s["out"])
        ev[2 * i + 1].record(stream)
        msda.msda_backward(s["value"], ss, ls, s["loc"], s["attn"], s["grad_out"],
                           grad_value=s["gv"], grad_loc=s["gl"], grad_attn=s["ga"], workspace=s["ws"])
        ev[2 * i + 2].record(stream)
    torch.cuda.synchronize()
    fwd_ms = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)])
    bwd_ms = np.array([ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(args.steps)])

    def pass_stats(ms, b):
        t = float(ms.mean()) * 1e-3
        return {"us_mean": round(t * 1e6, 2), "us_median": round(float(np.median(ms)) * 1e3, 2),
                "us_p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
                "us_p90": round(float(np.percentile(ms, 90)) * 1e3, 2),
                "points_per_s": pts / t, "alg_bytes": b, "alg_GBps": round(b / t / 1e9, 1),
                "hbm_frac": round(b / t / 1e9 / HBM_PEAK_GBPS, 4)}

    fwd = pass_stats(fwd_ms, b_fwd)
    bwd = pass_stats(bwd_ms, b_bwd)

    def fwd_only(s):
        msda.msda_forward(s["value"], ss, ls, s["loc"], s["attn"], out=s["out"])

    def bwd_only(s):
        msda.msda_backward(s["value"], ss, ls, s["loc"], s["attn"], s["grad_out"],
                           grad_value=s["gv"], grad_loc=s["gl"], grad_attn=s["ga"], workspace=s["ws"])
    copy_gbps = None if args.main_only else copy_ceiling(torch, dev)
    warm = None
    if not args.main_only:
        # secondary: back-to-back launches on one buffer set (inputs left in the caches)
        s0 = sets[:1]
        for _ in range(3):
            step(s0[0])
        warm = {"fwd_us_mean": round(time_launches(torch, fwd_only, s0, 20)[0] * 1e3, 2),
                "bwd_us_mean": round(time_launches(torch, bwd_only, s0, 20)[0] * 1e3, 2)}
    if copy_gbps:
        for st in (fwd, bwd):
            st["frac_of_copy_ceiling"] = round(st["alg_GBps"] / copy_gbps, 4)
    traffic = measured_traffic()
    dom, dom_name, dom_b = (bwd, "bwd", b_bwd) if bwd["us_mean"] >= fwd["us_mean"] else (fwd, "fwd", b_fwd)
    achieved = dom_b / (dom["us_mean"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": None if traffic is None or dom_name not in traffic else traffic[dom_name],
                "kernel": "msda_backward (all its kernels)" if dom_name == "bwd" else "fwd_kernel",
                "alg_bytes_per_launch": dom_b, "alg_bytes_per_point": dom_b / pts,
                "event_us_mean": dom["us_mean"]}
    traced = traced_durations()
    # the same pass in the committed kernel-trace summary (None if that was
    # taken on another kernel source)
    roofline["trace_us_mean"] = None if traced is None else traced.get(dom_name)

    result = {
        "metric": "sampled points/sec (N*Lq*M*L*K), forward + backward",
        "value": value, "unit": "sampled points/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "encoder-shape fwd+bwd: N=1, levels 100x167/50x84/25x42/13x21, "
                               "S=Lq=22223, M=8, D=32, K=4, fp32, offsets N(0,2px), softmax weights",
                   "points_per_step": pts, "buffer_sets_cycled": args.rotate},
        "roofline": roofline,
        "fwd": fwd, "bwd": bwd,
        "copy_ceiling_GBps": None if copy_gbps is None else round(copy_gbps, 1),
        "warm_same_buffers": warm,
        "kernel_source_sha256": kernel_source_hash(),
    }
    if not args.main_only:
        del sets
        result["decoder_latency"] = decoder_latency(msda, torch, dev)
        result["fused_inputs"] = fused_passes(msda, torch, dev, min(args.steps, 30), args.rotate)
        result["deformable_groups"] = grouped_passes(msda, torch, dev, min(args.steps, 20), args.rotate)
        result["other_configs"] = config_passes(msda, torch, dev, min(args.steps, 20))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        result["cpu_baseline_pool"] = cpu_baseline_pool(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
