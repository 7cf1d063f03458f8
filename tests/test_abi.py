"""The C-ABI library on the host (no GPU needed): it loads, exports every symbol
the header declares, and rejects bad arguments before making any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import scale_deformable_attention_msda_amd as msda
from scale_deformable_attention_msda_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msda.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libmsda.so not built (run __graft_entry__.build())")

COCO = np.array([[100, 167], [50, 84], [25, 42], [13, 21]], dtype=np.int64)
STARTS = np.array([0, 16700, 20900, 21950], dtype=np.int64)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["msda_backward", "msda_backward_static", "msda_backward_workspace_size",
                                    "msda_forward",
                                    "msda_fused_backward", "msda_fused_backward_workspace_size",
                                    "msda_fused_forward", "msda_grouped_backward",
                                    "msda_grouped_backward_workspace_size", "msda_grouped_forward",
                                    "msda_status_string", "msda_validate"]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(7):
        s = msda.msda_status_string(code)
        assert s.startswith("MSDA_")
    assert "unknown" in msda.msda_status_string(99)


def v(*args, **kw):
    return msda.msda_validate(*args, **kw)


def test_validate_accepts_the_workload_shapes():
    assert v(COCO, STARTS, 1, 22223, 8, 32, 4, 22223, 4) == 0
    assert v(COCO, STARTS, 8, 22223, 8, 32, 4, 22223, 4, dtype=1) == 0
    assert v(COCO, STARTS, 2, 22223, 8, 32, 4, 300, 8) == 0
    assert v(COCO, STARTS, 0, 22223, 8, 32, 4, 0, 4) == 0  # empty batch is a no-op


@pytest.mark.parametrize("args,code", [
    ((1, 22223, 8, 32, 4, 100, 4, 2), 2),        # unknown dtype
    ((-1, 22223, 8, 32, 4, 100, 4, 0), 1),       # negative N
    ((1, 22223, 8, 32, 4, -3, 4, 0), 1),         # negative Lq
    ((1, 22223, 0, 32, 4, 100, 4, 0), 1),        # M = 0
    ((1, 22223, 8, 0, 4, 100, 4, 0), 1),         # D = 0
    ((1, 22223, 8, 32, 4, 100, 0, 0), 1),        # K = 0
    ((1, 22223, 8, 32, 4, 100, 17, 0), 2),       # K > 16
    ((1, 22223, 8, 1025, 4, 100, 4, 0), 2),      # D > 1024
    ((1, 22222, 8, 32, 4, 100, 4, 0), 1),        # last level runs past S
    ((1, 22223, 16, 1024, 4, 100, 4, 0), 2),     # S*M*D beyond the per-image limit
])
def test_validate_rejects(args, code):
    N, S, M, D, L, Lq, K, dt = args
    assert v(COCO, STARTS, N, S, M, D, L, Lq, K, dtype=dt) == code


def test_validate_level_geometry():
    lib = binding.load_library()
    ss = np.array([[4, 4], [0, 3]], dtype=np.int64)
    ls = np.array([0, 16], dtype=np.int64)
    assert lib.msda_validate(ss.ctypes.data, ls.ctypes.data, 1, 40, 1, 1, 2, 1, 1, 0) == 1  # H = 0
    ss = np.array([[4, 4], [2, 3]], dtype=np.int64)
    ls = np.array([0, -1], dtype=np.int64)
    assert lib.msda_validate(ss.ctypes.data, ls.ctypes.data, 1, 40, 1, 1, 2, 1, 1, 0) == 1  # start < 0
    ls = np.array([0, 16], dtype=np.int64)
    assert lib.msda_validate(ss.ctypes.data, ls.ctypes.data, 1, 22, 1, 1, 2, 1, 1, 0) == 0
    assert lib.msda_validate(ss.ctypes.data, ls.ctypes.data, 1, 21, 1, 1, 2, 1, 1, 0) == 1
    ss17 = np.ones((17, 2), dtype=np.int64)
    ls17 = np.arange(17, dtype=np.int64)
    assert lib.msda_validate(ss17.ctypes.data, ls17.ctypes.data, 1, 17, 1, 1, 17, 1, 1, 0) == 2
    ssbig = np.array([[1, 1 << 24]], dtype=np.int64)
    assert lib.msda_validate(ssbig.ctypes.data, np.zeros(1, np.int64).ctypes.data,
                             1, 1 << 24, 1, 1, 1, 1, 1, 0) == 2
    assert lib.msda_validate(None, None, 1, 4, 1, 1, 1, 1, 1, 0) == 1  # null host tables


def test_entry_points_reject_bad_pointers_before_any_hip_call():
    lib = binding.load_library()
    ss = COCO.ctypes.data
    ls = STARTS.ctypes.data
    dims = (1, 22223, 8, 32, 4, 22223, 4)
    A = 0x10000  # never dereferenced: every call below fails its checks first
    # null device pointers
    assert lib.msda_forward(None, ss, ls, A, A, A, *dims, 0, None) == 1
    assert lib.msda_forward(A, ss, ls, A, A, None, *dims, 0, None) == 1
    W, WB = 0x100000, 1 << 40  # a workspace pointer and a size large enough for any check
    assert lib.msda_backward(A, ss, ls, A, A, A, None, A, A, *dims, 0, W, WB, None) == 1
    assert lib.msda_backward(A, ss, ls, A, A, None, A, A, A, *dims, 0, W, WB, None) == 1
    # missing or short workspace
    assert lib.msda_backward(A, ss, ls, A, A, A, A, A, A, *dims, 0, None, WB, None) == 5
    assert lib.msda_backward(A, ss, ls, A, A, A, A, A, A, *dims, 0, W, 1024, None) == 5
    assert lib.msda_backward(A, ss, ls, A, A, A, A, A, A, *dims, 0, W + 64, WB, None) == 3
    # misaligned: loc must be 8-byte aligned, fp32 arrays 4-byte, bf16 2-byte
    assert lib.msda_forward(A, ss, ls, A + 4, A, A, *dims, 0, None) == 3
    assert lib.msda_forward(A + 2, ss, ls, A, A, A, *dims, 0, None) == 3
    assert lib.msda_forward(A + 1, ss, ls, A, A, A, *dims, 1, None) == 3
    assert lib.msda_backward(A, ss, ls, A, A, A, A + 2, A, A, *dims, 0, W, WB, None) == 3
    assert lib.msda_backward(A, ss, ls, A, A, A, A, A + 4, A, *dims, 0, W, WB, None) == 3
    # invalid shapes reach no pointer at all
    assert lib.msda_forward(A, ss, ls, A, A, A, 1, 22223, 8, 32, 4, 22223, 17, 0, None) == 2
    assert lib.msda_backward(A, ss, ls, A, A, A, A, A, A, 1, 22223, 8, 32, 4, 22223, 4, 5, W, WB, None) == 2
    # an empty problem is a successful no-op without touching memory
    assert lib.msda_forward(None, ss, ls, None, None, None, 0, 22223, 8, 32, 4, 10, 4, 0, None) == 0
    assert lib.msda_forward(None, ss, ls, None, None, None, 1, 22223, 8, 32, 4, 0, 4, 0, None) == 0


def test_fused_entry_points_reject_bad_arguments_before_any_hip_call():
    lib = binding.load_library()
    ss = COCO.ctypes.data
    ls = STARTS.ctypes.data
    dims = (1, 22223, 8, 32, 4, 22223, 4)
    A, W, WB = 0x10000, 0x100000, 1 << 40
    # reference layout: 2 (points) or 4 (boxes) floats per query
    for rd in (0, 1, 3, 5, -2):
        assert lib.msda_fused_forward(A, ss, ls, A, rd, A, A, A, *dims, 0, None) == 1
        assert lib.msda_fused_backward(A, ss, ls, A, rd, A, A, A, A, A, A, A, *dims, 0, W, WB, None) == 1
    # null reference, null outputs; grad_ref alone may be null (not computed)
    assert lib.msda_fused_forward(A, ss, ls, None, 2, A, A, A, *dims, 0, None) == 1
    assert lib.msda_fused_forward(A, ss, ls, A, 4, A, A, None, *dims, 0, None) == 1
    assert lib.msda_fused_backward(A, ss, ls, None, 4, A, A, A, A, A, A, A, *dims, 0, W, WB, None) == 1
    assert lib.msda_fused_backward(A, ss, ls, A, 2, A, A, A, A, None, A, None, *dims, 0, W, WB, None) == 1
    # alignment: ref and offsets 8 bytes, logits and grad_ref 4 bytes
    assert lib.msda_fused_forward(A, ss, ls, A + 4, 2, A, A, A, *dims, 0, None) == 3
    assert lib.msda_fused_forward(A, ss, ls, A, 2, A + 4, A, A, *dims, 0, None) == 3
    assert lib.msda_fused_forward(A, ss, ls, A, 2, A, A + 2, A, *dims, 0, None) == 3
    assert lib.msda_fused_backward(A, ss, ls, A, 4, A, A, A, A, A, A, A + 2, *dims, 0, W, WB, None) == 3
    assert lib.msda_fused_backward(A, ss, ls, A, 4, A, A, A, A, A + 4, A, A, *dims, 0, W, WB, None) == 3
    # workspace as for the sampling core's backward
    assert lib.msda_fused_backward(A, ss, ls, A, 4, A, A, A, A, A, A, A, *dims, 0, W, 1024, None) == 5
    # empty problems are no-ops
    assert lib.msda_fused_forward(None, ss, ls, None, 2, None, None, None, 0, 22223, 8, 32, 4, 10, 4, 0,
                                  None) == 0


def test_grouped_entry_points_check_groups():
    lib = binding.load_library()
    ss = COCO.ctypes.data
    ls = STARTS.ctypes.data
    A, W, WB = 0x10000, 0x100000, 1 << 40
    # G must divide M
    for G in (0, -1, 3, 16):
        dims = (1, 22223, 8, 32, 4, 22223, 4, G)
        assert lib.msda_grouped_forward(A, ss, ls, A, A, A, *dims, 0, None) == 1
        assert lib.msda_grouped_backward(A, ss, ls, A, A, A, A, A, A, *dims, 0, W, WB, None) == 1
    # (M/G)*D beyond the channel limit: 8 heads of 256 channels in one group
    assert lib.msda_grouped_forward(A, ss, ls, A, A, A, 1, 22223, 8, 256, 4, 22223, 4, 1, 0, None) == 2
    # a group's workspace is the core's with G heads of (M/G)*D channels
    n_g = ctypes.c_size_t(0)
    assert lib.msda_grouped_backward_workspace_size(ss, ls, 1, 22223, 8, 32, 4, 22223, 4, 2, 0,
                                                    ctypes.byref(n_g)) == 0
    assert n_g.value == msda.msda_backward_workspace_size(COCO, STARTS, 1, 22223, 2, 128, 4, 22223, 4)
    # misalignment is checked on the group shape: 128 bf16 channels, value 2 bytes off
    assert lib.msda_grouped_forward(A + 1, ss, ls, A, A, A, 1, 22223, 8, 32, 4, 22223, 4, 2, 1, None) == 3


def test_workspace_size_and_overlapping_levels():
    lib = binding.load_library()
    n = msda.msda_backward_workspace_size(COCO, STARTS, 2, 22223, 8, 32, 4, 22223, 4)
    samples = 2 * 22223 * 8 * 4 * 4
    pairs = 2 * 22223 * 8
    assert 64 * samples <= n <= 64 * samples + (1 << 20)
    nf = msda.msda_fused_backward_workspace_size(COCO, STARTS, 2, 22223, 8, 32, 4, 22223, 4)
    assert nf == n + 12 * samples + 16 * pairs or 0 < nf - (n + 12 * samples + 16 * pairs) <= 3 * 256
    # overlapping level row ranges are rejected
    ss = np.array([[4, 4], [2, 2]], dtype=np.int64)
    ls = np.array([0, 14], dtype=np.int64)
    assert lib.msda_validate(ss.ctypes.data, ls.ctypes.data, 1, 40, 1, 1, 2, 1, 1, 0) == 1
    ls = np.array([0, 16], dtype=np.int64)
    assert lib.msda_validate(ss.ctypes.data, ls.ctypes.data, 1, 40, 1, 1, 2, 1, 1, 0) == 0


def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", binding.LIB_PATH + ".absent")
    with pytest.raises(RuntimeError, match="missing"):
        binding.load_library()


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 4, 1, 1)
    loc = torch.zeros(1, 1, 1, 1, 1, 2)
    attn = torch.zeros(1, 1, 1, 1, 1)
    with pytest.raises(ValueError, match="device tensor"):
        msda.msda_forward(x, [[2, 2]], [0], loc, attn)


def test_binding_host_arrays():
    """spatial_shapes / level_start: an int64 C-contiguous array of the right
    shape is passed through as is; other integer arrays, lists and CPU tensors
    are converted; a wrong entry count raises before any library call."""
    torch = pytest.importorskip("torch")
    ss = np.array([[100, 167], [50, 84]], dtype=np.int64)
    assert binding._host_i64(ss, (2, 2), "spatial_shapes") is ss
    for a in (ss.astype(np.int32), ss.tolist(), torch.from_numpy(ss.copy()), np.asfortranarray(ss)):
        got = binding._host_i64(a, (2, 2), "spatial_shapes")
        assert got.dtype == np.int64 and got.flags.c_contiguous and np.array_equal(got, ss)
    flat = binding._host_i64(np.array([0, 16700]), (2,), "level_start")
    assert flat.shape == (2,) and flat.dtype == np.int64
    with pytest.raises(ValueError, match="3 entries"):
        binding._host_i64([0, 1, 2], (2,), "level_start")


def test_header_compiles_as_c_and_links(tmp_path):
    """A plain C11 program (tests/c/abi_host.c) includes the header, links the
    library and runs its host-side paths: validation, status strings,
    workspace size and the checks made before any HIP call."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    rocm_inc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
    lib_dir = os.path.dirname(binding.LIB_PATH)
    exe = str(tmp_path / "abi_host")
    cmd = [cc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", rocm_inc,
           os.path.join(ROOT, "tests", "c", "abi_host.c"), "-o", exe,
           "-L", lib_dir, "-lmsda", "-Wl,-rpath," + lib_dir]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.strip().endswith("OK")


def test_static_scratch_backward_rejects_oversized_problems_before_any_hip_call():
    """The allocation-free backward checks the workspace it would need against its
    static scratch on the host: an encoder-sized problem is refused with
    MSDA_ERROR_SCRATCH (null device pointers are never touched), and a bad
    argument still gets the ordinary validation status."""
    lib = binding.load_library()
    ss, ls = COCO.ctypes.data, STARTS.ctypes.data
    st = lib.msda_backward_static(None, ss, ls, None, None, None, None, None, None,
                                  1, 22223, 8, 32, 4, 22223, 4, 0, None)
    assert st == binding.MSDA_ERROR_SCRATCH
    assert "static scratch" in msda.msda_status_string(st)
    need = msda.msda_backward_workspace_size(COCO, STARTS, 1, 22223, 8, 32, 4, 22223, 4)
    assert need > (64 << 20)
    st = lib.msda_backward_static(None, ss, ls, None, None, None, None, None, None,
                                  1, 22223, 8, 32, 4, 22223, 17, 0, None)
    assert st == binding.MSDA_ERROR_NOT_SUPPORTED  # K > 16
