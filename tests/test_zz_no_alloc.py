"""The allocation-free backward (msda_backward_static, for callers that cannot
allocate) against msda_backward with a caller's workspace: two calls in a row,
the second on a smaller problem, so the second runs on whatever the first left
in the library's static scratch."""
import numpy as np
import pytest
import torch

import scale_deformable_attention_msda_amd as msda
from tests.gpu_util import assert_f32, device_inputs, note, to_f64
from workloads import encoder_workload, uniform_workload

pytestmark = pytest.mark.gpu

SMALL_LEVELS = ((20, 34), (10, 17), (5, 9), (3, 5))


def _both(w):
    value, loc, attn, grad_out = device_inputs(w)
    ss, ls = w.spatial_shapes, w.level_start
    ref = msda.msda_backward(value, ss, ls, loc, attn, grad_out)
    got = (torch.full_like(value, float("nan"), dtype=torch.float32), torch.full_like(loc, float("nan")),
           torch.full_like(attn, float("nan")))
    msda.msda_backward_static(value, ss, ls, loc, attn, grad_out, *got)
    torch.cuda.synchronize()
    return [to_f64(t) for t in ref], [to_f64(t) for t in got]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_static_scratch_backward_matches_workspace_backward(dtype):
    # dense route (tile sort in the scratch), then a smaller problem on it
    big = encoder_workload(N=2, shapes=SMALL_LEVELS, M=8, D=32, K=4, dtype=dtype, seed=901, with_grad=True)
    small = uniform_workload(N=1, shapes=((9, 12), (5, 6)), Lq=40, M=4, D=32, K=4, dtype=dtype, seed=902,
                             with_grad=True)
    d = big.dims
    need = msda.msda_backward_workspace_size(big.spatial_shapes, big.level_start, d["N"], d["S"], d["M"], d["D"],
                                             d["L"], d["Lq"], d["K"])
    assert 0 < need <= 64 << 20
    for name, w in (("encoder-shaped N=2 small maps", big), ("uniform N=1 two levels", small)):
        note(f"static-scratch backward vs workspace backward: {name} {dtype}")
        (rgv, rgl, rga), (gv, gl, ga) = _both(w)
        assert_f32("grad_value", gv, rgv)
        # grad_loc and grad_attn come from the same deterministic kernels
        assert np.array_equal(gl, rgl), name
        assert np.array_equal(ga, rga), name
