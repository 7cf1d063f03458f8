"""Multi-scale deformable attention sampling core on AMD Instinct MI355X (gfx950).

The forward and backward of the sampling step of MSDeformAttn (page "Deformable
DETR", section "Multi-scale deformable attention") as hand-written HIP kernels
behind a C ABI (include/msda.h, libmsda.so). This package holds the kernels'
sources (csrc/), the in-tree build and the ctypes binding.
"""
from .binding import (MSDA_BF16, MSDA_F32, MSDAError, MSDeformAttnFused,  # noqa: F401
                      MSDeformAttnGrouped, MSDeformAttnSampling, load_library, msda_backward,
                      msda_backward_static, msda_backward_workspace_size, msda_forward, msda_fused_backward,
                      msda_fused_backward_workspace_size,
                      msda_fused_forward, msda_fused_sample, msda_grouped_backward,
                      msda_grouped_forward, msda_grouped_sample, msda_sample,
                      msda_status_string, msda_validate)
