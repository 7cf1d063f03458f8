"""CPU oracle (float64, NumPy) of the multi-scale deformable attention sampling core.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding. It shares no
code with the HIP path.
"""
from .msda_oracle import (fused_locations, msda_backward, msda_forward,  # noqa: F401
                          msda_fused_backward, msda_fused_forward, msda_grad_value_rows,
                          msda_grouped_backward, msda_grouped_forward, pixel_coordinate,
                          softmax_weights)
