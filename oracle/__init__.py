"""CPU oracle for the NVFP4 fake-quantized attention QAT path (fp64, NumPy).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.
"""
from .nvfp4 import (E2M1_GRID, E4M3_GRID, GROUP, e2m1_code, e4m3_scale_code,  # noqa: F401
                    fake_nvfp4, fake_nvfp4_values)
from .attention import (qat_backward, qat_backward_head, qat_forward,  # noqa: F401
                        qat_forward_head)
