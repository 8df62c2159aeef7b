"""MI355X-native NVFP4 fake-quantized attention QAT (hand-written HIP for gfx950).

The compute lives in ``libattnqat.so`` (C ABI in include/attnqat.h);
:mod:`nvfp4_fake_quantized_amd.binding` marshals torch tensors into it.
"""
from .binding import (AttnQatError, attnqat_bwd, attnqat_bwd_workspace_bytes,  # noqa: F401
                      attnqat_check_device, attnqat_check_support, attnqat_fake_nvfp4,
                      attnqat_fwd, attnqat_fwd_workspace_bytes, attnqat_version,
                      attnqat_workspace_layout, make_problem, nvfp4_attention_qat_backward,
                      nvfp4_attention_qat_forward, problem_for, status_string)
