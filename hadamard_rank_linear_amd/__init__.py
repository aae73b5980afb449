"""MI355X-native (gfx950) HLQ/HOT linear-layer backward.

The compute lives in ``libhlq.so`` (hand-written HIP kernels behind the C ABI
of ``include/hlq.h``); :mod:`hadamard_rank_linear_amd.hlq` is its ctypes
binding.  Binding names are re-exported here on first access, which loads the
library and raises ImportError if it has not been built.
"""
from __future__ import annotations

import importlib

_BINDING_NAMES = {
    "hlq_compress_act", "hlq_linear_forward", "hlq_linear_backward", "hlq_linear_backward_workspace_size",
    "hlq_workspace_layout_query", "hlq_linear_backward_noalloc", "HLQ_NOALLOC_SCRATCH_BYTES",
    "hlq_gemm_pair_acc", "hlq_gemm_gx_acc", "hlq_gemm_gw_acc", "HLQError",
    "HLQ_F32", "HLQ_BF16", "HLQ_PER_TOKEN", "HLQ_PER_TENSOR", "HLQ_SUM", "HLQ_MEAN",
    "version", "status_string", "lib_handle", "LIB_PATH", "EXPORTED", "STEP_NAMES",
    "HLQ_STEPS_ALL", "hlq_lqs_workspace_size", "hlq_lqs_accumulate", "hlq_lqs_select",
    "HLQ_LQS_STATS", "HLQ_LQS_THRESHOLD", "hlq_conv_backward",
    "hlq_conv_backward_workspace_size", "hlq_conv_gemm_acc", "hlq_linear_backward_ablation",
    "hlq_ablation_workspace_size", "VARIANT_NAMES", "HLQ_VAR_HQ4", "HLQ_VAR_Q4", "HLQ_VAR_HLA8_INT",
    "HLQ_VAR_HLA8_EXT",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        return getattr(importlib.import_module(".hlq", __name__), name)
    raise AttributeError(name)
