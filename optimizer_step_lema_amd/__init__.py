"""MI355X-native mixed-precision AdamW hot path of streamed fine-tuning.

The product is the C-ABI library ``liblema.so`` (include/lema.h), built for
gfx950 from csrc/ by ``optimizer_step_lema_amd.build``.  This package is its
thin Python binding.  The library is loaded on first use (``load()``), which
raises ImportError if it has not been built: no step has a non-HIP fallback.
"""
from ._native import LemaError, load  # noqa: F401
from .api import (AccumPlan, AccumSegment, AdamwPlan, AdamwSegment, MergeSegment, SlotPool,  # noqa: F401
                  adamw_constants, adamw_step, device_info, grad_accum, measure_copy,
                  merge_delta, pinned_empty, probe_fp32)
