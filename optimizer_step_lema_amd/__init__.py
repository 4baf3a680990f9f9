"""MI355X-native mixed-precision AdamW hot path of streamed fine-tuning.

The product is the C-ABI library ``liblema.so`` (include/lema.h), built for
gfx950 from csrc/ by ``optimizer_step_lema_amd.build``.  This package is its
thin Python binding.  The library is loaded on first use (``load()``), which
raises ImportError if it has not been built: no step has a non-HIP fallback.
"""
from ._native import LemaError, load  # noqa: F401
from .api import (AccumPlan, AccumQ8Plan, AccumQ8Segment, AccumSegment, AdamwPlan,  # noqa: F401
                  AdamwQ8Plan, AdamwQ8Segment, AdamwSegment, FlatState, MergeSegment, Q8,
                  SlotPool, adamw_constants, adamw_step, adamw_step_noalloc, adamw_step_q8,
                  checkpoint_tensors, dequantize_rows, device_info, flat_adamw_state, flat_q8_state,
                  grad_accum, grad_accum_q8, load_checkpoint, measure_copy, merge_delta,
                  pinned_empty, probe_fp32, probe_q8_reciprocal, probe_residency, quantize_rows,
                  save_checkpoint, step_occupancy, table_cache_stats)
