"""Fused linear cross-entropy for AMD MI355X (gfx950): HIP kernels behind the
C ABI of include/lce.h, with a thin ctypes binding (``lm_head_linear_amd.lce``)."""
from . import lce  # noqa: F401
from .lce import (LceError, backward, ce_logits, distill, forward, forward_backward,  # noqa: F401
                  lce_backward, lce_ce_logits_fwd_bwd, lce_chunk_check, lce_dims_check,
                  lce_distill_fwd_bwd, lce_distill_workspace_bytes, lce_forward,
                  lce_forward_backward, lce_forward_backward_workspace_bytes, lce_logit_cells,
                  lce_loss_fetch,
                  lce_peak_cells, lce_shard_backward, lce_shard_forward, lce_shard_merge,
                  lce_status_name, lce_work_fits, lce_workspace_bytes)
