"""libmhc: the mHC hyper-connection hot path on MI355X (gfx950).

The compute lives in the HIP shared library ``libmhc.so`` built from
``csrc/`` (``python -m manifold_constrained_hyper_mhc_amd.build``).  This
package only marshals torch tensors into the C ABI of ``include/mhc.h``:
it checks dtypes, shapes and devices, allocates outputs and the workspace
with torch, and passes raw device pointers and torch's current stream.
Importing it never needs a GPU; the library is loaded on first use and a
missing library is an error, never a fallback.
"""
from .params import Params
from .binding import (FLAG_DEFER_SINKHORN, prepare_sinkhorn, sinkhorn, ERR_EXPIRED, ERR_SCRATCH, MhcError, Prepared, check, coeffs, coeffs_prepacked, fused_outputs, lib, pack_phi, post, post_pre_fused,
                      post_int8, post_int8_pre_fused, post_pre_fused_prepacked, post_pre_fused_prepacked_static, pre, pre_broadcast, prepare_pack_phi,
                      prepare_post_pre_fused_prepacked, schedule, workspace, workspace_error)

__all__ = ["FLAG_DEFER_SINKHORN", "sinkhorn", "prepare_sinkhorn", "Params", "MhcError", "ERR_EXPIRED", "ERR_SCRATCH", "check", "lib", "post_pre_fused_prepacked_static", "coeffs", "coeffs_prepacked", "pre", "post",
           "post_pre_fused", "post_pre_fused_prepacked", "pack_phi", "workspace",
           "schedule", "workspace_error", "Prepared", "prepare_pack_phi", "prepare_post_pre_fused_prepacked",
           "pre_broadcast", "post_int8", "post_int8_pre_fused", "fused_outputs"]
