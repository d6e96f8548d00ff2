"""tp_reduce_mhc_amd: the fused TP-reduce + mHC + RMSNorm sublayer boundary
on AMD Instinct MI355X (gfx950).

The product is libmhcb.so (HIP kernels + C ABI, include/mhcb.h); this
package is its thin Python binding.  See ``tp_reduce_mhc_amd.mhcb``.
"""
from .mhcb import (  # noqa: F401
    EXPORTED, LIBRARY_PATH, MHCB_EALIGN, MHCB_EINVAL, MHCB_ELAUNCH, MHCB_ETIMEOUT,
    MHCB_EUNSUPPORTED, MHCB_OK, GlmBoundary, IndexerProjection, Mailbox, MhcbError, boundary, boundary_glm, finalize,
    mhcb_boundary, mhcb_boundary_glm, mhcb_boundary_glm_noalloc, mhcb_finalize, mhcb_finalize_ex,
    mhcb_finalize_glm, mhcb_finalize_glm_workspace_bytes, finalize_glm, mhcb_workspace_bytes,
    mhcb_workspace_init, mhcb_workspace_status, mhcb_set_token_slices, new_workspace, workspace,
    mhcb_finalize_workspace_bytes, mhcb_workspace_set_spin_limit, workspace_status, mailbox_status,
    mhcb_indexer_workspace_bytes, mhcb_indexer_workspace_init, mhcb_indexer_projection,
    indexer_projection, indexer_workspace,
    mhcb_last_error, mhcb_mailbox, mhcb_mailbox_init, mhcb_mailbox_status, mhcb_mixes,
    mhcb_mxfp8_scale_bytes, mhcb_publish, mhcb_quant_mxfp8, mhcb_version, mixes, quant_mxfp8)

__version__ = mhcb_version()
