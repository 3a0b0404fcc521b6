"""Nexus Sampling eviction step for AMD Instinct MI355X (gfx950).

The work runs in libnexus.so (HIP kernels behind the C ABI of include/nexus.h);
this package is its build script and a thin torch-facing binding.  Importing
the binding fails loudly when the library has not been built.
"""

from ._lib import (  # noqa: F401
    NX_OK, NX_EINVAL, NX_EALIAS, NX_EWORKSPACE, NX_EUNSUPPORTED, NX_ENONFINITE, NX_EHIP,
    NX_BF16, NX_F32, NX_COMPACT_COPY, NX_COMPACT_INPLACE, NX_HEADS_UNIFORM, NX_HEADS_GIVEN,
    NX_HEADS_ALLOC, NX_MAX_ALLOC_HEADS, NX_SCRATCH_BYTES, NxDesc, NxUnit, NexusError, LIB_PATH,
    load, status_str, check,
)
from .api import (  # noqa: F401
    NexusConfig, TOPK, workspace_bytes, new_workspace, nx_evict_step, nx_evict_step_noalloc, nx_nexus_weights,
    nx_reservoir_select, nx_kv_compact, nx_head_budgets, make_units, nx_evict_batch,
    nx_read_device_status,
    profile_enable, profile_read,
)
