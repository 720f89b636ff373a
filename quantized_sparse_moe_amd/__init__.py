"""MI355X (gfx950) routed-expert MoE layer: a C-ABI HIP library with a thin
Python front end. See ``include/qsmoe.h`` for the entry points."""
from ._lib import EXPORTED, LIB_PATH, MoeError, load  # noqa: F401
from .api import (  # noqa: F401
    DeviceExperts,
    DeviceLayer,
    DeviceQTensor,
    Intermediates,
    combine,
    device_error,
    expert_ffn,
    forward,
    forward_noalloc,
    forward_probed,
    forward_staged,
    mhc_sinkhorn,
    permute,
    probe_mfma,
    probe_stream,
    quantize_affine,
    route,
    router_logits,
    workspace_init,
    ws_region,
)
