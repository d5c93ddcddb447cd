"""Lightning Attention-2 tiled causal linear attention on MI355X (gfx950).

The HIP library (``lib/libla2.so``, C ABI in ``include/la2.h``) is loaded on
first use of the binding; ``inputs`` (seeded synthetic workloads) imports
without it.
"""
from .binding import (  # noqa: F401
    LA2Error,
    LA2Function,
    LA2StateFunction,
    backward,
    backward_normalized,
    backward_state,
    decode_step,
    forward,
    forward_normalized,
    forward_serial,
    forward_state,
    la2_abi_version,
    la2_backward,
    la2_backward_normalized,
    la2_backward_normalized_saved,
    la2_backward_saved,
    la2_backward_state,
    la2_decode_step,
    la2_forward,
    la2_forward_noalloc,
    la2_forward_normalized,
    la2_forward_serial,
    la2_forward_state,
    la2_normalized_workspace_bytes,
    la2_status_string,
    la2_workspace_bytes,
    lightning_attention,
    lightning_attention_state,
    load_library,
    normalized_workspace_for,
    workspace_for,
)
