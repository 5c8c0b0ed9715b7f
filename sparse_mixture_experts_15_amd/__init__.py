"""MI355X (gfx950) sparse Mixture-of-Experts feed-forward layer, forward pass.

The layer runs in hand-written HIP kernels behind the C ABI declared in
``include/moe.h`` (library ``lib/libmoe.so``); ``binding`` exposes the same
entry points to Python with torch tensors as device buffers, and ``layer``
wraps them in a small object that owns a handle and its workspace.
"""
from .binding import (EXPORTS, MoEError, load_library, make_desc, moe_combine,  # noqa: F401
                      moe_create, moe_desc, moe_destroy, moe_expert_ffn, moe_forward,
                      moe_permute, moe_profile_results, moe_profile_start, moe_profile_stop,
                      moe_route, moe_shared_expert, moe_workspace_size)
