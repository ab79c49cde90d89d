"""MI355X (gfx950) MLA tree-verify attention over a paged latent KV cache.

The compute path is the HIP library ``libverify_attn.so`` (C ABI in include/verify_attn.h);
``binding`` marshals torch tensors into it. Importing this package fails if the library has
not been built.
"""
from .binding import (VerifyAttn, VerifyAttnError, verify_attn_create, verify_attn_destroy,  # noqa: F401
                      verify_attn_get_info, verify_attn_last_error,
                      verify_attn_read_device_status, verify_attn_run,
                      verify_attn_workspace_bytes)
