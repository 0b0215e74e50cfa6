"""libfp4idx: fused q/k RoPE + E2M1/UE8M0 pack + paged index-cache store for gfx950.

The compute path is the HIP library ``libfp4idx.so`` (C-ABI in
``include/fp4idx.h``); ``pack_token_amd.fp4idx`` is its thin ctypes binding.
Importing this package does not load the library; the binding does, and it
raises if the library is missing.
"""
__all__ = ["fp4idx", "workloads"]
