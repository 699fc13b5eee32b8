"""MI355X (gfx950) selective-scan library: Mamba's fused selective-scan forward, its gradients and
the single-token state update, as hand-written HIP kernels behind a plain C ABI.

The Python names mirror the C entry points (``mamba_scan_fwd``, ``mamba_scan_bwd``,
``mamba_state_update``); they only
marshal torch tensors into pointers and sizes.  Importing this package does not load the native
library; the first call does, and raises if it has not been built.
"""

__all__ = ["mamba_scan_fwd", "mamba_scan_fwd_noalloc", "mamba_scan_fwd_conv", "mamba_state_update",
           "mamba_scan_workspace_bytes", "mamba_scan_bwd", "mamba_gemm_bf16",
           "mamba_block_fwd", "mamba_block_workspace_bytes", "mamba_scan_bwd_workspace_bytes", "mamba_status_string",
           "mamba_abi_version", "library_path"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
