"""Exact IO-aware attention forward (FlashAttention) for MI355X / gfx950.

The computation runs in the HIP kernels of ``libfa.so`` (C ABI in
``include/fa.h``); this package only marshals torch tensors into that call.
There is no CPU or PyTorch fallback: if the library is missing or the device
is not gfx950, calls raise.
"""
from ._lib import (  # noqa: F401
    FA_BF16, FA_F16, FA_F32, STATUS, check_seqlens, debug_force_order, debug_forced_order,
    kernel_name, kernel_name_ex, kernel_name_kv, load, status_string,
    bwd_workspace_bytes, num_splits, split_workspace_bytes, supported, version,
    workspace_bytes,
)
from .autograd import attention  # noqa: F401
from .bwd import bwd  # noqa: F401
from .fwd import fwd, flops, pack_v  # noqa: F401
