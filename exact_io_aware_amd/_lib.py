"""ctypes binding of libfa.so (include/fa.h).  Argument marshalling only."""
from __future__ import annotations

import contextlib
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
POISON_LIB_PATH = os.path.join(os.path.dirname(LIB_PATH), "libfa_poison.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK = 0
STATUS = {
    "FA_OK": 0, "FA_ERR_NULL": -1, "FA_ERR_SHAPE": -2, "FA_ERR_HEADDIM": -3,
    "FA_ERR_GQA": -4, "FA_ERR_DTYPE": -5, "FA_ERR_ALIGN": -6, "FA_ERR_ALIAS": -7,
    "FA_ERR_SCALE": -8, "FA_ERR_DEVICE": -9, "FA_ERR_LAUNCH": -10,
    "FA_ERR_WORKSPACE": -11, "FA_ERR_ALLOC": -12, "FA_ERR_SEQLENS": -13,
    "FA_ERR_SCRATCH": -14,
}

_lib = None


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m exact_io_aware_amd.build` "
            "(there is no fallback path)")
    return _bind(ctypes.CDLL(path))


def load() -> ctypes.CDLL:
    """Load libfa.so once.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


@contextlib.contextmanager
def poisoned_lds():
    """Test aid: while the block runs, every call goes to libfa_poison.so,
    the same kernels built with their LDS filled with NaN before use (so a
    read of LDS the kernel never wrote shows up as NaN).  Not thread-safe."""
    global _lib
    saved = load()
    _lib = _open(POISON_LIB_PATH)
    try:
        yield _lib
    finally:
        _lib = saved


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, vp, i, i]
    lib.fa_fwd.restype = i
    z = ctypes.c_size_t
    lib.fa_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_workspace_bytes.restype = z
    lib.fa_pack_v.argtypes = [vp, vp, z, i, i, i, i, vp, vp, i]
    lib.fa_pack_v.restype = i
    lib.fa_fwd_packed.argtypes = [vp, vp, vp, z, vp, vp, i, i, i, i, i, i, f, vp, vp, i, i]
    lib.fa_fwd_packed.restype = i
    lib.fa_fwd_kv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, vp, i, i]
    lib.fa_fwd_kv.restype = i
    lib.fa_fwd_kv_packed.argtypes = [vp, vp, vp, z, vp, vp, i, i, i, i, i, i, i, f, vp, vp, vp,
                                     i, i]
    lib.fa_fwd_kv_packed.restype = i
    lib.fa_num_splits.argtypes = [i, i, i, i, i, i, i]
    lib.fa_num_splits.restype = i
    lib.fa_split_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_split_workspace_bytes.restype = z
    lib.fa_fwd_kv_split_packed.argtypes = [vp, vp, vp, z, vp, vp, i, i, i, i, i, i, i, f, vp,
                                           vp, i, vp, z, vp, i, i]
    lib.fa_fwd_kv_split_packed.restype = i
    lib.fa_fwd_kv_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, i, vp,
                                    z, vp, i, i]
    lib.fa_fwd_kv_split.restype = i
    lib.fa_fwd_kv_split_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp,
                                            i, vp, i, i]
    lib.fa_fwd_kv_split_noalloc.restype = i
    lib.fa_noalloc_scratch_bytes.argtypes = []
    lib.fa_noalloc_scratch_bytes.restype = z
    lib.fa_fwd_sparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, vp, i, i,
                                  vp, i, i]
    lib.fa_fwd_sparse.restype = i
    lib.fa_fwd_sparse_packed.argtypes = [vp, vp, vp, z, vp, vp, i, i, i, i, i, i, i, f, vp, vp,
                                         vp, i, i, vp, i, i]
    lib.fa_fwd_sparse_packed.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = z
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, vp, z,
                           vp, i, i, i]
    lib.fa_bwd.restype = i
    lib.fa_fwd_check.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i, i]
    lib.fa_fwd_check.restype = i
    lib.fa_kernel_name.argtypes = [i, i, i, i, i]
    lib.fa_kernel_name.restype = ctypes.c_char_p
    lib.fa_kernel_name_kv.argtypes = [i, i, i, i, i, i, i, i]
    lib.fa_kernel_name_kv.restype = ctypes.c_char_p
    lib.fa_kernel_name_ex.argtypes = [i, i, i, i, i, i, i, i, i, i]
    lib.fa_kernel_name_ex.restype = ctypes.c_char_p
    lib.fa_check_seqlens.argtypes = [vp, i, i]
    lib.fa_check_seqlens.restype = i
    lib.fa_supported.argtypes = [i, i, i]
    lib.fa_supported.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    lib.fa_debug_force_order.argtypes = [i]
    lib.fa_debug_force_order.restype = i
    lib.fa_debug_forced_order.argtypes = []
    lib.fa_debug_forced_order.restype = i
    lib.fa_build_flags.argtypes = []
    lib.fa_build_flags.restype = i
    return lib


def status_string(status: int) -> str:
    return load().fa_status_string(status).decode()


def version() -> int:
    return load().fa_version()


def debug_force_order(order: int) -> None:
    """fa_debug_force_order: -1 restores the library's own launch order; 0-3
    force unit-major / +XCD remap / row-block-major / +XCD remap."""
    st = load().fa_debug_force_order(order)
    if st != 0:
        raise ValueError(f"fa_debug_force_order({order}): {status_string(st)}")


def debug_forced_order() -> int:
    """The launch order currently forced (-1: the library's own choice)."""
    return load().fa_debug_forced_order()


def kernel_name(in_dtype: int, d: int, causal: bool, varlen: bool, out_dtype: int):
    s = load().fa_kernel_name(in_dtype, d, int(causal), int(varlen), out_dtype)
    return None if s is None else s.decode()


def kernel_name_kv(in_dtype: int, d: int, causal: bool, varlen: bool, out_dtype: int,
                   Hq: int, Hkv: int, Nq: int):
    """fa_kernel_name_kv: the kernel fa_fwd_kv runs for this query count."""
    s = load().fa_kernel_name_kv(in_dtype, d, int(causal), int(varlen), out_dtype, Hq, Hkv, Nq)
    return None if s is None else s.decode()


def kernel_name_ex(in_dtype: int, d: int, causal: bool, varlen: bool, out_dtype: int,
                   Hq: int, Hkv: int, Nq: int, sparse: bool = False, vt_packed: bool = False):
    """fa_kernel_name_ex: the kernel a given entry point runs (block-sparse
    and/or packed V)."""
    s = load().fa_kernel_name_ex(in_dtype, d, int(causal), int(varlen), out_dtype, Hq, Hkv, Nq,
                                 int(sparse), int(vt_packed))
    return None if s is None else s.decode()


def check_seqlens(cu_seqlens_host, B: int, n_max: int) -> int:
    """fa_check_seqlens on a host int32 array (a numpy array or None)."""
    if cu_seqlens_host is None:
        return load().fa_check_seqlens(None, B, n_max)
    import numpy as np
    a = np.ascontiguousarray(cu_seqlens_host, dtype=np.int32)
    return load().fa_check_seqlens(a.ctypes.data, B, n_max)


def supported(in_dtype: int, d: int, causal: bool) -> bool:
    return bool(load().fa_supported(in_dtype, d, int(causal)))


def fwd_check(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, cu_seqlens,
              in_dtype, out_dtype) -> int:
    """fa_fwd_check with raw integer addresses (no GPU needed)."""
    return load().fa_fwd_check(q, k, v, o, lse, B, Hq, Hkv, N, d, int(causal),
                               scale, cu_seqlens, in_dtype, out_dtype)


def fwd_raw(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, cu_seqlens,
            stream, in_dtype, out_dtype) -> int:
    """fa_fwd with raw integer device addresses and a raw hipStream_t."""
    return load().fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, int(causal), scale,
                         cu_seqlens, stream, in_dtype, out_dtype)


def workspace_bytes(B, Hkv, N, d, in_dtype) -> int:
    """fa_workspace_bytes: size of the packed-V workspace (0 if none)."""
    return load().fa_workspace_bytes(B, Hkv, N, d, in_dtype)


def pack_v_raw(v, vt, vt_bytes, B, Hkv, N, d, cu_seqlens, stream, in_dtype) -> int:
    """fa_pack_v with raw integer device addresses and a raw hipStream_t."""
    return load().fa_pack_v(v, vt, vt_bytes, B, Hkv, N, d, cu_seqlens, stream, in_dtype)


def fwd_packed_raw(q, k, vt, vt_bytes, o, lse, B, Hq, Hkv, N, d, causal, scale,
                   cu_seqlens, stream, in_dtype, out_dtype) -> int:
    """fa_fwd_packed with raw integer device addresses and a raw hipStream_t."""
    return load().fa_fwd_packed(q, k, vt, vt_bytes, o, lse, B, Hq, Hkv, N, d, int(causal),
                                scale, cu_seqlens, stream, in_dtype, out_dtype)


def fwd_kv_raw(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, cu_q, cu_k,
               stream, in_dtype, out_dtype) -> int:
    """fa_fwd_kv with raw integer device addresses and a raw hipStream_t."""
    return load().fa_fwd_kv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, int(causal), scale,
                            cu_q, cu_k, stream, in_dtype, out_dtype)


def fwd_kv_packed_raw(q, k, vt, vt_bytes, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                      cu_q, cu_k, stream, in_dtype, out_dtype) -> int:
    """fa_fwd_kv_packed with raw integer device addresses and a raw hipStream_t."""
    return load().fa_fwd_kv_packed(q, k, vt, vt_bytes, o, lse, B, Hq, Hkv, Nq, Nk, d,
                                   int(causal), scale, cu_q, cu_k, stream, in_dtype, out_dtype)


def num_splits(B, Hq, Hkv, Nq, Nk, d, in_dtype) -> int:
    """fa_num_splits: split-KV count for these sizes on the current device."""
    return load().fa_num_splits(B, Hq, Hkv, Nq, Nk, d, in_dtype)


def split_workspace_bytes(B, Hq, Nq, d, n_splits) -> int:
    """fa_split_workspace_bytes: bytes of the split-KV partials."""
    return load().fa_split_workspace_bytes(B, Hq, Nq, d, n_splits)


def fwd_kv_split_packed_raw(q, k, vt, vt_bytes, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                            cu_q, cu_k, n_splits, part, part_bytes, stream, in_dtype,
                            out_dtype) -> int:
    """fa_fwd_kv_split_packed with raw integer device addresses."""
    return load().fa_fwd_kv_split_packed(q, k, vt, vt_bytes, o, lse, B, Hq, Hkv, Nq, Nk, d,
                                         int(causal), scale, cu_q, cu_k, n_splits, part,
                                         part_bytes, stream, in_dtype, out_dtype)


def fwd_kv_split_raw(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, cu_q, cu_k,
                     n_splits, part, part_bytes, stream, in_dtype, out_dtype) -> int:
    """fa_fwd_kv_split with raw integer device addresses."""
    return load().fa_fwd_kv_split(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, int(causal), scale,
                                  cu_q, cu_k, n_splits, part, part_bytes, stream, in_dtype,
                                  out_dtype)


def fwd_kv_split_noalloc_raw(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, cu_q,
                             cu_k, n_splits, stream, in_dtype, out_dtype) -> int:
    """fa_fwd_kv_split_noalloc with raw integer device addresses."""
    return load().fa_fwd_kv_split_noalloc(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, int(causal),
                                          scale, cu_q, cu_k, n_splits, stream, in_dtype,
                                          out_dtype)


def noalloc_scratch_bytes() -> int:
    """fa_noalloc_scratch_bytes: size of the library's fixed scratch."""
    return load().fa_noalloc_scratch_bytes()


def bwd_workspace_bytes(B, Hq, Hkv, N, d, in_dtype) -> int:
    """fa_bwd_workspace_bytes."""
    return load().fa_bwd_workspace_bytes(B, Hq, Hkv, N, d, in_dtype)


def bwd_raw(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, cu_seqlens,
            workspace, ws_bytes, stream, in_dtype, o_dtype, grad_dtype) -> int:
    """fa_bwd with raw integer device addresses and a raw hipStream_t."""
    return load().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, int(causal),
                         scale, cu_seqlens, workspace, ws_bytes, stream, in_dtype, o_dtype,
                         grad_dtype)


def fwd_sparse_raw(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, cu_q, cu_k,
                   mask, mask_batches, mask_heads, stream, in_dtype, out_dtype) -> int:
    """fa_fwd_sparse with raw integer device addresses and a raw hipStream_t."""
    return load().fa_fwd_sparse(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, int(causal), scale,
                                cu_q, cu_k, mask, mask_batches, mask_heads, stream, in_dtype,
                                out_dtype)


def fwd_sparse_packed_raw(q, k, vt, vt_bytes, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                          cu_q, cu_k, mask, mask_batches, mask_heads, stream, in_dtype,
                          out_dtype) -> int:
    """fa_fwd_sparse_packed with raw integer device addresses."""
    return load().fa_fwd_sparse_packed(q, k, vt, vt_bytes, o, lse, B, Hq, Hkv, Nq, Nk, d,
                                       int(causal), scale, cu_q, cu_k, mask, mask_batches,
                                       mask_heads, stream, in_dtype, out_dtype)
