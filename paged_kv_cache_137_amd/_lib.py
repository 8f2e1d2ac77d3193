"""ctypes loader for libpkv.so, the C ABI declared in include/pkv.h.

Argument marshalling only.  Every step of the path runs in the library's HIP
kernels.  There is no fallback: if the library is missing or cannot load,
every call raises.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")

PKV_F32, PKV_F16, PKV_BF16 = 0, 1, 2
PKV_PARTITION_AUTO = -1  # the library picks the decode's context partition
PKV_OK, PKV_EINVAL, PKV_ENOTSUP, PKV_ELAUNCH, PKV_EDEVICE, PKV_EWORKSPACE = 0, -1, -2, -3, -4, -5
PKV_NOALLOC_SCRATCH_BYTES = 64 << 20  # the device scratch of pkv_paged_attn_decode_noalloc, per GPU

# Every function include/pkv.h declares, with its ctypes signature.
_i32, _i64, _sz, _vp, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_DECODE_ARGS = [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _f32, _vp, _i32, _i32, _vp, _sz, _vp]
SIGNATURES = {
    "pkv_abi_version": ([], ctypes.c_int),
    "pkv_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "pkv_check_device": ([], ctypes.c_int),
    "pkv_kv_cache_write": ([_vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp], ctypes.c_int),
    "pkv_decode_workspace_bytes": ([_i32, _i32, _i32, _i32, _i32], _sz),
    "pkv_decode_partition": ([_i32, _i32, _i32, _i32, _i32, _vp], ctypes.c_int),
    "pkv_decode_partition_for_lengths": ([_vp, _i32, _i32, _vp], ctypes.c_int),
    "pkv_paged_attn_decode": (_DECODE_ARGS, ctypes.c_int),
    "pkv_paged_attn_decode_partial": (_DECODE_ARGS, ctypes.c_int),
    "pkv_paged_attn_decode_reduce": (_DECODE_ARGS, ctypes.c_int),
    "pkv_decode_shared_workspace_bytes": ([_i32, _i32, _i32, _i32, _i32], _sz),
    "pkv_paged_attn_decode_shared": (_DECODE_ARGS, ctypes.c_int),
    "pkv_paged_attn_decode_noalloc": ([_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _f32, _vp, _i32, _i32, _vp],
                                      ctypes.c_int),
    "pkv_copy_blocks": ([_vp, _vp, _vp, _vp, _i64, _vp], ctypes.c_int),
    "pkv_kv_read_probe": ([_vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _vp, _vp, _sz, _vp], ctypes.c_int),
    "pkv_swap_blocks": ([_vp, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp], ctypes.c_int),
    "pkv_paged_attn_prefill_cached": (
        [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i64, _i32, _i32, _f32, _vp, _i32, _vp],
        ctypes.c_int,
    ),
    "pkv_paged_attn_prefill": (
        [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _i32, _i64, _i32, _f32, _vp, _i32, _vp],
        ctypes.c_int,
    ),
}


class CacheDesc(ctypes.Structure):
    """pkv_cache_desc."""

    _fields_ = [
        ("num_blocks", ctypes.c_int64),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class PKVError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {code})")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')"
            )
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def check(fn: str, code: int) -> None:
    if code != PKV_OK:
        raise PKVError(fn, code, lib().pkv_status_str(code).decode())
