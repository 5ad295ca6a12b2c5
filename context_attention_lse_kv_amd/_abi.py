"""ctypes view of include/ra.h and the loader of libra.so.

There is no fallback: if the HIP library is not built or cannot be loaded,
``lib()`` raises.  Build it with ``python -m context_attention_lse_kv_amd.build``.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# RA_LIB selects another build of the same library (e.g. to compare kernel variants)
LIB_PATH = os.environ.get("RA_LIB") or os.path.join(_PKG, "libra.so")

RA_OK, RA_E_ARG, RA_E_SHAPE, RA_E_DTYPE, RA_E_ALIGN, RA_E_UNSUPPORTED, RA_E_WORKSPACE, RA_E_HIP = range(8)
RA_BF16, RA_F32 = 1, 2
STATUS_NAMES = ["RA_OK", "RA_E_ARG", "RA_E_SHAPE", "RA_E_DTYPE", "RA_E_ALIGN", "RA_E_UNSUPPORTED",
                "RA_E_WORKSPACE", "RA_E_HIP"]

# every symbol include/ra.h declares
EXPORTS = [
    "ra_fwd_chunk", "ra_merge_lse", "ra_bwd_delta", "ra_bwd_chunk", "ra_bwd_chunk_dkdv", "ra_bwd_chunk_dq",
    "ra_ring_fwd", "ra_ring_bwd",
    "ra_fwd_chunk_masked", "ra_bwd_chunk_masked", "ra_bwd_chunk_dkdv_masked", "ra_bwd_chunk_dq_masked",
    "ra_ring_fwd_masked", "ra_ring_bwd_masked", "ra_ring_fwd_noalloc",
    "ra_bwd_ds_bytes", "ra_bwd_chunk_dkdv_ds", "ra_bwd_chunk_dq_ds",
    "ra_ring_fwd_workspace_bytes", "ra_ring_bwd_workspace_bytes", "ra_ring_bwd_workspace_min_bytes",
    "ra_ring_bwd_plan", "ra_seq_head_permute",
    "ra_split_sizes", "ra_ring_order", "ra_status_string", "ra_last_error", "ra_version",
]


class RaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("sB", ctypes.c_int64), ("sS", ctypes.c_int64), ("sH", ctypes.c_int64)]


class RaLse(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("S", ctypes.c_int32),
                ("sB", ctypes.c_int64), ("sH", ctypes.c_int64)]


class RaKMask(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("sB", ctypes.c_int64)]


class RaChunks(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("start", ctypes.POINTER(ctypes.c_int32)),
                ("len", ctypes.POINTER(ctypes.c_int32)), ("order", ctypes.POINTER(ctypes.c_int32))]


T = ctypes.POINTER(RaTensor)
L = ctypes.POINTER(RaLse)
C = ctypes.POINTER(RaChunks)
K = ctypes.POINTER(RaKMask)
vp, f32, i32, sz = ctypes.c_void_p, ctypes.c_float, ctypes.c_int32, ctypes.c_size_t
I32P = ctypes.POINTER(ctypes.c_int32)

_SIGS = {
    "ra_fwd_chunk": (i32, [T, T, T, f32, T, L, i32, vp]),
    "ra_merge_lse": (i32, [T, L, T, L, vp]),
    "ra_bwd_delta": (i32, [T, T, L, vp]),
    "ra_bwd_chunk": (i32, [T, T, T, T, L, L, f32, T, T, T, i32, vp]),
    "ra_bwd_chunk_dkdv": (i32, [T, T, T, T, L, L, f32, T, T, i32, vp]),
    "ra_bwd_chunk_dq": (i32, [T, T, T, T, L, L, f32, T, vp]),
    "ra_ring_fwd": (i32, [T, T, T, C, f32, T, L, vp, sz, vp]),
    "ra_ring_bwd": (i32, [T, T, T, T, T, L, C, f32, T, T, T, vp, sz, vp]),
    "ra_fwd_chunk_masked": (i32, [T, T, T, K, f32, T, L, i32, vp]),
    "ra_bwd_chunk_masked": (i32, [T, T, T, T, L, L, K, f32, T, T, T, i32, vp]),
    "ra_bwd_chunk_dkdv_masked": (i32, [T, T, T, T, L, L, K, f32, T, T, i32, vp]),
    "ra_bwd_chunk_dq_masked": (i32, [T, T, T, T, L, L, K, f32, T, vp]),
    "ra_ring_fwd_masked": (i32, [T, T, T, K, C, f32, T, L, vp, sz, vp]),
    "ra_ring_bwd_masked": (i32, [T, T, T, T, T, L, K, C, f32, T, T, T, vp, sz, vp]),
    "ra_ring_fwd_noalloc": (i32, [T, T, T, K, C, f32, T, L, vp]),
    "ra_bwd_ds_bytes": (sz, [T, T]),
    "ra_bwd_chunk_dkdv_ds": (i32, [T, T, T, T, L, L, K, f32, T, T, i32, vp, sz, vp]),
    "ra_bwd_chunk_dq_ds": (i32, [T, T, vp, sz, f32, T, vp]),
    "ra_ring_fwd_workspace_bytes": (sz, [T, T]),
    "ra_ring_bwd_workspace_bytes": (sz, [T, T, T, T, T]),
    "ra_ring_bwd_workspace_min_bytes": (sz, [T, T, T, T, T]),
    "ra_ring_bwd_plan": (i32, [T, T, T, T, T, C, sz, I32P, I32P, ctypes.POINTER(ctypes.c_uint32)]),
    "ra_seq_head_permute": (i32, [T, i32, T, i32, i32, vp]),
    "ra_split_sizes": (i32, [i32, i32, I32P]),
    "ra_ring_order": (i32, [i32, i32, I32P]),
    "ra_status_string": (ctypes.c_char_p, [i32]),
    "ra_last_error": (ctypes.c_char_p, []),
    "ra_version": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """Load libra.so once; raise if it is missing (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is not built; run "
                               "`python -m context_attention_lse_kv_amd.build` (needs hipcc for gfx950)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


class RaError(RuntimeError):
    def __init__(self, status, fn):
        self.status = status
        detail = lib().ra_last_error().decode()
        super().__init__(f"{fn}: {STATUS_NAMES[status] if 0 <= status < 8 else status}: {detail}")


def check(status, fn):
    if status != RA_OK:
        raise RaError(status, fn)
