"""ctypes declarations of the C ABI in include/klein_attn.h.

Loading fails loudly when the HIP library has not been built: there is no
fallback path of any kind.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libklein_attn.so")
# the race check copy: the attention kernels with a full wait and a workgroup
# barrier at every stage boundary (tests compare it with the library)
SYNC_LIB_PATH = os.path.join(PKG, "libklein_attn_sync.so")

KLEIN_DTYPE_BF16 = 0
KLEIN_DTYPE_FP8_E4M3 = 1

KLEIN_OK = 0
KLEIN_ERR_INVALID_ARG = 1
KLEIN_ERR_UNSUPPORTED = 2
KLEIN_ERR_NO_DEVICE = 3
KLEIN_ERR_LAUNCH = 4
KLEIN_NOALLOC_SCRATCH_BYTES = 320 * 1024 * 1024
KLEIN_DEFAULT_BUFFER_LIMIT = 2 << 30
KLEIN_SPARSE_QBLOCK = 256
KLEIN_SPARSE_KBLOCK = 64

_lib = None

_vp, _i32p, _int, _f32 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float

SIGNATURES = {
    "klein_rope4d_attn_fwd": (_int, [_vp, _vp, _vp, _i32p, _vp, _int, _int, _int, _int, _int, _vp]),
    "klein_rope4d_attn_fwd_fp8": (_int, [_vp, _vp, _vp, _i32p, _vp, _int, _int, _int, _int,
                                         _f32, _f32, _f32, _vp]),
    "klein_rope4d_attn_fwd_blocksparse": (_int, [_vp, _vp, _vp, _i32p, _vp, _int, _int, _int,
                                                 _int, _int, _f32, _f32, _f32, _vp, _vp]),
    "klein_rope4d_attn_fwd_blocksparse_ws": (_int, [_vp, _vp, _vp, _i32p, _vp, _int, _int,
                                                    _int, _int, _int, _f32, _f32, _f32, _vp, _vp,
                                                    ctypes.c_size_t, _vp]),
    "klein_rope4d_attn_fwd_ws": (_int, [_vp, _vp, _vp, _i32p, _vp, _int, _int, _int, _int, _int,
                                        _f32, _f32, _f32, _vp, ctypes.c_size_t, _vp]),
    "klein_rope4d_attn_fwd_noalloc": (_int, [_vp, _vp, _vp, _i32p, _vp, _int, _int, _int, _int,
                                             _int, _f32, _f32, _f32, _vp]),
    "klein_set_buffer_limit": (_int, [ctypes.c_size_t]),
    "klein_attn_workspace_size": (_int, [_int, _int, _int, _int, _int,
                                         ctypes.POINTER(ctypes.c_size_t)]),
    "klein_splitkv_plan": (_int, [_int, _int, _int, _int, _int, ctypes.POINTER(ctypes.c_int),
                                  ctypes.POINTER(ctypes.c_size_t)]),
    "klein_rope4d_attn_fwd_lse": (_int, [_vp, _vp, _vp, _i32p, _vp, _vp, _int, _int, _int, _int,
                                         _vp]),
    "klein_rope4d_attn_fwd_lse_ws": (_int, [_vp, _vp, _vp, _i32p, _vp, _vp, _int, _int, _int,
                                            _int, _vp, ctypes.c_size_t, _vp]),
    "klein_rope4d_attn_bwd": (_int, [_vp, _vp, _vp, _i32p, _vp, _vp, _vp, _vp, _vp, _vp, _int,
                                     _int, _int, _int, _vp, ctypes.c_size_t, _vp]),
    "klein_attn_bwd_workspace_size": (_int, [_int, _int, _int, _int,
                                             ctypes.POINTER(ctypes.c_size_t)]),
    "klein_qkv_rope4d_proj": (_int, [_vp, _vp, _vp, _i32p, _vp, _vp, _vp, _int, _int, _int,
                                     _int, _int, _vp]),
    "klein_qkv_rope4d_proj_fp8": (_int, [_vp, _vp, _vp, _i32p, _vp, _vp, _vp, _int, _int, _int,
                                         _int, _int, _f32, _f32, _vp]),
    "klein_attn_fwd_prerotated": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp]),
    "klein_rope4d_apply": (_int, [_vp, _i32p, _vp, _int, _int, _int, _int, _vp]),
    "klein_status_string": (ctypes.c_char_p, [_int]),
    "klein_version": (_int, []),
}


def load(path):
    """A build of the library at `path` (ctypes.CDLL) with the ABI's signatures."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m joint_attention_rope_amd.build)")
    l = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(l, name)
        fn.restype = res
        fn.argtypes = args
    return l


def lib():
    """The loaded library (ctypes.CDLL), loading it on first use."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib
