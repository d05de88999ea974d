"""RoPE-4D joint self-attention for MI355X (gfx950): Python binding.

The functions here carry the names of the C ABI in include/klein_attn.h and
only marshal arguments: torch tensors (already on the GPU) become device
pointers and sizes, torch's current stream becomes the HIP stream, and a
non-zero status becomes a KleinError.  Every step of the computation runs in
the HIP kernels of libklein_attn.so; if that library is missing the calls
raise instead of computing anything another way.
"""

import torch

from . import _capi
from ._capi import (KLEIN_DTYPE_BF16, KLEIN_DTYPE_FP8_E4M3, KLEIN_ERR_INVALID_ARG,
                    KLEIN_ERR_LAUNCH, KLEIN_ERR_NO_DEVICE, KLEIN_ERR_UNSUPPORTED, KLEIN_OK,
                    KLEIN_DEFAULT_BUFFER_LIMIT, KLEIN_NOALLOC_SCRATCH_BYTES, KLEIN_SPARSE_KBLOCK,
                    KLEIN_SPARSE_QBLOCK)

__all__ = [
    "KleinError", "klein_rope4d_attn_fwd", "klein_rope4d_attn_fwd_fp8",
    "klein_rope4d_attn_fwd_blocksparse", "klein_rope4d_apply", "klein_status_string",
    "klein_version", "library_path", "KLEIN_DTYPE_BF16", "KLEIN_DTYPE_FP8_E4M3",
    "KLEIN_SPARSE_QBLOCK", "KLEIN_SPARSE_KBLOCK", "blocksparse_mask_shape",
    "klein_qkv_rope4d_proj", "klein_attn_fwd_prerotated", "klein_rope4d_attn_fwd_ws",
    "klein_attn_workspace_size", "klein_splitkv_plan", "klein_rope4d_attn_fwd_lse",
    "klein_rope4d_attn_bwd", "klein_attn_bwd_workspace_size", "klein_rope4d_attn_fwd_noalloc",
    "KLEIN_NOALLOC_SCRATCH_BYTES", "klein_set_buffer_limit", "KLEIN_DEFAULT_BUFFER_LIMIT",
]


class KleinError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({klein_status_string(status)})")


def library_path() -> str:
    return _capi.LIB_PATH


def klein_status_string(status: int) -> str:
    return _capi.lib().klein_status_string(int(status)).decode()


def klein_version() -> int:
    return _capi.lib().klein_version()


def _stream(stream, dev):
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(st, where):
    if st != KLEIN_OK:
        raise KleinError(st, where)


def _bshd(t, name):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, S, H, D], got shape {tuple(t.shape)}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return tuple(t.shape)


def _pos(pos, S):
    if pos.dtype != torch.int32 or tuple(pos.shape) != (S, 4) or not pos.is_cuda \
            or not pos.is_contiguous():
        raise ValueError(f"pos_thwl must be a contiguous int32 GPU tensor [S, 4] = [{S}, 4]")


_FP8_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def klein_rope4d_attn_fwd(q, k, v, pos_thwl, out, dtype=None, stream=None):
    """out <- RoPE-4D joint attention of q, k, v ([B, S, H, D]) at pos_thwl [S, 4].

    dtype: KLEIN_DTYPE_BF16 (q/k/v bfloat16) or KLEIN_DTYPE_FP8_E4M3 (E4M3 codes,
    descale 1); inferred from q.dtype when None.  out: bfloat16 [B, S, H, D].
    """
    B, S, H, D = _bshd(q, "q")
    for t, n in ((k, "k"), (v, "v"), (out, "out")):
        if _bshd(t, n) != (B, S, H, D):
            raise ValueError(f"{n} must have q's shape {(B, S, H, D)}")
    _pos(pos_thwl, S)
    if dtype is None:
        dtype = KLEIN_DTYPE_FP8_E4M3 if q.dtype in _FP8_DTYPES else KLEIN_DTYPE_BF16
    want = torch.bfloat16 if dtype == KLEIN_DTYPE_BF16 else None
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if (want is not None and t.dtype != want) or (want is None and t.dtype not in _FP8_DTYPES):
            raise ValueError(f"{n} has dtype {t.dtype}, which does not match the dtype code {dtype}")
    if out.dtype != torch.bfloat16:
        raise ValueError("out must be bfloat16")
    st = _capi.lib().klein_rope4d_attn_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), pos_thwl.data_ptr(), out.data_ptr(),
        B, S, H, D, int(dtype), _stream(stream, q.device))
    _check(st, "klein_rope4d_attn_fwd")
    return out


def klein_rope4d_attn_fwd_fp8(q, k, v, pos_thwl, out, q_descale, k_descale, v_descale,
                              stream=None):
    """FP8 E4M3 q, k, v (uint8 or float8_e4m3fn) with per-tensor descales; bf16 out."""
    B, S, H, D = _bshd(q, "q")
    for t, n in ((k, "k"), (v, "v"), (out, "out")):
        if _bshd(t, n) != (B, S, H, D):
            raise ValueError(f"{n} must have q's shape {(B, S, H, D)}")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype not in _FP8_DTYPES:
            raise ValueError(f"{n} must hold E4M3 codes (uint8 or float8_e4m3fn)")
    if out.dtype != torch.bfloat16:
        raise ValueError("out must be bfloat16")
    _pos(pos_thwl, S)
    st = _capi.lib().klein_rope4d_attn_fwd_fp8(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), pos_thwl.data_ptr(), out.data_ptr(),
        B, S, H, D, float(q_descale), float(k_descale), float(v_descale),
        _stream(stream, q.device))
    _check(st, "klein_rope4d_attn_fwd_fp8")
    return out


def klein_set_buffer_limit(max_bytes=KLEIN_DEFAULT_BUFFER_LIMIT):
    """Limit of the buffer klein_rope4d_attn_fwd / _fp8 keep per GPU (0: those
    calls allocate nothing and run the kernels that need no memory)."""
    _check(_capi.lib().klein_set_buffer_limit(int(max_bytes)), "klein_set_buffer_limit")


def klein_attn_workspace_size(B, S, H, D, dtype=KLEIN_DTYPE_BF16):
    """Bytes of workspace klein_rope4d_attn_fwd_ws needs for this shape on the
    current device: the rotated keys, then the split partials (if any)."""
    import ctypes
    n = ctypes.c_size_t(0)
    st = _capi.lib().klein_attn_workspace_size(int(B), int(S), int(H), int(D), int(dtype),
                                               ctypes.byref(n))
    _check(st, "klein_attn_workspace_size")
    return n.value


def klein_splitkv_plan(B, S, H, D, n_cu):
    """The split-KV plan of klein_rope4d_attn_fwd_ws on a GPU with n_cu compute
    units (host only): (whole items, cut items, chunks per cut item, partial
    bytes)."""
    import ctypes
    plan = (ctypes.c_int * 3)()
    n = ctypes.c_size_t(0)
    st = _capi.lib().klein_splitkv_plan(int(B), int(S), int(H), int(D), int(n_cu), plan,
                                        ctypes.byref(n))
    _check(st, "klein_splitkv_plan")
    return plan[0], plan[1], plan[2], n.value


def _ws_call_args(q, k, v, pos_thwl, out, dtype):
    """Shape and dtype checks of the split-KV entry points: (B, S, H, D, dtype)."""
    B, S, H, D = _bshd(q, "q")
    for t, n in ((k, "k"), (v, "v"), (out, "out")):
        if _bshd(t, n) != (B, S, H, D):
            raise ValueError(f"{n} must have q's shape {(B, S, H, D)}")
    _pos(pos_thwl, S)
    if dtype is None:
        dtype = KLEIN_DTYPE_FP8_E4M3 if q.dtype in _FP8_DTYPES else KLEIN_DTYPE_BF16
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        ok = t.dtype == torch.bfloat16 if dtype == KLEIN_DTYPE_BF16 else t.dtype in _FP8_DTYPES
        if not ok:
            raise ValueError(f"{n} has dtype {t.dtype}, which does not match the dtype code {dtype}")
    if out.dtype != torch.bfloat16:
        raise ValueError("out must be bfloat16")
    return B, S, H, D, dtype


def klein_rope4d_attn_fwd_noalloc(q, k, v, pos_thwl, out, dtype=None,
                                  descales=(1.0, 1.0, 1.0), stream=None):
    """klein_rope4d_attn_fwd_ws with the library's static per-GPU scratch
    (KLEIN_NOALLOC_SCRATCH_BYTES) as its workspace: allocates nothing.
    Calls that overlap on one GPU race.  A shape whose workspace exceeds the
    scratch raises KleinError (status UNSUPPORTED)."""
    B, S, H, D, dtype = _ws_call_args(q, k, v, pos_thwl, out, dtype)
    dq, dk, dv = (float(x) for x in descales)
    st = _capi.lib().klein_rope4d_attn_fwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), pos_thwl.data_ptr(), out.data_ptr(),
        B, S, H, D, int(dtype), dq, dk, dv, _stream(stream, q.device))
    _check(st, "klein_rope4d_attn_fwd_noalloc")
    return out


def klein_rope4d_attn_fwd_ws(q, k, v, pos_thwl, out, workspace, dtype=None,
                             descales=(1.0, 1.0, 1.0), stream=None):
    """The dense attention on the split-KV schedule (whole rounds of query
    tiles, then the remaining tiles cut into key chunks over every compute unit).

    workspace: a contiguous GPU tensor (any dtype) of at least
    klein_attn_workspace_size(B, S, H, D, dtype) bytes, or None when that is 0.
    dtype: inferred from q.dtype when None; descales (q, k, v) apply to fp8 only.
    """
    B, S, H, D, dtype = _ws_call_args(q, k, v, pos_thwl, out, dtype)
    if workspace is None:
        wp, wb = 0, 0
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        wp, wb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    dq, dk, dv = (float(x) for x in descales)
    st = _capi.lib().klein_rope4d_attn_fwd_ws(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), pos_thwl.data_ptr(), out.data_ptr(),
        B, S, H, D, int(dtype), dq, dk, dv, wp, wb, _stream(stream, q.device))
    _check(st, "klein_rope4d_attn_fwd_ws")
    return out


def _same_bshd(ref, named, dtype=torch.bfloat16):
    shape = _bshd(ref, "q")
    for t, n in named:
        if _bshd(t, n) != shape:
            raise ValueError(f"{n} must have q's shape {shape}")
        if t.dtype != dtype:
            raise ValueError(f"{n} must be {dtype}")
    return shape


def _lse_tensor(lse, B, S, H):
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S) or not lse.is_cuda \
            or not lse.is_contiguous():
        raise ValueError(f"lse must be a contiguous float32 GPU tensor [B, H, S] = [{B}, {H}, {S}]")


def klein_rope4d_attn_fwd_lse(q, k, v, pos_thwl, out, lse, stream=None, workspace=None):
    """bf16 forward that also writes lse [B, H, S] (float32, natural log of the
    softmax denominator) for klein_rope4d_attn_bwd.  With a workspace (a uint8
    GPU tensor of klein_attn_workspace_size bytes) it runs on the split-KV
    schedule of klein_rope4d_attn_fwd_ws (klein_rope4d_attn_fwd_lse_ws)."""
    B, S, H, D = _same_bshd(q, ((q, "q"), (k, "k"), (v, "v"), (out, "out")))
    _pos(pos_thwl, S)
    _lse_tensor(lse, B, S, H)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), pos_thwl.data_ptr(), out.data_ptr(),
            lse.data_ptr(), B, S, H, D)
    if workspace is None:
        st = _capi.lib().klein_rope4d_attn_fwd_lse(*args, _stream(stream, q.device))
        _check(st, "klein_rope4d_attn_fwd_lse")
    else:
        if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 GPU tensor")
        st = _capi.lib().klein_rope4d_attn_fwd_lse_ws(*args, workspace.data_ptr(),
                                                      workspace.numel(), _stream(stream, q.device))
        _check(st, "klein_rope4d_attn_fwd_lse_ws")
    return out, lse


def klein_attn_bwd_workspace_size(B, S, H, D):
    """Bytes of workspace klein_rope4d_attn_bwd needs."""
    import ctypes
    n = ctypes.c_size_t(0)
    st = _capi.lib().klein_attn_bwd_workspace_size(int(B), int(S), int(H), int(D), ctypes.byref(n))
    _check(st, "klein_attn_bwd_workspace_size")
    return n.value


def klein_rope4d_attn_bwd(q, k, v, pos_thwl, out, dout, lse, dq, dk, dv, workspace, stream=None):
    """dq, dk, dv <- gradients of the RoPE-4D joint attention (bf16 [B, S, H, D])
    given the forward's out and lse and dout = dL/dout.  workspace: a contiguous
    GPU tensor of at least klein_attn_bwd_workspace_size(B, S, H, D) bytes."""
    B, S, H, D = _same_bshd(q, ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout"),
                                (dq, "dq"), (dk, "dk"), (dv, "dv")))
    _pos(pos_thwl, S)
    _lse_tensor(lse, B, S, H)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    st = _capi.lib().klein_rope4d_attn_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), pos_thwl.data_ptr(), out.data_ptr(),
        dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, S, H, D,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(stream, q.device))
    _check(st, "klein_rope4d_attn_bwd")
    return dq, dk, dv


def blocksparse_mask_shape(B, S, H):
    """Shape of the block mask of klein_rope4d_attn_fwd_blocksparse."""
    return (B, H, -(-S // KLEIN_SPARSE_QBLOCK), -(-S // KLEIN_SPARSE_KBLOCK))


def klein_rope4d_attn_fwd_blocksparse(q, k, v, pos_thwl, out, block_mask, dtype=None,
                                      descales=(1.0, 1.0, 1.0), stream=None, workspace=None):
    """Block-sparse RoPE-4D joint attention: queries of query block I attend to
    the keys of the blocks J with block_mask[b, h, I, J] != 0 only.

    block_mask: uint8 (or bool) GPU tensor of blocksparse_mask_shape(B, S, H).
    dtype: KLEIN_DTYPE_BF16 or KLEIN_DTYPE_FP8_E4M3 (inferred from q.dtype when
    None); descales (q, k, v) apply to fp8 only.  out: bfloat16 [B, S, H, D].
    workspace: None, or a uint8 GPU tensor (klein_attn_workspace_size bytes is
    enough) into which the keys are rotated once (klein_rope4d_attn_fwd_blocksparse_ws;
    the same result).
    """
    B, S, H, D = _bshd(q, "q")
    for t, n in ((k, "k"), (v, "v"), (out, "out")):
        if _bshd(t, n) != (B, S, H, D):
            raise ValueError(f"{n} must have q's shape {(B, S, H, D)}")
    _pos(pos_thwl, S)
    if dtype is None:
        dtype = KLEIN_DTYPE_FP8_E4M3 if q.dtype in _FP8_DTYPES else KLEIN_DTYPE_BF16
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        ok = t.dtype == torch.bfloat16 if dtype == KLEIN_DTYPE_BF16 else t.dtype in _FP8_DTYPES
        if not ok:
            raise ValueError(f"{n} has dtype {t.dtype}, which does not match the dtype code {dtype}")
    if out.dtype != torch.bfloat16:
        raise ValueError("out must be bfloat16")
    if block_mask.dtype not in (torch.uint8, torch.bool) or not block_mask.is_cuda \
            or not block_mask.is_contiguous() \
            or tuple(block_mask.shape) != blocksparse_mask_shape(B, S, H):
        raise ValueError("block_mask must be a contiguous uint8/bool GPU tensor of shape "
                         f"{blocksparse_mask_shape(B, S, H)}")
    dq, dk, dv = (float(x) for x in descales)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), pos_thwl.data_ptr(), out.data_ptr(),
            B, S, H, D, int(dtype), dq, dk, dv, block_mask.data_ptr())
    if workspace is None:
        st = _capi.lib().klein_rope4d_attn_fwd_blocksparse(*args, _stream(stream, q.device))
        _check(st, "klein_rope4d_attn_fwd_blocksparse")
    else:
        if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 GPU tensor")
        st = _capi.lib().klein_rope4d_attn_fwd_blocksparse_ws(
            *args, workspace.data_ptr(), workspace.numel(), _stream(stream, q.device))
        _check(st, "klein_rope4d_attn_fwd_blocksparse_ws")
    return out


def klein_qkv_rope4d_proj(x, w, bias, pos_thwl, q_out, k_out, v_out, stream=None,
                          descales=None):
    """q_out, k_out (fp16, rotated), v_out (bf16) [B, S, H, D] <- x W^T + bias.

    x: bf16 [B, S, C]; w: bf16 [3 H D, C]; bias: bf16 [3 H D] or None.  With
    descales = (x_descale, w_descale), x and w are E4M3 codes (uint8 tensors)
    and the FP8 entry point computes (x_code w_code^T) x_descale w_descale.
    """
    fp8 = descales is not None
    xt = torch.uint8 if fp8 else torch.bfloat16
    if x.dim() != 3 or x.dtype != xt or not x.is_cuda or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous {xt} GPU tensor [B, S, C]")
    B, S, C = x.shape
    Bq, Sq, H, D = _bshd(q_out, "q_out")
    if (Bq, Sq) != (B, S) or _bshd(k_out, "k_out") != (B, S, H, D) \
            or _bshd(v_out, "v_out") != (B, S, H, D):
        raise ValueError("q_out, k_out, v_out must be [B, S, H, D] for x's B, S")
    if q_out.dtype != torch.float16 or k_out.dtype != torch.float16 or v_out.dtype != torch.bfloat16:
        raise ValueError("q_out and k_out must be float16, v_out bfloat16")
    if w.dtype != xt or tuple(w.shape) != (3 * H * D, C) or not w.is_cuda \
            or not w.is_contiguous():
        raise ValueError(f"w must be a contiguous {xt} GPU tensor [{3 * H * D}, {C}]")
    if bias is not None and (bias.dtype != torch.bfloat16 or tuple(bias.shape) != (3 * H * D,)
                             or not bias.is_cuda or not bias.is_contiguous()):
        raise ValueError(f"bias must be None or a bfloat16 GPU tensor [{3 * H * D}]")
    _pos(pos_thwl, S)
    ptrs = (x.data_ptr(), w.data_ptr(), 0 if bias is None else bias.data_ptr(),
            pos_thwl.data_ptr(), q_out.data_ptr(), k_out.data_ptr(), v_out.data_ptr(),
            B, S, C, H, D)
    if fp8:
        st = _capi.lib().klein_qkv_rope4d_proj_fp8(*ptrs, float(descales[0]), float(descales[1]),
                                                   _stream(stream, x.device))
        _check(st, "klein_qkv_rope4d_proj_fp8")
    else:
        st = _capi.lib().klein_qkv_rope4d_proj(*ptrs, _stream(stream, x.device))
        _check(st, "klein_qkv_rope4d_proj")
    return q_out, k_out, v_out


def klein_attn_fwd_prerotated(q, k, v, out, stream=None):
    """out <- joint attention of already rotated fp16 q, k and bf16 v [B, S, H, D]."""
    B, S, H, D = _bshd(q, "q")
    for t, n in ((k, "k"), (v, "v"), (out, "out")):
        if _bshd(t, n) != (B, S, H, D):
            raise ValueError(f"{n} must have q's shape {(B, S, H, D)}")
    if q.dtype != torch.float16 or k.dtype != torch.float16:
        raise ValueError("q and k must be float16 (rotated)")
    if v.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise ValueError("v and out must be bfloat16")
    st = _capi.lib().klein_attn_fwd_prerotated(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                               out.data_ptr(), B, S, H, D,
                                               _stream(stream, q.device))
    _check(st, "klein_attn_fwd_prerotated")
    return out


def klein_rope4d_apply(x, pos_thwl, y, stream=None):
    """y <- RoPE-4D(x) for bfloat16 x, y [B, S, H, D] (the kernels' own routine)."""
    B, S, H, D = _bshd(x, "x")
    if _bshd(y, "y") != (B, S, H, D) or x.dtype != torch.bfloat16 or y.dtype != torch.bfloat16:
        raise ValueError("x and y must be bfloat16 tensors of one shape")
    _pos(pos_thwl, S)
    st = _capi.lib().klein_rope4d_apply(x.data_ptr(), pos_thwl.data_ptr(), y.data_ptr(),
                                        B, S, H, D, _stream(stream, x.device))
    _check(st, "klein_rope4d_apply")
    return y
