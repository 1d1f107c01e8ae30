"""ctypes binding of libpostmix.so: argument marshalling only.

Every step of the computation runs in the gfx950 kernels behind the C ABI
(include/postmix.h).  PyTorch supplies device memory and the current stream.
There is no CPU fallback: if the library is not built, or the device is not
gfx950, the calls raise.

Entry points keep the C names:
    postmix_fwd(O, W, rope_cos, rope_sin, positions, nope, pe, out=None)
    postmix_bwd_dx(dY, W, rope_cos, rope_sin, positions, nope, pe, out=None)
    postmix_bwd_dw(dY, O, rope_cos, rope_sin, positions, nope, pe, out=None, workspace=None)
    postmix_bwd_dw_workspace_bytes(sq, nh, nope, pe)
    postmix_bwd(dY, O, W, rope_cos, rope_sin, positions, nope, pe, ...)  -> (dO, dW)
    postmix_rope_table(theta, pe, table_rows, device=None)
    postmix_kv_index_remap(idx, sq, seqlen_kv, pad_value=-1, out=None)
    postmix_rope_apply(X, rope_cos, rope_sin, positions, nope, pe, direction, out=None)
    postmix_set_general_kernels(enable)
The unfused comparison route (unfused_fwd, unfused_bwd) is composed of these
entry points only.
Tensors: O/Y/dY/dO bfloat16 [sq, nh, nope+pe]; W bfloat16 [nh, nh] (W[g,h], g =
output head); rope_cos/rope_sin float32 [rows, pe/2]; positions int32 [sq];
dW float32 [nh, nh].  Dtype mismatches raise ValueError naming the tensor (the
convention of PaddleFleet PR #1776, which rejects non-bf16 inputs by name).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpostmix.so")

PM_OK = 0
PM_ERR_NULL = -1
PM_ERR_SHAPE = -2
PM_ERR_ALIGN = -3
PM_ERR_OVERLAP = -4
PM_ERR_WORKSPACE = -5
PM_ERR_DEVICE = -6
PM_ERR_HIP = -7

_lib = None


class PostmixError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{message} (status {code})")
        self.code = code


def lib():
    """The loaded C library with argument types set (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m rope_head_mixing_amd.build` "
            "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ, F64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_double
    L.postmix_fwd.argtypes = [P, P, P, P, I64, P, I64, I32, I32, I32, P, P]
    L.postmix_fwd.restype = ctypes.c_int
    L.postmix_bwd_dx.argtypes = [P, P, P, P, I64, P, I64, I32, I32, I32, P, P]
    L.postmix_bwd_dx.restype = ctypes.c_int
    L.postmix_bwd_dw_workspace_bytes.argtypes = [I64, I32, I32, I32]
    L.postmix_bwd_dw_workspace_bytes.restype = SZ
    L.postmix_bwd_dw.argtypes = [P, P, P, P, I64, P, I64, I32, I32, I32, P, P, SZ, P]
    L.postmix_bwd_dw.restype = ctypes.c_int
    L.postmix_bwd.argtypes = [P, P, P, P, P, I64, P, I64, I32, I32, I32, P, P, P, SZ, P]
    L.postmix_bwd.restype = ctypes.c_int
    L.postmix_rope_apply.argtypes = [P, P, P, I64, P, I64, I32, I32, I32, I32, P, P]
    L.postmix_rope_apply.restype = ctypes.c_int
    L.postmix_kv_index_remap.argtypes = [P, I64, I64, I64, I64, I32, P, P]
    L.postmix_kv_index_remap.restype = ctypes.c_int
    L.postmix_rope_table.argtypes = [F64, I32, I64, P, P, P]
    L.postmix_rope_table.restype = ctypes.c_int
    L.postmix_status_string.argtypes = [ctypes.c_int]
    L.postmix_status_string.restype = ctypes.c_char_p
    L.postmix_last_error.argtypes = []
    L.postmix_last_error.restype = ctypes.c_char_p
    L.postmix_set_general_kernels.argtypes = [ctypes.c_int]
    L.postmix_set_general_kernels.restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != PM_OK:
        msg = lib().postmix_last_error().decode(errors="replace")
        raise PostmixError(rc, msg or lib().postmix_status_string(rc).decode())


def _torch():
    import torch
    return torch


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, name, dtype, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    return t


def _rope_ptrs(rope_cos, rope_sin, positions, pe, sq):
    torch = _torch()
    if pe == 0:
        return None, None, 0, None
    _need(rope_cos, "rope_cos", torch.float32, 2)
    _need(rope_sin, "rope_sin", torch.float32, 2)
    _need(positions, "positions", torch.int32, 1)
    if rope_cos.shape != rope_sin.shape or rope_cos.shape[1] != pe // 2:
        raise ValueError(f"rope_cos/rope_sin must both be [rows, {pe // 2}]")
    if positions.shape[0] != sq:
        raise ValueError(f"positions must have {sq} entries")
    return rope_cos.data_ptr(), rope_sin.data_ptr(), rope_cos.shape[0], positions.data_ptr()


def _act_shape(X, name, nope, pe):
    sq, nh, d = X.shape
    if d != nope + pe:
        raise ValueError(f"{name} last dim {d} != nope + pe = {nope + pe}")
    return sq, nh, d


def postmix_fwd(O, W, rope_cos, rope_sin, positions, nope: int, pe: int, out=None):
    """Y = inv_rope(W . O) per token (== W . inv_rope(O)), bf16 out."""
    torch = _torch()
    _need(O, "O", torch.bfloat16, 3)
    sq, nh, d = _act_shape(O, "O", nope, pe)
    _need(W, "W", torch.bfloat16, 2)
    c, s, rows, p = _rope_ptrs(rope_cos, rope_sin, positions, pe, sq)
    Y = torch.empty_like(O) if out is None else _need(out, "out", torch.bfloat16, 3)
    _check(lib().postmix_fwd(O.data_ptr(), W.data_ptr(), c, s, rows, p, sq, nh, nope, pe,
                             Y.data_ptr(), _stream_handle(O.device)))
    return Y


def postmix_bwd_dx(dY, W, rope_cos, rope_sin, positions, nope: int, pe: int, out=None):
    """dO = rope(W^T . dY) per token, bf16 out."""
    torch = _torch()
    _need(dY, "dY", torch.bfloat16, 3)
    sq, nh, d = _act_shape(dY, "dY", nope, pe)
    _need(W, "W", torch.bfloat16, 2)
    c, s, rows, p = _rope_ptrs(rope_cos, rope_sin, positions, pe, sq)
    dO = torch.empty_like(dY) if out is None else _need(out, "out", torch.bfloat16, 3)
    _check(lib().postmix_bwd_dx(dY.data_ptr(), W.data_ptr(), c, s, rows, p, sq, nh, nope, pe,
                                dO.data_ptr(), _stream_handle(dY.device)))
    return dO


def postmix_bwd_dw_workspace_bytes(sq: int, nh: int, nope: int, pe: int) -> int:
    return int(lib().postmix_bwd_dw_workspace_bytes(sq, nh, nope, pe))


def postmix_bwd_dw(dY, O, rope_cos, rope_sin, positions, nope: int, pe: int, out=None,
                   workspace=None):
    """dW[g,h] = sum_{s,c} dY[s,g,c] * inv_rope(O)[s,h,c], fp32, deterministic."""
    torch = _torch()
    _need(dY, "dY", torch.bfloat16, 3)
    _need(O, "O", torch.bfloat16, 3)
    sq, nh, d = _act_shape(dY, "dY", nope, pe)
    if tuple(O.shape) != tuple(dY.shape):
        raise ValueError("O and dY must have the same shape")
    c, s, rows, p = _rope_ptrs(rope_cos, rope_sin, positions, pe, sq)
    dW = (torch.empty((nh, nh), dtype=torch.float32, device=dY.device) if out is None
          else _need(out, "out", torch.float32, 2))
    need = postmix_bwd_dw_workspace_bytes(sq, nh, nope, pe)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dY.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().postmix_bwd_dw(dY.data_ptr(), O.data_ptr(), c, s, rows, p, sq, nh, nope, pe,
                                dW.data_ptr(), workspace.data_ptr(), ws_bytes,
                                _stream_handle(dY.device)))
    return dW


def postmix_bwd(dY, O, W, rope_cos, rope_sin, positions, nope: int, pe: int, out_dO=None,
                out_dW=None, workspace=None):
    """Both gradients in one call: (dO, dW) as postmix_bwd_dx and postmix_bwd_dw."""
    torch = _torch()
    _need(dY, "dY", torch.bfloat16, 3)
    _need(O, "O", torch.bfloat16, 3)
    _need(W, "W", torch.bfloat16, 2)
    sq, nh, d = _act_shape(dY, "dY", nope, pe)
    if tuple(O.shape) != tuple(dY.shape):
        raise ValueError("O and dY must have the same shape")
    c, s, rows, p = _rope_ptrs(rope_cos, rope_sin, positions, pe, sq)
    dO = torch.empty_like(dY) if out_dO is None else _need(out_dO, "out_dO", torch.bfloat16, 3)
    dW = (torch.empty((nh, nh), dtype=torch.float32, device=dY.device) if out_dW is None
          else _need(out_dW, "out_dW", torch.float32, 2))
    need = postmix_bwd_dw_workspace_bytes(sq, nh, nope, pe)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dY.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().postmix_bwd(dY.data_ptr(), O.data_ptr(), W.data_ptr(), c, s, rows, p, sq, nh,
                             nope, pe, dO.data_ptr(), dW.data_ptr(), workspace.data_ptr(),
                             ws_bytes, _stream_handle(dY.device)))
    return dO, dW


def postmix_rope_apply(X, rope_cos, rope_sin, positions, nope: int, pe: int, direction: int,
                       out=None):
    """Out = inv_rope(X) (direction -1) or rope(X) (+1), materialised in bf16."""
    torch = _torch()
    _need(X, "X", torch.bfloat16, 3)
    sq, nh, d = _act_shape(X, "X", nope, pe)
    c, s, rows, p = _rope_ptrs(rope_cos, rope_sin, positions, pe, sq)
    Out = torch.empty_like(X) if out is None else _need(out, "out", torch.bfloat16, 3)
    _check(lib().postmix_rope_apply(X.data_ptr(), c, s, rows, p, sq, nh, nope, pe, int(direction),
                                    Out.data_ptr(), _stream_handle(X.device)))
    return Out


def unfused_fwd(O, W, rope_cos, rope_sin, positions, nope: int, pe: int):
    """The unfused route: X = inv_rope(O) materialised (bf16), then Y = W . X."""
    X = postmix_rope_apply(O, rope_cos, rope_sin, positions, nope, pe, -1)
    return postmix_fwd(X, W, None, None, None, nope + pe, 0)


def unfused_bwd(dY, O, W, rope_cos, rope_sin, positions, nope: int, pe: int, workspace=None):
    """The unfused backward route: rebuild X = inv_rope(O), the plain mix's
    gradients dX = W^T dY and dW = sum dY X^T, then dO = rope(dX)."""
    X = postmix_rope_apply(O, rope_cos, rope_sin, positions, nope, pe, -1)
    dX = postmix_bwd_dx(dY, W, None, None, None, nope + pe, 0)
    dW = postmix_bwd_dw(dY, X, None, None, None, nope + pe, 0, workspace=workspace)
    dO = postmix_rope_apply(dX, rope_cos, rope_sin, positions, nope, pe, +1)
    return dO, dW


def postmix_kv_index_remap(idx, sq: int, seqlen_kv: int, pad_value: int = -1, out=None):
    """Per-batch-local KV column indices -> flat-global: idx [b*sq, topk] int32."""
    torch = _torch()
    _need(idx, "idx", torch.int32, 2)
    rows, topk = idx.shape
    out = torch.empty_like(idx) if out is None else _need(out, "out", torch.int32, 2)
    _check(lib().postmix_kv_index_remap(idx.data_ptr(), rows, sq, topk, seqlen_kv, pad_value,
                                        out.data_ptr(), _stream_handle(idx.device)))
    return out


def postmix_set_general_kernels(enable: bool) -> bool:
    """Route fwd/dx through the general kernel for every shape; returns the previous setting."""
    return bool(lib().postmix_set_general_kernels(1 if enable else 0))


def postmix_rope_table(theta: float, pe: int, table_rows: int, device=None):
    """(cos, sin) fp32 [table_rows, pe/2] built on the GPU from an fp64 angle."""
    torch = _torch()
    device = torch.device("cuda") if device is None else torch.device(device)
    cos = torch.empty((table_rows, pe // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    _check(lib().postmix_rope_table(float(theta), pe, table_rows, cos.data_ptr(), sin.data_ptr(),
                                    _stream_handle(device)))
    return cos, sin
