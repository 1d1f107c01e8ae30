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
    postmix_bwd_noalloc(dY, O, W, rope_cos, rope_sin, positions, nope, pe, out_dO, out_dW)
    postmix_rope_table(theta, pe, table_rows, device=None)
    postmix_kv_index_remap(idx, sq, seqlen_kv, pad_value=-1, out=None)
    postmix_rope_apply(X, rope_cos, rope_sin, positions, nope, pe, direction, out=None)
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
    L.postmix_bwd_noalloc.argtypes = [P, P, P, P, P, I64, P, I64, I32, I32, I32, P, P, P]
    L.postmix_bwd_noalloc.restype = ctypes.c_int
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
    # test hook (csrc/postmix_testing.h), not part of the public interface
    L.pm_testing_set_general_kernels.argtypes = [ctypes.c_int]
    L.pm_testing_set_general_kernels.restype = ctypes.c_int
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


def _fmt_shape(shape):
    return "[" + ", ".join("*" if s is None else str(s) for s in shape) + "]"


class _Spec:
    """One tensor argument: its name, dtype and expected shape (None = any size)."""

    def __init__(self, t, name, dtype, shape):
        self.t, self.name, self.dtype, self.shape = t, name, dtype, shape


def _validate(*specs):
    """Check every tensor argument, in two passes: first what needs no device
    (type, dtype, shape, contiguity) for all of them, then that all live on
    one GPU device.  The C ABI sees only pointers and sizes, so a tensor that
    is smaller than the sizes say would be read or written past its end; these
    checks are what prevents that.  Returns the common device."""
    torch = _torch()
    for s in specs:
        t = s.t
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{s.name} must be a torch.Tensor")
        if t.dtype != s.dtype:
            raise ValueError(f"{s.name} must be {s.dtype}, got {t.dtype}")
        if s.shape is not None and (t.dim() != len(s.shape) or any(
                want is not None and got != want for got, want in zip(t.shape, s.shape))):
            raise ValueError(f"{s.name} must have shape {_fmt_shape(s.shape)}, got {list(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{s.name} must be contiguous")
    device = None
    for s in specs:
        if not s.t.is_cuda:
            raise ValueError(f"{s.name} must be on a GPU device, got {s.t.device}")
        if device is None:
            device = s.t.device
        elif s.t.device != device:
            raise ValueError(f"{s.name} is on {s.t.device}, but {specs[0].name} is on {device}: "
                             "all tensors must be on one device")
    return device


def _rope_specs(rope_cos, rope_sin, positions, pe, sq):
    """Specs of the table arguments (none when pe == 0: they are not read)."""
    torch = _torch()
    if pe == 0:
        return []
    rows = rope_cos.shape[0] if isinstance(rope_cos, torch.Tensor) and rope_cos.dim() == 2 else None
    return [_Spec(rope_cos, "rope_cos", torch.float32, (rows, pe // 2)),
            _Spec(rope_sin, "rope_sin", torch.float32, (rows, pe // 2)),
            _Spec(positions, "positions", torch.int32, (sq,))]


def _rope_ptrs(rope_cos, rope_sin, positions, pe):
    if pe == 0:
        return None, None, 0, None
    return rope_cos.data_ptr(), rope_sin.data_ptr(), rope_cos.shape[0], positions.data_ptr()


def _act_dims(X, name, nope, pe):
    """(sq, nh) of an activation [sq, nh, nope + pe]; raises on a wrong rank or width."""
    torch = _torch()
    if not isinstance(X, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if X.dim() != 3 or X.shape[2] != nope + pe:
        raise ValueError(f"{name} must have shape [sq, nh, {nope + pe}] (nope + pe = {nope} + {pe}), "
                         f"got {list(X.shape)}")
    return X.shape[0], X.shape[1]


class _on_device:
    """Make `device` current for a call (the library launches on the current
    device's stream and checks that device), restoring the previous one."""

    def __init__(self, device):
        self.device = device
        self.prev = None

    def __enter__(self):
        torch = _torch()
        cur = torch.cuda.current_device()
        if self.device.index is not None and self.device.index != cur:
            self.prev = cur
            torch.cuda.set_device(self.device)
        return self

    def __exit__(self, *exc):
        if self.prev is not None:
            _torch().cuda.set_device(self.prev)
        return False


def postmix_fwd(O, W, rope_cos, rope_sin, positions, nope: int, pe: int, out=None):
    """Y = inv_rope(W . O) per token (== W . inv_rope(O)), bf16 out."""
    torch = _torch()
    sq, nh = _act_dims(O, "O", nope, pe)
    d = nope + pe
    specs = [_Spec(O, "O", torch.bfloat16, (sq, nh, d)), _Spec(W, "W", torch.bfloat16, (nh, nh)),
             *_rope_specs(rope_cos, rope_sin, positions, pe, sq)]
    if out is not None:
        specs.append(_Spec(out, "out", torch.bfloat16, (sq, nh, d)))
    dev = _validate(*specs)
    c, s, rows, p = _rope_ptrs(rope_cos, rope_sin, positions, pe)
    Y = torch.empty_like(O) if out is None else out
    with _on_device(dev):
        _check(lib().postmix_fwd(O.data_ptr(), W.data_ptr(), c, s, rows, p, sq, nh, nope, pe,
                                 Y.data_ptr(), _stream_handle(dev)))
    return Y


def postmix_bwd_dx(dY, W, rope_cos, rope_sin, positions, nope: int, pe: int, out=None):
    """dO = rope(W^T . dY) per token, bf16 out."""
    torch = _torch()
    sq, nh = _act_dims(dY, "dY", nope, pe)
    d = nope + pe
    specs = [_Spec(dY, "dY", torch.bfloat16, (sq, nh, d)), _Spec(W, "W", torch.bfloat16, (nh, nh)),
             *_rope_specs(rope_cos, rope_sin, positions, pe, sq)]
    if out is not None:
        specs.append(_Spec(out, "out", torch.bfloat16, (sq, nh, d)))
    dev = _validate(*specs)
    c, s, rows, p = _rope_ptrs(rope_cos, rope_sin, positions, pe)
    dO = torch.empty_like(dY) if out is None else out
    with _on_device(dev):
        _check(lib().postmix_bwd_dx(dY.data_ptr(), W.data_ptr(), c, s, rows, p, sq, nh, nope, pe,
                                    dO.data_ptr(), _stream_handle(dev)))
    return dO


def postmix_bwd_dw_workspace_bytes(sq: int, nh: int, nope: int, pe: int) -> int:
    return int(lib().postmix_bwd_dw_workspace_bytes(sq, nh, nope, pe))


def _workspace_spec(workspace):
    """A caller's workspace (any dtype; its size in bytes is passed on and checked by the library)."""
    return [] if workspace is None else [_Spec(workspace, "workspace",
                                               getattr(workspace, "dtype", None), None)]


def postmix_bwd_dw(dY, O, rope_cos, rope_sin, positions, nope: int, pe: int, out=None,
                   workspace=None):
    """dW[g,h] = sum_{s,c} dY[s,g,c] * inv_rope(O)[s,h,c], fp32, deterministic."""
    torch = _torch()
    sq, nh = _act_dims(dY, "dY", nope, pe)
    d = nope + pe
    specs = [_Spec(dY, "dY", torch.bfloat16, (sq, nh, d)), _Spec(O, "O", torch.bfloat16, (sq, nh, d)),
             *_rope_specs(rope_cos, rope_sin, positions, pe, sq)]
    if out is not None:
        specs.append(_Spec(out, "out", torch.float32, (nh, nh)))
    specs += _workspace_spec(workspace)
    dev = _validate(*specs)
    c, s, rows, p = _rope_ptrs(rope_cos, rope_sin, positions, pe)
    dW = torch.empty((nh, nh), dtype=torch.float32, device=dev) if out is None else out
    need = postmix_bwd_dw_workspace_bytes(sq, nh, nope, pe)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    with _on_device(dev):
        _check(lib().postmix_bwd_dw(dY.data_ptr(), O.data_ptr(), c, s, rows, p, sq, nh, nope, pe,
                                    dW.data_ptr(), workspace.data_ptr(), ws_bytes,
                                    _stream_handle(dev)))
    return dW


def postmix_bwd(dY, O, W, rope_cos, rope_sin, positions, nope: int, pe: int, out_dO=None,
                out_dW=None, workspace=None):
    """Both gradients in one call: (dO, dW) as postmix_bwd_dx and postmix_bwd_dw."""
    torch = _torch()
    sq, nh = _act_dims(dY, "dY", nope, pe)
    d = nope + pe
    specs = [_Spec(dY, "dY", torch.bfloat16, (sq, nh, d)), _Spec(O, "O", torch.bfloat16, (sq, nh, d)),
             _Spec(W, "W", torch.bfloat16, (nh, nh)),
             *_rope_specs(rope_cos, rope_sin, positions, pe, sq)]
    if out_dO is not None:
        specs.append(_Spec(out_dO, "out_dO", torch.bfloat16, (sq, nh, d)))
    if out_dW is not None:
        specs.append(_Spec(out_dW, "out_dW", torch.float32, (nh, nh)))
    specs += _workspace_spec(workspace)
    dev = _validate(*specs)
    c, s, rows, p = _rope_ptrs(rope_cos, rope_sin, positions, pe)
    dO = torch.empty_like(dY) if out_dO is None else out_dO
    dW = torch.empty((nh, nh), dtype=torch.float32, device=dev) if out_dW is None else out_dW
    need = postmix_bwd_dw_workspace_bytes(sq, nh, nope, pe)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    with _on_device(dev):
        _check(lib().postmix_bwd(dY.data_ptr(), O.data_ptr(), W.data_ptr(), c, s, rows, p, sq, nh,
                                 nope, pe, dO.data_ptr(), dW.data_ptr(), workspace.data_ptr(),
                                 ws_bytes, _stream_handle(dev)))
    return dO, dW


def postmix_bwd_noalloc(dY, O, W, rope_cos, rope_sin, positions, nope: int, pe: int, out_dO=None,
                        out_dW=None):
    """postmix_bwd with the library's static scratch instead of a workspace
    (the C entry point allocates nothing; outputs not given are allocated
    here, by torch)."""
    torch = _torch()
    sq, nh = _act_dims(dY, "dY", nope, pe)
    d = nope + pe
    specs = [_Spec(dY, "dY", torch.bfloat16, (sq, nh, d)), _Spec(O, "O", torch.bfloat16, (sq, nh, d)),
             _Spec(W, "W", torch.bfloat16, (nh, nh)),
             *_rope_specs(rope_cos, rope_sin, positions, pe, sq)]
    if out_dO is not None:
        specs.append(_Spec(out_dO, "out_dO", torch.bfloat16, (sq, nh, d)))
    if out_dW is not None:
        specs.append(_Spec(out_dW, "out_dW", torch.float32, (nh, nh)))
    dev = _validate(*specs)
    c, s, rows, p = _rope_ptrs(rope_cos, rope_sin, positions, pe)
    dO = torch.empty_like(dY) if out_dO is None else out_dO
    dW = torch.empty((nh, nh), dtype=torch.float32, device=dev) if out_dW is None else out_dW
    with _on_device(dev):
        _check(lib().postmix_bwd_noalloc(dY.data_ptr(), O.data_ptr(), W.data_ptr(), c, s, rows, p, sq, nh,
                                         nope, pe, dO.data_ptr(), dW.data_ptr(), _stream_handle(dev)))
    return dO, dW


def postmix_rope_apply(X, rope_cos, rope_sin, positions, nope: int, pe: int, direction: int,
                       out=None):
    """Out = inv_rope(X) (direction -1) or rope(X) (+1), materialised in bf16."""
    torch = _torch()
    sq, nh = _act_dims(X, "X", nope, pe)
    d = nope + pe
    specs = [_Spec(X, "X", torch.bfloat16, (sq, nh, d)),
             *_rope_specs(rope_cos, rope_sin, positions, pe, sq)]
    if out is not None:
        specs.append(_Spec(out, "out", torch.bfloat16, (sq, nh, d)))
    dev = _validate(*specs)
    c, s, rows, p = _rope_ptrs(rope_cos, rope_sin, positions, pe)
    Out = torch.empty_like(X) if out is None else out
    with _on_device(dev):
        _check(lib().postmix_rope_apply(X.data_ptr(), c, s, rows, p, sq, nh, nope, pe,
                                        int(direction), Out.data_ptr(), _stream_handle(dev)))
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
    if not isinstance(idx, torch.Tensor) or idx.dim() != 2:
        raise ValueError("idx must be a 2-dimensional torch.Tensor [rows, topk]")
    rows, topk = idx.shape
    specs = [_Spec(idx, "idx", torch.int32, (rows, topk))]
    if out is not None:
        specs.append(_Spec(out, "out", torch.int32, (rows, topk)))
    dev = _validate(*specs)
    out = torch.empty_like(idx) if out is None else out
    with _on_device(dev):
        _check(lib().postmix_kv_index_remap(idx.data_ptr(), rows, sq, topk, seqlen_kv, pad_value,
                                            out.data_ptr(), _stream_handle(dev)))
    return out


def testing_set_general_kernels(enable: bool) -> bool:
    """Test hook: this thread's later calls run the general kernels for every
    shape; returns the thread's previous setting."""
    return bool(lib().pm_testing_set_general_kernels(1 if enable else 0))


def postmix_rope_table(theta: float, pe: int, table_rows: int, device=None):
    """(cos, sin) fp32 [table_rows, pe/2] built on the GPU from an fp64 angle."""
    torch = _torch()
    device = torch.device("cuda") if device is None else torch.device(device)
    if device.type != "cuda":
        raise ValueError(f"device must be a GPU device, got {device}")
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    cos = torch.empty((table_rows, pe // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    with _on_device(device):
        _check(lib().postmix_rope_table(float(theta), pe, table_rows, cos.data_ptr(), sin.data_ptr(),
                                        _stream_handle(device)))
    return cos, sin
