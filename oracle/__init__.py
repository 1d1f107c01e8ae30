"""fp64 CPU oracle for the inverse-RoPE + VHA postmix path (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  The product path (the HIP library and its binding) never
does, and this package imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C loops in fp64); this module only
builds it with gcc, loads it with ctypes and marshals numpy arrays.  See the
header of ``oracle.c`` for the passages each function follows:
PaddleFleet PR #1772 "Fuse HCA inverse RoPE into the VHA postmix, and the
sparse-attention KV index remap" (PR body item 1; description part 一).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, invariants, a textbook-GEMM special case, brute force with
explicit rotation matrices and central finite differences).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F64 = ctypes.c_double


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (fp64, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_variant(src_text: str, out_path: str) -> str:
    """Compile a modified copy of oracle.c (used by the mutation tests)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-w",
                           "-fno-fast-math", "-ffp-contract=off", "-o", out_path, src,
                           "-lm", "-lpthread"])
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def use_library(path: str | None):
    """Point every function at another build of the oracle (None: the real one).
    Returns the previously loaded library handle."""
    global _lib
    prev = _lib
    _lib = None
    if path is not None:
        _lib = _bind(ctypes.CDLL(path))
    return prev


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    sig = {
        "oracle_default_threads": ([], _I32),
        "oracle_rope_angles": ([_F64, _I32, _P, _I64, _P, _P], None),
        "oracle_fwd_bf16": ([_P, _P, _P, _F64, _I64, _I32, _I32, _I32, _P, _I32], _I32),
        "oracle_fwd_f64": ([_P, _P, _P, _F64, _I64, _I32, _I32, _I32, _P, _I32], _I32),
        "oracle_bwd_dx_bf16": ([_P, _P, _P, _F64, _I64, _I32, _I32, _I32, _P, _I32], _I32),
        "oracle_bwd_dx_f64": ([_P, _P, _P, _F64, _I64, _I32, _I32, _I32, _P, _I32], _I32),
        "oracle_bwd_dw_bf16": ([_P, _P, _P, _F64, _I64, _I32, _I32, _I32, _P, _I32], _I32),
        "oracle_bwd_dw_f64": ([_P, _P, _P, _F64, _I64, _I32, _I32, _I32, _P, _I32], _I32),
        "oracle_bwd_dw_abs_bf16": ([_P, _P, _P, _F64, _I64, _I32, _I32, _I32, _P, _I32], _I32),
        "oracle_rotate_f64": ([_P, _P, _P, _F64, _I64, _I32, _I32, _I32, _I32], _I32),
        "oracle_fwd_at_bf16": ([_P, _P, _P, _F64, _I64, _I32, _I32, _I32, _P, _I64, _P], _I32),
        "oracle_bwd_dx_at_bf16": ([_P, _P, _P, _F64, _I64, _I32, _I32, _I32, _P, _I64, _P], _I32),
        "oracle_bwd_dw_at_bf16": ([_P, _P, _P, _F64, _I64, _I32, _I32, _I32, _P, _I64, _P, _I32], _I32),
        "oracle_kv_remap": ([_P, _I64, _I64, _I64, _I64, _I32, _P], _I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


def default_threads() -> int:
    return int(_load().oracle_default_threads())


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check_rc(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def _tensor(x: np.ndarray, name: str):
    """Return (contiguous array, kind) with kind 'bf16' for uint16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, "bf16"
    if x.dtype == np.float64:
        return x, "f64"
    raise TypeError(f"{name}: oracle takes bf16 bits (uint16) or float64, got {x.dtype}")


def _positions(positions, sq: int) -> np.ndarray:
    p = np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
    if p.shape != (sq,):
        raise ValueError(f"positions must have shape ({sq},), got {p.shape}")
    return p


def rope_angles(theta: float, pe: int, positions) -> tuple[np.ndarray, np.ndarray]:
    """fp64 cos/sin of positions[s]*theta^(-2i/pe), shape [sq, pe//2]."""
    p = np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
    sq = p.shape[0]
    c = np.zeros((sq, pe // 2), np.float64)
    s = np.zeros((sq, pe // 2), np.float64)
    _load().oracle_rope_angles(float(theta), int(pe), _ptr(p), sq, _ptr(c), _ptr(s))
    return c, s


def _same_kind(a, b, na, nb):
    a, ka = _tensor(a, na)
    b, kb = _tensor(b, nb)
    if ka != kb:
        raise TypeError(f"{na} and {nb} must both be bf16 bits or both float64")
    return a, b, ka


def fwd(O, W, positions, theta, nope, pe, nthreads=None) -> np.ndarray:
    """Y = W . inv_rope(O) per token; O [sq, nh, d], W [nh, nh]; returns fp64."""
    O, W, kind = _same_kind(O, W, "O", "W")
    sq, nh, d = O.shape
    assert d == nope + pe and W.shape == (nh, nh)
    p = _positions(positions, sq)
    Y = np.empty((sq, nh, d), np.float64)
    fn = _load().oracle_fwd_bf16 if kind == "bf16" else _load().oracle_fwd_f64
    nt = default_threads() if nthreads is None else nthreads
    _check_rc(fn(_ptr(O), _ptr(W), _ptr(p), float(theta), sq, nh, nope, pe, _ptr(Y), nt), "fwd")
    return Y


def bwd_dx(dY, W, positions, theta, nope, pe, nthreads=None) -> np.ndarray:
    """dO = rope(W^T . dY) per token; returns fp64 [sq, nh, d]."""
    dY, W, kind = _same_kind(dY, W, "dY", "W")
    sq, nh, d = dY.shape
    assert d == nope + pe and W.shape == (nh, nh)
    p = _positions(positions, sq)
    dO = np.empty((sq, nh, d), np.float64)
    fn = _load().oracle_bwd_dx_bf16 if kind == "bf16" else _load().oracle_bwd_dx_f64
    nt = default_threads() if nthreads is None else nthreads
    _check_rc(fn(_ptr(dY), _ptr(W), _ptr(p), float(theta), sq, nh, nope, pe, _ptr(dO), nt), "bwd_dx")
    return dO


def bwd_dw(dY, O, positions, theta, nope, pe, nthreads=None) -> np.ndarray:
    """dW[g,h] = sum_{s,c} dY[s,g,c] * inv_rope(O)[s,h,c]; returns fp64 [nh, nh]."""
    dY, O, kind = _same_kind(dY, O, "dY", "O")
    sq, nh, d = dY.shape
    assert O.shape == dY.shape and d == nope + pe
    p = _positions(positions, sq)
    dW = np.empty((nh, nh), np.float64)
    fn = _load().oracle_bwd_dw_bf16 if kind == "bf16" else _load().oracle_bwd_dw_f64
    nt = default_threads() if nthreads is None else nthreads
    _check_rc(fn(_ptr(dY), _ptr(O), _ptr(p), float(theta), sq, nh, nope, pe, _ptr(dW), nt), "bwd_dw")
    return dW


def bwd_dw_abs(dY, O, positions, theta, nope, pe, nthreads=None) -> np.ndarray:
    """A[g,h] = sum_{s,c} |dY[s,g,c] * inv_rope(O)[s,h,c]| (the magnitude of the
    terms of each dW entry, i.e. its conditioning); bf16 inputs; fp64 [nh, nh]."""
    dY, O, kind = _same_kind(dY, O, "dY", "O")
    assert kind == "bf16"
    sq, nh, d = dY.shape
    assert O.shape == dY.shape and d == nope + pe
    p = _positions(positions, sq)
    A = np.empty((nh, nh), np.float64)
    nt = default_threads() if nthreads is None else nthreads
    _check_rc(_load().oracle_bwd_dw_abs_bf16(_ptr(dY), _ptr(O), _ptr(p), float(theta), sq, nh, nope, pe,
                                             _ptr(A), nt), "bwd_dw_abs")
    return A


def rotate(X, positions, theta, nope, pe, direction) -> np.ndarray:
    """direction=-1: inv_rope(X); direction=+1: rope(X). X fp64 [sq, nh, d]."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    sq, nh, d = X.shape
    p = _positions(positions, sq)
    out = np.empty_like(X)
    _check_rc(_load().oracle_rotate_f64(_ptr(X), _ptr(out), _ptr(p), float(theta), sq, nh,
                                        nope, pe, int(direction)), "rotate")
    return out


def inv_rope(X, positions, theta, nope, pe):
    return rotate(X, positions, theta, nope, pe, -1)


def rope(X, positions, theta, nope, pe):
    return rotate(X, positions, theta, nope, pe, +1)


def fwd_at(O, W, positions, theta, nope, pe, flat_idx) -> np.ndarray:
    """Y at flat indices (s*nh + g)*d + c, each computed on its own; bf16 inputs."""
    O, W, kind = _same_kind(O, W, "O", "W")
    assert kind == "bf16"
    sq, nh, d = O.shape
    p = _positions(positions, sq)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    out = np.empty(idx.shape[0], np.float64)
    _check_rc(_load().oracle_fwd_at_bf16(_ptr(O), _ptr(W), _ptr(p), float(theta), sq, nh, nope,
                                         pe, _ptr(idx), idx.shape[0], _ptr(out)), "fwd_at")
    return out


def bwd_dx_at(dY, W, positions, theta, nope, pe, flat_idx) -> np.ndarray:
    """dO at flat indices (s*nh + h)*d + c, each computed on its own; bf16 inputs."""
    dY, W, kind = _same_kind(dY, W, "dY", "W")
    assert kind == "bf16"
    sq, nh, d = dY.shape
    p = _positions(positions, sq)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    out = np.empty(idx.shape[0], np.float64)
    _check_rc(_load().oracle_bwd_dx_at_bf16(_ptr(dY), _ptr(W), _ptr(p), float(theta), sq, nh,
                                            nope, pe, _ptr(idx), idx.shape[0], _ptr(out)),
              "bwd_dx_at")
    return out


def bwd_dw_at(dY, O, positions, theta, nope, pe, flat_idx, nthreads=None) -> np.ndarray:
    """dW at flat indices g*nh + h, each a full sum over (s, c); bf16 inputs."""
    dY, O, kind = _same_kind(dY, O, "dY", "O")
    assert kind == "bf16"
    sq, nh, d = dY.shape
    p = _positions(positions, sq)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    out = np.empty(idx.shape[0], np.float64)
    nt = default_threads() if nthreads is None else nthreads
    _check_rc(_load().oracle_bwd_dw_at_bf16(_ptr(dY), _ptr(O), _ptr(p), float(theta), sq, nh,
                                            nope, pe, _ptr(idx), idx.shape[0], _ptr(out), nt),
              "bwd_dw_at")
    return out


def kv_remap(idx, sq, seqlen_kv, pad_value=-1) -> np.ndarray:
    """Flat-global KV column indices: idx [b*sq, topk] int32; row r belongs to
    batch r // sq; valid (>= 0) entries get + batch * seqlen_kv, negative
    entries become pad_value."""
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    rows, topk = idx.shape
    out = np.empty_like(idx)
    _check_rc(_load().oracle_kv_remap(_ptr(idx), rows, int(sq), topk, int(seqlen_kv),
                                      int(pad_value), _ptr(out)), "kv_remap")
    return out
