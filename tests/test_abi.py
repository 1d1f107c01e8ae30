"""C ABI checks that need no GPU: the library loads, exports every function
include/postmix.h declares, and rejects bad arguments before any HIP call.

Pointers here are fake, suitably aligned integers: validation never
dereferences them, and every case below fails validation, so no device call
is made.
"""
import ctypes
import os
import re

import pytest

from rope_head_mixing_amd import postmix as pm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "postmix.h")

A = 0x10000      # 16-byte aligned fake device addresses, far apart
B = 0x40000000
C = 0x80000000
D = 0xC0000000
E = 0x100000000
F = 0x140000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(postmix_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["postmix_fwd", "postmix_bwd_dx", "postmix_bwd_dw", "postmix_bwd", "postmix_bwd_dw_workspace_bytes",
              "postmix_rope_table", "postmix_status_string", "postmix_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = pm.lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_exports_nothing_undeclared():
    """The shared object's dynamic symbols named postmix_* are exactly the header's."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", pm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(set(re.findall(r"\b(postmix_[a-z0-9_]+)\b", out)))
    assert exported == declared_functions()


def test_status_strings():
    L = pm.lib()
    codes = [pm.PM_OK, pm.PM_ERR_NULL, pm.PM_ERR_SHAPE, pm.PM_ERR_ALIGN, pm.PM_ERR_OVERLAP,
             pm.PM_ERR_WORKSPACE, pm.PM_ERR_DEVICE, pm.PM_ERR_HIP]
    texts = [L.postmix_status_string(c).decode() for c in codes]
    assert len(set(texts)) == len(codes)
    assert L.postmix_status_string(12345).decode() == "unknown status"


def fwd(**kw):
    args = dict(O=A, W=B, cos=C, sin=D, rows=32768, pos=E, sq=16, nh=64, nope=448, pe=64, Y=F)
    args.update(kw)
    L = pm.lib()
    rc = L.postmix_fwd(args["O"], args["W"], args["cos"], args["sin"], args["rows"], args["pos"],
                       args["sq"], args["nh"], args["nope"], args["pe"], args["Y"], None)
    return rc, L.postmix_last_error().decode()


def dx(**kw):
    args = dict(dY=A, W=B, cos=C, sin=D, rows=32768, pos=E, sq=16, nh=64, nope=448, pe=64, dO=F)
    args.update(kw)
    L = pm.lib()
    rc = L.postmix_bwd_dx(args["dY"], args["W"], args["cos"], args["sin"], args["rows"], args["pos"],
                          args["sq"], args["nh"], args["nope"], args["pe"], args["dO"], None)
    return rc, L.postmix_last_error().decode()


def dw(**kw):
    sq, nh, nope, pe = kw.get("sq", 16), kw.get("nh", 64), kw.get("nope", 448), kw.get("pe", 64)
    need = pm.lib().postmix_bwd_dw_workspace_bytes(sq, nh, nope, pe)
    args = dict(dY=A, O=B, cos=C, sin=D, rows=32768, pos=E, sq=sq, nh=nh, nope=nope, pe=pe, dW=F,
                ws=0x180000000, wsb=need)
    args.update(kw)
    L = pm.lib()
    rc = L.postmix_bwd_dw(args["dY"], args["O"], args["cos"], args["sin"], args["rows"], args["pos"],
                          args["sq"], args["nh"], args["nope"], args["pe"], args["dW"], args["ws"],
                          args["wsb"], None)
    return rc, L.postmix_last_error().decode()


@pytest.mark.parametrize("call", [fwd, dx])
@pytest.mark.parametrize("kw,code,word", [
    (dict(nh=0), pm.PM_ERR_SHAPE, "nh"),
    (dict(nh=129), pm.PM_ERR_SHAPE, "nh"),
    (dict(nope=-8), pm.PM_ERR_SHAPE, "nope"),
    (dict(nope=12), pm.PM_ERR_SHAPE, "nope"),
    (dict(pe=8), pm.PM_ERR_SHAPE, "pe"),
    (dict(pe=-16), pm.PM_ERR_SHAPE, "pe"),
    (dict(nope=0, pe=0), pm.PM_ERR_SHAPE, "nope + pe"),
    (dict(nope=(1 << 24) - 48, pe=64), pm.PM_ERR_SHAPE, "2^24"),
    (dict(nope=2 ** 31 - 8, pe=16), pm.PM_ERR_SHAPE, "2^24"),  # int32 sum would wrap
    (dict(sq=-1), pm.PM_ERR_SHAPE, "sq"),
    (dict(rows=0), pm.PM_ERR_SHAPE, "table_rows"),
    (dict(W=0), pm.PM_ERR_NULL, "W"),
    (dict(cos=0), pm.PM_ERR_NULL, "rope_cos"),
    (dict(sin=0), pm.PM_ERR_NULL, "rope_sin"),
    (dict(pos=0), pm.PM_ERR_NULL, "positions"),
    (dict(cos=C + 4), pm.PM_ERR_ALIGN, "rope_cos"),
    (dict(pos=E + 2), pm.PM_ERR_ALIGN, "positions"),
    (dict(W=B + 1), pm.PM_ERR_ALIGN, "W"),
])
def test_mix_argument_errors(call, kw, code, word):
    rc, msg = call(**kw)
    assert rc == code, msg
    assert word in msg


@pytest.mark.parametrize("call,xname,oname", [(fwd, "O", "Y"), (dx, "dY", "dO")])
def test_mix_named_tensor_errors(call, xname, oname):
    rc, msg = call(**{xname: 0})
    assert rc == pm.PM_ERR_NULL and xname in msg
    rc, msg = call(**{oname: 0})
    assert rc == pm.PM_ERR_NULL and oname in msg
    rc, msg = call(**{xname: A + 8})
    assert rc == pm.PM_ERR_ALIGN and xname in msg
    rc, msg = call(**{oname: F + 2})
    assert rc == pm.PM_ERR_ALIGN and oname in msg
    # output overlapping the input (sq*nh*d*2 bytes = 1 MiB here)
    rc, msg = call(**{oname: A + 4096})
    assert rc == pm.PM_ERR_OVERLAP and oname in msg and xname in msg
    rc, msg = call(**{oname: B})  # output on top of W
    assert rc == pm.PM_ERR_OVERLAP and "W" in msg


def test_pe_zero_does_not_need_tables():
    """With pe == 0 the tables may be NULL; the call gets past validation
    (then fails at the device check on a host without a gfx950)."""
    rc, msg = fwd(pe=0, nope=512, cos=0, sin=0, pos=0, rows=0)
    assert rc not in (pm.PM_ERR_NULL, pm.PM_ERR_SHAPE, pm.PM_ERR_ALIGN, pm.PM_ERR_OVERLAP), msg


def test_widest_rows_pass_the_shape_check():
    """nope + pe = 2^24 is the widest accepted row (then the call fails at
    the device check on a host without a gfx950)."""
    rc, msg = fwd(sq=1, nh=1, nope=(1 << 24) - 64, pe=64)
    assert rc not in (pm.PM_ERR_NULL, pm.PM_ERR_SHAPE, pm.PM_ERR_ALIGN, pm.PM_ERR_OVERLAP), msg


def test_rope_apply_shares_the_shape_limits():
    L = pm.lib()
    rc = L.postmix_rope_apply(A, C, D, 32768, E, 1, 1, (1 << 24) - 48, 64, -1, F, None)
    assert rc == pm.PM_ERR_SHAPE and "2^24" in L.postmix_last_error().decode()
    rc = L.postmix_rope_apply(A, C, D, 32768, E, 1, 0, 448, 64, -1, F, None)
    assert rc == pm.PM_ERR_SHAPE and "nh" in L.postmix_last_error().decode()


def test_empty_sq_is_a_noop_before_any_pointer_check():
    rc, _ = fwd(sq=0, O=0, Y=0, W=0)
    assert rc == pm.PM_OK
    rc, _ = dx(sq=0, dY=0, dO=0, W=0)
    assert rc == pm.PM_OK
    rc, msg = fwd(sq=0, nh=0)
    assert rc == pm.PM_ERR_SHAPE


@pytest.mark.parametrize("kw,code,word", [
    (dict(dW=0), pm.PM_ERR_NULL, "dW"),
    (dict(dY=0), pm.PM_ERR_NULL, "dY"),
    (dict(O=0), pm.PM_ERR_NULL, "O"),
    (dict(ws=0), pm.PM_ERR_NULL, "workspace"),
    (dict(wsb=256), pm.PM_ERR_WORKSPACE, "workspace"),
    (dict(ws=0x180000000 + 8), pm.PM_ERR_ALIGN, "workspace"),
    (dict(dY=A + 4), pm.PM_ERR_ALIGN, "dY"),
    (dict(dW=F + 2), pm.PM_ERR_ALIGN, "dW"),
    (dict(dW=A + 64), pm.PM_ERR_OVERLAP, "dW"),
    (dict(ws=B), pm.PM_ERR_OVERLAP, "workspace"),
    (dict(nh=200), pm.PM_ERR_SHAPE, "nh"),
    (dict(nope=(1 << 24) - 48, pe=64), pm.PM_ERR_SHAPE, "2^24"),
    (dict(pos=0), pm.PM_ERR_NULL, "positions"),
])
def test_dw_argument_errors(kw, code, word):
    rc, msg = dw(**kw)
    assert rc == code, msg
    assert word in msg


def test_workspace_size_is_a_function_of_the_shape():
    L = pm.lib()
    # sq*nh = 2^20 -> 32 tokens per block -> 512 blocks of nh*nh fp32 partials
    # nh = 64 with d a multiple of 128: the single-pass backward's 1024 blocks of 16 tokens
    assert L.postmix_bwd_dw_workspace_bytes(16384, 64, 448, 64) == 1024 * 64 * 64 * 4
    # otherwise the weight-gradient kernels' 512 blocks of 32 tokens
    assert L.postmix_bwd_dw_workspace_bytes(16384, 64, 440, 64) == 512 * 64 * 64 * 4
    # nh <= 32: several tokens per chunk; block sizes as for 64 heads, so the
    # single-pass backward's 1024 blocks again (16 and 128 tokens)
    assert L.postmix_bwd_dw_workspace_bytes(16384, 32, 448, 64) == 1024 * 32 * 32 * 4
    assert L.postmix_bwd_dw_workspace_bytes(131072, 8, 448, 64) == 1024 * 8 * 8 * 4
    # nh = 3: 21 tokens per chunk, so the single pass takes blocks of 21 tokens
    # (391 blocks); the weight-gradient kernels' 512 blocks of 16 are more
    assert L.postmix_bwd_dw_workspace_bytes(8192, 3, 448, 64) == 512 * 3 * 3 * 4
    # not fused (nh = 1 with pe = 16): the weight-gradient kernels' blocks
    assert L.postmix_bwd_dw_workspace_bytes(16384, 1, 496, 16) == 512 * 1 * 1 * 4
    # nh = 128 with pe rotated in registers: the single-pass backward's 512 blocks
    assert L.postmix_bwd_dw_workspace_bytes(8192, 128, 448, 64) == 512 * 128 * 128 * 4
    # nh = 128 with pe = 80 (not fused): the weight-gradient kernels' 256 blocks
    assert L.postmix_bwd_dw_workspace_bytes(8192, 128, 432, 80) == 256 * 128 * 128 * 4
    # single pass, last round of 256 blocks less than 3/4 full: the block count
    # goes to the nearest multiple of 256 (547 blocks of 20 tokens -> 512;
    # 834 of 12 -> 768); otherwise it stays (1000 blocks of 12 tokens)
    assert L.postmix_bwd_dw_workspace_bytes(10923, 96, 448, 64) == 512 * 96 * 96 * 4
    assert L.postmix_bwd_dw_workspace_bytes(10000, 64, 448, 64) == 768 * 64 * 64 * 4
    assert L.postmix_bwd_dw_workspace_bytes(12000, 32, 448, 64) == 1000 * 32 * 32 * 4
    # the weight-gradient kernels round the same way above 64 heads (one
    # workgroup per CU): 304 blocks of 36 tokens -> 256; not fused (pe = 80)
    assert L.postmix_bwd_dw_workspace_bytes(10923, 96, 432, 80) == 256 * 96 * 96 * 4
    # accumulation chains capped at 2^14 k-steps of 16 channels: one token of
    # 2^24 channels (2^20 k-steps) is split into 64 channel spans, each with
    # its own partial; two such tokens make 2 x 64
    assert L.postmix_bwd_dw_workspace_bytes(1, 128, (1 << 24) - 64, 64) == 64 * 128 * 128 * 4
    assert L.postmix_bwd_dw_workspace_bytes(2, 128, (1 << 24) - 64, 64) == 128 * 128 * 128 * 4
    assert L.postmix_bwd_dw_workspace_bytes(1, 128, (1 << 24) - 72, 64) == 64 * 128 * 128 * 4
    # 2^20 channels: 2^16 k-steps per token -> 4 spans per token
    assert L.postmix_bwd_dw_workspace_bytes(8, 64, (1 << 20) - 64, 64) == 32 * 64 * 64 * 4
    # 4096 channels (256 k-steps per token): the weight-gradient blocks of 256
    # tokens (65536 k-steps) and the single pass's blocks of 128 both become
    # blocks of 64 tokens (16384 k-steps): 2048 partials
    assert L.postmix_bwd_dw_workspace_bytes(131072, 64, 4032, 64) == 2048 * 64 * 64 * 4
    assert L.postmix_bwd_dw_workspace_bytes(0, 64, 448, 64) == 0
    assert L.postmix_bwd_dw_workspace_bytes(16, 0, 448, 64) == 0
    for args in [(64, 4, 48, 16), (8192, 3, 448, 64), (7, 5, 8, 16)]:
        assert L.postmix_bwd_dw_workspace_bytes(*args) % 256 == 0
        assert L.postmix_bwd_dw_workspace_bytes(*args) >= args[1] * args[1] * 4


def test_rope_table_argument_errors():
    L = pm.lib()
    assert L.postmix_rope_table(0.0, 64, 10, A, B, None) == pm.PM_ERR_SHAPE
    assert L.postmix_rope_table(1e4, 24, 10, A, B, None) == pm.PM_ERR_SHAPE
    assert L.postmix_rope_table(1e4, 64, 10, 0, B, None) == pm.PM_ERR_NULL
    assert L.postmix_rope_table(1e4, 64, 10, A + 4, B, None) == pm.PM_ERR_ALIGN
    assert L.postmix_rope_table(1e4, 64, 10, A, A + 16, None) == pm.PM_ERR_OVERLAP
    assert L.postmix_rope_table(1e4, 64, 0, 0, 0, None) == pm.PM_OK


def test_last_error_is_thread_local():
    import threading
    rc, msg = fwd(nh=0)
    assert "nh" in msg
    seen = []

    def other():
        seen.append(pm.lib().postmix_last_error().decode())

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen == [""]
    assert "nh" in pm.lib().postmix_last_error().decode()


def test_binding_rejects_wrong_dtypes_by_name():
    torch = pytest.importorskip("torch")
    O = torch.zeros((2, 4, 64), dtype=torch.float16)
    W = torch.zeros((4, 4), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="O must be torch.bfloat16"):
        pm.postmix_fwd(O, W, None, None, None, 48, 16)
    with pytest.raises(ValueError, match="dY must be torch.bfloat16"):
        pm.postmix_bwd_dw(O, O, None, None, None, 48, 16)


def test_binding_checks_shapes_before_any_launch():
    """The C ABI sees pointers and sizes only, so the binding checks every
    tensor's shape against the sizes it passes (a short W or output would
    otherwise be read or written past its end on the device).  All of these
    are CPU tensors: the shape checks come before the device check, so each
    case raises before any launch."""
    import re as _re
    torch = pytest.importorskip("torch")
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    O = torch.zeros((3, 4, 64), dtype=bf)
    W = torch.zeros((4, 4), dtype=bf)
    cos, sin = torch.zeros((8, 8), dtype=f32), torch.zeros((8, 8), dtype=f32)
    pos = torch.zeros((3,), dtype=i32)
    idx = torch.zeros((6, 16), dtype=i32)
    cases = [
        (lambda: pm.postmix_fwd(O, torch.zeros((4, 5), dtype=bf), cos, sin, pos, 48, 16), "W must have shape [4, 4]"),
        (lambda: pm.postmix_fwd(O, torch.zeros((3, 3), dtype=bf), cos, sin, pos, 48, 16), "W must have shape [4, 4]"),
        (lambda: pm.postmix_fwd(O, W, cos, sin, pos, 48, 16, out=torch.zeros((2, 4, 64), dtype=bf)),
         "out must have shape [3, 4, 64]"),
        (lambda: pm.postmix_fwd(O, W, cos, sin, pos, 40, 16), "O must have shape [sq, nh, 56]"),
        (lambda: pm.postmix_fwd(O, W, cos, torch.zeros((8, 4), dtype=f32), pos, 48, 16), "rope_sin must have shape [8, 8]"),
        (lambda: pm.postmix_fwd(O, W, cos, torch.zeros((7, 8), dtype=f32), pos, 48, 16), "rope_sin must have shape [8, 8]"),
        (lambda: pm.postmix_fwd(O, W, cos, sin, torch.zeros((2,), dtype=i32), 48, 16), "positions must have shape [3]"),
        (lambda: pm.postmix_bwd_dx(O, W, cos, sin, pos, 48, 16, out=torch.zeros((3, 4, 48), dtype=bf)),
         "out must have shape [3, 4, 64]"),
        (lambda: pm.postmix_bwd_dx(O, torch.zeros((16,), dtype=bf), cos, sin, pos, 48, 16), "W must have shape [4, 4]"),
        (lambda: pm.postmix_bwd_dw(O, torch.zeros((3, 2, 64), dtype=bf), cos, sin, pos, 48, 16),
         "O must have shape [3, 4, 64]"),
        (lambda: pm.postmix_bwd_dw(O, O, cos, sin, pos, 48, 16, out=torch.zeros((4, 3), dtype=f32)),
         "out must have shape [4, 4]"),
        (lambda: pm.postmix_bwd(O, O, torch.zeros((2, 2), dtype=bf), cos, sin, pos, 48, 16), "W must have shape [4, 4]"),
        (lambda: pm.postmix_bwd(O, O, W, cos, sin, pos, 48, 16, out_dO=torch.zeros((3, 4, 63), dtype=bf)),
         "out_dO must have shape [3, 4, 64]"),
        (lambda: pm.postmix_bwd(O, O, W, cos, sin, pos, 48, 16, out_dW=torch.zeros((5, 5), dtype=f32)),
         "out_dW must have shape [4, 4]"),
        (lambda: pm.postmix_bwd(O, O, W, cos, sin, pos, 48, 16, workspace=[0] * 4), "workspace must be a torch.Tensor"),
        (lambda: pm.postmix_rope_apply(O, cos, sin, pos, 48, 16, -1, out=torch.zeros((4, 4, 64), dtype=bf)),
         "out must have shape [3, 4, 64]"),
        (lambda: pm.postmix_kv_index_remap(idx, 3, 100, out=torch.zeros((6, 15), dtype=i32)),
         "out must have shape [6, 16]"),
        (lambda: pm.postmix_kv_index_remap(torch.zeros((96,), dtype=i32), 3, 100), "idx must be a 2-dimensional"),
    ]
    for fn, msg in cases:
        with pytest.raises(ValueError, match=_re.escape(msg)):
            fn()
    # well-formed CPU tensors pass the shape checks and stop at the device check
    with pytest.raises(ValueError, match="must be on a GPU device"):
        pm.postmix_fwd(O, W, cos, sin, pos, 48, 16)
    with pytest.raises(ValueError, match="must be on a GPU device"):
        pm.postmix_bwd(O, O, W, cos, sin, pos, 48, 16, out_dO=torch.zeros_like(O),
                       out_dW=torch.zeros((4, 4), dtype=f32))


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(pm, "_lib", None)
    monkeypatch.setattr(pm, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        pm.lib()


def bwd(**kw):
    sq, nh, nope, pe = kw.get("sq", 16), kw.get("nh", 64), kw.get("nope", 448), kw.get("pe", 64)
    need = pm.lib().postmix_bwd_dw_workspace_bytes(sq, nh, nope, pe)
    args = dict(dY=A, O=B, W=0x200000000, cos=C, sin=D, rows=32768, pos=E, sq=sq, nh=nh, nope=nope,
                pe=pe, dO=F, dW=0x240000000, ws=0x180000000, wsb=need)
    args.update(kw)
    L = pm.lib()
    rc = L.postmix_bwd(args["dY"], args["O"], args["W"], args["cos"], args["sin"], args["rows"],
                       args["pos"], args["sq"], args["nh"], args["nope"], args["pe"], args["dO"],
                       args["dW"], args["ws"], args["wsb"], None)
    return rc, L.postmix_last_error().decode()


@pytest.mark.parametrize("kw,code,word", [
    (dict(dW=0), pm.PM_ERR_NULL, "dW"),
    (dict(dO=0), pm.PM_ERR_NULL, "dO"),
    (dict(W=0), pm.PM_ERR_NULL, "W"),
    (dict(dY=0), pm.PM_ERR_NULL, "dY"),
    (dict(O=0), pm.PM_ERR_NULL, "O"),
    (dict(ws=0), pm.PM_ERR_NULL, "workspace"),
    (dict(wsb=16), pm.PM_ERR_WORKSPACE, "workspace"),
    (dict(W=0x200000000 + 1), pm.PM_ERR_ALIGN, "W"),
    (dict(dO=F + 8), pm.PM_ERR_ALIGN, "dO"),
    (dict(dO=A + 1024), pm.PM_ERR_OVERLAP, "dO"),
    (dict(dW=F + 64), pm.PM_ERR_OVERLAP, "dW"),
    (dict(ws=0x200000000), pm.PM_ERR_OVERLAP, "workspace"),
    (dict(nope=20), pm.PM_ERR_SHAPE, "nope"),
    (dict(nope=(1 << 24) - 48, pe=64), pm.PM_ERR_SHAPE, "2^24"),
    (dict(sin=0), pm.PM_ERR_NULL, "rope_sin"),
])
def test_fused_backward_argument_errors(kw, code, word):
    rc, msg = bwd(**kw)
    assert rc == code, msg
    assert word in msg


def bwd_noalloc(**kw):
    sq, nh, nope, pe = kw.get("sq", 16), kw.get("nh", 64), kw.get("nope", 448), kw.get("pe", 64)
    args = dict(dY=A, O=B, W=0x200000000, cos=C, sin=D, rows=32768, pos=E, sq=sq, nh=nh, nope=nope,
                pe=pe, dO=F, dW=0x240000000)
    args.update(kw)
    L = pm.lib()
    rc = L.postmix_bwd_noalloc(args["dY"], args["O"], args["W"], args["cos"], args["sin"], args["rows"],
                               args["pos"], args["sq"], args["nh"], args["nope"], args["pe"], args["dO"],
                               args["dW"], None)
    return rc, L.postmix_last_error().decode()


@pytest.mark.parametrize("kw,code,word", [
    (dict(dW=0), pm.PM_ERR_NULL, "dW"),
    (dict(dO=0), pm.PM_ERR_NULL, "dO"),
    (dict(W=0x200000000 + 1), pm.PM_ERR_ALIGN, "W"),
    (dict(dO=A + 1024), pm.PM_ERR_OVERLAP, "dO"),
    (dict(nh=129), pm.PM_ERR_SHAPE, "nh"),
    # 2^20 tokens at 64 heads: 2048 partials of 16 KiB, 32 MiB, fit exactly;
    # 2^21 tokens need 4096 (64 MiB), more than the static scratch
    (dict(sq=1 << 21), pm.PM_ERR_WORKSPACE, "static scratch"),
    # 16 tokens of 2^24 channels at 128 heads: 16 x 64 spans of 64 KiB
    (dict(sq=16, nh=128, nope=(1 << 24) - 64), pm.PM_ERR_WORKSPACE, "static scratch"),
])
def test_noalloc_backward_argument_errors(kw, code, word):
    """The no-allocation backward validates like postmix_bwd, and rejects
    shapes whose partials exceed its 32 MiB static scratch before any device
    call."""
    rc, msg = bwd_noalloc(**kw)
    assert rc == code, msg
    assert word in msg


def test_noalloc_scratch_covers_the_workloads():
    """The production and sweep shapes fit the 32 MiB static scratch."""
    L = pm.lib()
    for args in [(16384, 64, 448, 64), (8192, 128, 448, 64), (16384, 128, 448, 64), (8192, 3, 448, 64),
                 (1024, 64, 448, 64), (64, 4, 48, 16), (1 << 20, 64, 448, 64),
                 (4, 128, (1 << 24) - 64, 64)]:
        assert L.postmix_bwd_dw_workspace_bytes(*args) <= 32 << 20, args
    assert L.postmix_bwd_dw_workspace_bytes(1 << 21, 64, 448, 64) > 32 << 20


def remap(**kw):
    args = dict(idx=A, rows=8, sq=4, topk=16, seqlen_kv=1000, pad=-1, out=F)
    args.update(kw)
    L = pm.lib()
    rc = L.postmix_kv_index_remap(args["idx"], args["rows"], args["sq"], args["topk"],
                                  args["seqlen_kv"], args["pad"], args["out"], None)
    return rc, L.postmix_last_error().decode()


@pytest.mark.parametrize("kw,code,word", [
    (dict(rows=9), pm.PM_ERR_SHAPE, "multiple of sq"),
    (dict(sq=0), pm.PM_ERR_SHAPE, "sq"),
    (dict(topk=-1), pm.PM_ERR_SHAPE, "topk"),
    (dict(seqlen_kv=-5), pm.PM_ERR_SHAPE, "seqlen_kv"),
    (dict(rows=8, sq=1, seqlen_kv=1 << 29), pm.PM_ERR_SHAPE, "int32"),
    (dict(idx=0), pm.PM_ERR_NULL, "idx"),
    (dict(out=0), pm.PM_ERR_NULL, "out"),
    (dict(idx=A + 2), pm.PM_ERR_ALIGN, "idx"),
    (dict(out=A + 64), pm.PM_ERR_OVERLAP, "out"),
])
def test_kv_remap_argument_errors(kw, code, word):
    rc, msg = remap(**kw)
    assert rc == code, msg
    assert word in msg


def test_kv_remap_empty_and_in_place_pass_validation():
    assert remap(rows=0, idx=0, out=0)[0] == pm.PM_OK
    assert remap(topk=0, idx=0, out=0)[0] == pm.PM_OK
    rc, msg = remap(out=A)  # in place: validation passes, then the device check decides
    assert rc not in (pm.PM_ERR_NULL, pm.PM_ERR_SHAPE, pm.PM_ERR_ALIGN, pm.PM_ERR_OVERLAP), msg


def test_benchmark_kernel_names_exist_in_the_library():
    """bench.py attributes trace and counter rows to ops by kernel name; every
    name it uses must be a kernel the library actually contains."""
    import shutil
    import subprocess
    import bench
    from rope_head_mixing_amd import postmix as pm
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-C", pm.LIB_PATH], capture_output=True, text=True, check=True).stdout
    for workload, table in bench.KERNELS_BY_WORKLOAD.items():
        for op, names in table.items():
            for name in (n.strip() for n in names.split("+")):
                assert f"pm::{name}(" in out, f"{workload} {op}: kernel {name!r} not in {pm.LIB_PATH}"


def test_benchmark_refuses_more_than_one_gpu():
    """bench.py runs on one GPU; asked for more it says so and exits non-zero
    before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert r.stdout == ""
    assert "exactly one GPU" in r.stderr
