"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.

Pointers passed here are fake (never dereferenced): every call below must fail
validation, which happens before the library touches the HIP runtime."""
import ctypes
import os
import re

import pytest

import kernelized_linear_attention_chunked_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "liblinattn.h")

OK, NULL_ARG, DTYPE, SHAPE, STATE, BAD_ARG, UNSUPPORTED, WORKSPACE, DEVICE = range(9)
P = ctypes.c_void_p


def fake(addr):
    return ctypes.c_void_p(addr)


@pytest.fixture(scope="module")
def lib():
    return la.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:la_status|const char\*)\s+(la_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 14
    assert sorted(la.EXPORTED_SYMBOLS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in enumerate(["LA_OK", "LA_ERR_NULL_ARG", "LA_ERR_DTYPE", "LA_ERR_SHAPE",
                                 "LA_ERR_STATE", "LA_ERR_BAD_ARG", "LA_ERR_UNSUPPORTED",
                                 "LA_ERR_WORKSPACE", "LA_ERR_DEVICE"]):
        assert lib.la_status_string(code).decode() == name


def fwd(lib, q=0x10000, k=0x20000000, v=0x40000000, mask=None, sik=None, sikk=None, sok=None,
        sokk=None, causal=1, fm=0, norm=1, eps=1e-6, out=0x60000000, B=2, T=100, H=4, Dk=64,
        Dv=64, dtype=1, ws=None, wsb=0):
    f = lambda a: None if a is None else fake(a)
    return lib.la_forward(f(q), f(k), f(v), f(mask), f(sik), f(sikk), f(sok), f(sokk), causal, fm,
                          norm, eps, f(out), B, T, H, Dk, Dv, dtype, f(ws), wsb, None)


def test_forward_argument_errors(lib):
    big = 1 << 40  # far-apart fake buffers
    assert fwd(lib, dtype=7) == DTYPE                      # non-floating dtype code
    assert fwd(lib, B=-1) == SHAPE
    assert fwd(lib, H=0) == SHAPE
    assert fwd(lib, Dk=48, Dv=48) == UNSUPPORTED
    assert fwd(lib, Dk=64, Dv=96) == UNSUPPORTED
    # Dk != Dv is accepted (each 32, 64 or 128): its checks use each side's size
    assert fwd(lib, Dk=64, Dv=128, causal=0) == WORKSPACE
    n = ctypes.c_size_t(0)
    assert lib.la_workspace_size(4, 16384, 16, 64, 128, 1, 0, ctypes.byref(n)) == OK
    assert n.value == 64 * 8 * (64 * 128 + 64) * 4
    assert fwd(lib, Dk=128, Dv=32, out=0x10000 + 2 * 100 * 4 * 128 * 2 - 16) == BAD_ARG  # out inside q (Dk wide)
    assert fwd(lib, fm=5) == BAD_ARG
    assert fwd(lib, eps=-1.0) == BAD_ARG
    assert fwd(lib, eps=float("nan")) == BAD_ARG
    assert fwd(lib, q=None) == NULL_ARG
    assert fwd(lib, out=None) == NULL_ARG
    # non-causal attention exposes no state
    assert fwd(lib, causal=0, sik=big, sikk=2 * big) == STATE
    assert fwd(lib, causal=0, sok=big, sokk=2 * big) == STATE
    # normalized state needs both parts; unnormalized only kv
    assert fwd(lib, sik=big) == STATE
    assert fwd(lib, sok=big) == STATE
    assert fwd(lib, norm=0, sik=big, sikk=2 * big) == STATE
    # alignment
    assert fwd(lib, q=0x10008) == BAD_ARG
    # out overlapping q
    assert fwd(lib, out=0x10000 + 64) == BAD_ARG
    # partial overlap of state_out with state_in (exact aliasing is allowed)
    assert fwd(lib, sik=big, sikk=2 * big, sok=big + 256, sokk=3 * big) == BAD_ARG
    # the workspace is required for a split sequence (few units) ...
    assert fwd(lib, B=1, H=2, T=4096) == WORKSPACE
    n = ctypes.c_size_t(0)
    assert lib.la_workspace_size(1, 4096, 2, 64, 64, 1, 1, ctypes.byref(n)) == OK
    assert fwd(lib, B=1, H=2, T=4096, ws=big, wsb=n.value - 16) == WORKSPACE
    # ... and for every non-causal call
    assert fwd(lib, causal=0) == WORKSPACE
    assert la.load_library().la_last_error_message().decode() != ""


def test_workspace_sizes(lib):
    n = ctypes.c_size_t(0)
    # enough (batch, head) units: one pass, no workspace
    assert lib.la_workspace_size(256, 1024, 32, 128, 128, 1, 1, ctypes.byref(n)) == OK
    assert n.value == 0
    # 128 units of 32 chunks: split into 4 segments of 8 chunks
    assert lib.la_workspace_size(8, 2048, 16, 64, 64, 1, 1, ctypes.byref(n)) == OK
    assert n.value == 128 * 4 * (64 * 64 + 64) * 4
    # non-causal: 64 units of 256 chunks split 8 ways
    assert lib.la_workspace_size(4, 16384, 16, 128, 128, 1, 0, ctypes.byref(n)) == OK
    assert n.value == 64 * 8 * (128 * 128 + 128) * 4
    # T == 0 needs nothing
    assert lib.la_workspace_size(4, 0, 16, 128, 128, 1, 0, ctypes.byref(n)) == OK
    assert n.value == 0
    assert lib.la_workspace_size(4, 16, 16, 128, 128, 9, 0, ctypes.byref(n)) == DTYPE
    # the workspace holds fp32 state partials: the same for every I/O dtype
    for dt in (0, 2):
        m = ctypes.c_size_t(0)
        assert lib.la_workspace_size(4, 16384, 16, 128, 128, dt, 0, ctypes.byref(m)) == OK
        assert m.value == 64 * 8 * (128 * 128 + 128) * 4
    assert lib.la_workspace_size(4, 16, 16, 128, 128, 3, 0, ctypes.byref(n)) == DTYPE
    assert lib.la_workspace_size(4, 16, 16, 128, 128, 1, 0, None) == NULL_ARG


def test_step_argument_errors(lib):
    f = fake
    base = dict(q=f(0x10000), k=f(0x20000), v=f(0x30000), m=None, si=f(1 << 32), sik=f(1 << 33),
                so=f(1 << 32), sok=f(1 << 33), fm=0, norm=1, eps=1e-6, out=f(0x40000), B=2, H=3,
                Dk=128, Dv=128, dt=1)

    def step(**kw):
        a = dict(base, **kw)
        return lib.la_step(a["q"], a["k"], a["v"], a["m"], a["si"], a["sik"], a["so"], a["sok"],
                           a["fm"], a["norm"], a["eps"], a["out"], a["B"], a["H"], a["Dk"], a["Dv"],
                           a["dt"], None)

    assert step(si=None) == STATE
    assert step(sik=None) == STATE
    assert step(norm=0) == STATE              # k parts given without the normalizer
    assert step(dt=3) == DTYPE
    assert step(Dk=96, Dv=96) == UNSUPPORTED
    assert step(Dk=128, Dv=64, out=f(0x10000 + 2 * 3 * 128 * 2 - 16)) == BAD_ARG  # out inside q (Dk wide)
    assert step(out=f(0x10000)) == BAD_ARG    # out aliases q
    assert step(so=f((1 << 32) + 512)) == BAD_ARG


def test_gated_argument_errors(lib):
    f = fake
    n = ctypes.c_size_t(0)
    assert lib.la_gated_workspace_size(2, 64, 6, 4, 128, 128, 1, 0, ctypes.byref(n)) == SHAPE
    # any group size is accepted (6 query heads per kv head: three groups of 2)
    assert lib.la_gated_workspace_size(2, 64, 48, 8, 128, 128, 1, 0, ctypes.byref(n)) == OK
    assert lib.la_gated_workspace_size(2, 64, 48, 8, 96, 96, 1, 0, ctypes.byref(n)) == UNSUPPORTED
    assert lib.la_gated_workspace_size(2, 32768, 32, 8, 128, 128, 1, 0, ctypes.byref(n)) == OK
    assert n.value > 0
    # 16 units of 512 chunks split 32 ways: D*D state slots plus the decay factors
    # of each slot (one, or one per key dim)
    assert n.value == 16 * 32 * 128 * 128 * 4 + 16 * 32 * 4
    m = ctypes.c_size_t(0)
    assert lib.la_gated_workspace_size(2, 32768, 32, 8, 128, 128, 1, 1, ctypes.byref(m)) == OK
    # ... plus one strong-decay flag (int) per (unit, segment) with a per-dim decay
    assert m.value == 16 * 32 * 128 * 128 * 4 + 16 * 32 * 128 * 4 + 16 * 32 * 4
    # without a split a per-dim decay still needs its flags: 2 units, padded to 16 bytes
    assert lib.la_gated_workspace_size(1, 64, 4, 2, 64, 64, 1, 0, ctypes.byref(m)) == OK and m.value == 0
    assert lib.la_gated_workspace_size(1, 64, 4, 2, 64, 64, 1, 1, ctypes.byref(m)) == OK and m.value == 16

    def g(**kw):
        a = dict(q=f(1 << 30), k=f(2 << 30), v=f(3 << 30), d=None, pd=0, past=None, pres=f(4 << 30),
                 out=f(5 << 30), B=1, T=64, Hq=4, Hkv=2, Dk=64, Dv=64, dt=1, scale=0.0, ws=None,
                 wsb=0)
        a.update(kw)
        return lib.la_gated_forward(a["q"], a["k"], a["v"], a["d"], a["pd"], a["past"], a["pres"], a["out"],
                                    a["B"], a["T"], a["Hq"], a["Hkv"], a["Dk"], a["Dv"], a["dt"],
                                    ctypes.c_float(a["scale"]), a["ws"], a["wsb"], None)

    assert g(Hq=3) == SHAPE
    assert g(Hkv=0) == SHAPE
    assert g(pres=None) == NULL_ARG
    assert g(dt=5) == DTYPE
    assert g(scale=float("inf")) == BAD_ARG
    assert g(T=4096) == WORKSPACE             # 2 units: the sequence is split
    assert g(d=f(6 << 30), pd=1) == WORKSPACE  # a per-dim decay's strong-decay flags
    assert g(d=f(6 << 30), pd=1, ws=f(7 << 30), wsb=8) == WORKSPACE
    assert g(out=f(1 << 30)) == BAD_ARG       # out aliases q
    # fp32 per-dim decay at head size 128 runs token by token: no workspace
    n = ctypes.c_size_t(1)
    assert lib.la_gated_workspace_size(1, 4096, 4, 2, 128, 128, 0, 1, ctypes.byref(n)) == OK and n.value == 0
    assert lib.la_gated_workspace_size(1, 4096, 4, 2, 128, 128, 1, 1, ctypes.byref(n)) == OK and n.value > 0
    # a per-dim decay overlapping out (its extent is Hkv*Dk per token)
    assert g(d=f((5 << 30) - 64 * 2 * 64 * 2 + 16), pd=1) == BAD_ARG
    assert g(d=f((6 << 30) + 2), pd=1) == BAD_ARG  # per-dim decays are read as 16-byte vectors


def test_gated_step_argument_errors(lib):
    f = fake

    def g(**kw):
        a = dict(q=f(1 << 30), k=f(2 << 30), v=f(3 << 30), d=None, past=f(6 << 30), pres=f(6 << 30),
                 out=f(5 << 30), B=2, Hq=8, Hkv=2, Dk=128, Dv=128, dt=2, scale=0.0)
        a.update(kw)
        return lib.la_gated_step(a["q"], a["k"], a["v"], a["d"], 0, a["past"], a["pres"], a["out"],
                                 a["B"], a["Hq"], a["Hkv"], a["Dk"], a["Dv"], a["dt"],
                                 ctypes.c_float(a["scale"]), None)

    assert g(Hq=3) == SHAPE
    assert g(Hq=2 * 16, q=None) == NULL_ARG   # 16 query heads per kv head pass the shape checks
    assert g(Dk=96, Dv=96) == UNSUPPORTED
    assert g(dt=3) == DTYPE
    assert g(pres=None) == NULL_ARG
    assert g(q=None) == NULL_ARG
    assert g(scale=float("nan")) == BAD_ARG
    assert g(out=f(1 << 30)) == BAD_ARG       # out aliases q
    assert g(pres=f((6 << 30) + 4096)) == BAD_ARG  # partial overlap of the states
    assert g(past=f((6 << 30) + 4)) == BAD_ARG     # misaligned state
    assert g(B=0) == OK                       # nothing to do, nothing touched


def test_delta_argument_errors(lib):
    f = fake

    def g(**kw):
        a = dict(q=f(1 << 30), k=f(2 << 30), v=f(3 << 30), d=None, pd=0, beta=f(7 << 30), bph=1,
                 past=None, pres=f(4 << 30), out=f(5 << 30), B=1, T=64, Hq=4, Hkv=2, Dk=64, Dv=64,
                 dt=1, scale=0.0, ws=None, wsb=0)
        a.update(kw)
        return lib.la_delta_forward(a["q"], a["k"], a["v"], a["d"], a["pd"], a["beta"], a["bph"],
                                    a["past"], a["pres"], a["out"], a["B"], a["T"], a["Hq"], a["Hkv"],
                                    a["Dk"], a["Dv"], a["dt"], ctypes.c_float(a["scale"]), a["ws"], a["wsb"], None)

    assert g(Hq=3) == SHAPE
    assert g(dt=4) == DTYPE
    assert g(beta=None) == NULL_ARG           # the delta rules need beta
    assert g(pres=None) == NULL_ARG
    assert g(Dk=96, Dv=96) == UNSUPPORTED
    assert g(dt=0, Dk=128, Dv=128, d=f((6 << 30) + 2), pd=1) == BAD_ARG  # misaligned per-dim decay
    assert g(scale=float("inf")) == BAD_ARG
    assert g(out=f(1 << 30)) == BAD_ARG       # out aliases q
    assert g(beta=f((5 << 30) + 64)) == BAD_ARG  # beta inside out
    assert g(d=f((6 << 30) + 2), pd=1) == BAD_ARG  # per-dim decays are read as 16-byte vectors
    assert g(ws=f((8 << 30) + 4), wsb=1 << 20) == BAD_ARG  # the workspace is 16-byte aligned
    assert g(ws=f((5 << 30) + 256), wsb=1 << 20) == BAD_ARG  # and overlaps no argument
    assert g(B=0) == OK


def test_delta_split_plan(lib):
    """Few (batch, kv head) units and a long sequence: the delta rules split over
    T, and the workspace holds the maps M, N of every segment but the last, the
    start state of every segment and the identity (D x D fp32 each)."""
    n = ctypes.c_size_t(0)
    E = 128 * 128 * 4
    # B=2, Hkv=8, G=4 (one query-head group per unit): 16 units, 512 chunks -> 16 segments
    assert lib.la_delta_workspace_size(2, 32768, 32, 8, 128, 128, 1, 0, ctypes.byref(n)) == OK
    assert n.value == E * (16 * 15 * 2 + 16 * 16 + 1)
    # enough units already (B=32, Hkv=8), T == 1, or too few chunks per segment: no split
    for args in ((32, 4096, 32, 8), (2, 1, 32, 8), (2, 200, 32, 8)):
        assert lib.la_delta_workspace_size(*args, 128, 128, 1, 0, ctypes.byref(n)) == OK and n.value == 0
    # fp32 at head size 128 with a per-dim decay runs token by token: no split
    assert lib.la_delta_workspace_size(1, 4096, 8, 1, 128, 128, 0, 1, ctypes.byref(n)) == OK and n.value == 0


def test_backward_argument_errors(lib):
    f = fake
    n = ctypes.c_size_t(0)
    assert lib.la_backward_workspace_size(2, 128, 3, 64, 64, 1, 1, ctypes.byref(n)) == OK and n.value > 0
    assert lib.la_backward_workspace_size(2, 0, 3, 64, 64, 1, 1, ctypes.byref(n)) == OK and n.value == 0
    big = 1 << 34

    def g(**kw):
        a = dict(q=f(1 << 30), k=f(2 << 30), v=f(3 << 30), m=None, si=None, sik=None, dout=f(4 << 30),
                 dso=None, dsok=None, fm=0, norm=1, eps=1e-6, dq=f(5 << 30), dk=f(6 << 30), dv=f(7 << 30),
                 dsi=f(8 << 30), dsik=f(9 << 30), B=1, T=64, H=2, Dk=64, Dv=64, dt=1, ws=f(big), wsb=1 << 40)
        a.update(kw)
        return lib.la_backward(a["q"], a["k"], a["v"], a["m"], a["si"], a["sik"], a["dout"], a["dso"],
                               a["dsok"], a["fm"], a["norm"], ctypes.c_float(a["eps"]), a["dq"], a["dk"], a["dv"],
                               a["dsi"], a["dsik"], a["B"], a["T"], a["H"], a["Dk"], a["Dv"], a["dt"], a["ws"],
                               a["wsb"], None)

    assert g(dt=5) == DTYPE
    assert g(fm=3) == BAD_ARG
    assert g(dsi=None) == NULL_ARG
    assert g(dsik=None) == NULL_ARG           # the normalizer's k-state gradient is required
    assert g(norm=0) == STATE                 # k parts given without the normalizer
    assert g(si=f(10 << 30)) == STATE         # kv state without its k part
    assert g(dq=f(1 << 30)) == BAD_ARG        # dq aliases q
    assert g(dq=f((5 << 30) + 8)) == BAD_ARG  # gradients are written as 16-byte vectors
    assert g(dout=f((4 << 30) + 4)) == BAD_ARG
    assert g(dk=f(5 << 30)) == BAD_ARG        # dk overlaps dq
    assert g(ws=None, wsb=0) == WORKSPACE
    assert g(Dk=96, Dv=96) == UNSUPPORTED
    assert g(Dk=64, Dv=128) == UNSUPPORTED   # unequal head sizes: 32 or 64 each, 16-bit inputs
    assert g(Dk=32, Dv=64, dt=0) == UNSUPPORTED
    for dt in (1, 2):
        for dk, dv in ((32, 64), (64, 32)):
            assert lib.la_backward_workspace_size(2, 128, 3, dk, dv, dt, 1, ctypes.byref(n)) == OK and n.value > 0
    assert g(B=0) == OK


def test_binding_buffer_checks_on_host_tensors():
    """The binding's argument checks (device-independent): outputs must be
    contiguous with the exact dtype and shape; inputs are copied when strided
    and rejected when their dtype or shape is wrong."""
    import torch
    x = torch.zeros((2, 3, 4, 4))
    assert la._output(x, "x", "cpu", torch.float32, (2, 3, 4, 4)) is x
    with pytest.raises(ValueError):
        la._output(x.transpose(2, 3), "x", "cpu", torch.float32, (2, 3, 4, 4))
    with pytest.raises(ValueError):
        la._output(x.to(torch.bfloat16), "x", "cpu", torch.float32, (2, 3, 4, 4))
    with pytest.raises(ValueError):
        la._output(x, "x", "cpu", torch.float32, (2, 3, 4, 5))
    y = la._input(x.transpose(2, 3), "y", "cpu", torch.float32, (2, 3, 4, 4))
    assert y.is_contiguous() and torch.equal(y, x.transpose(2, 3))
    with pytest.raises(ValueError):
        la._input(x.to(torch.bfloat16), "y", "cpu", torch.float32)
    # state pairs: the k part follows the normaliser setting
    z = torch.zeros((2, 3, 4))
    assert la._state_pair((x, z), 2, 3, 4, 4, True, "cpu", "s", output=True)[0] is x
    with pytest.raises(ValueError):
        la._state_pair((x, z), 2, 3, 4, 4, False, "cpu", "s", output=True)
    with pytest.raises(ValueError):
        la._state_pair((x, None), 2, 3, 4, 4, True, "cpu", "s", output=False)
    # a workspace smaller than needed, or strided, is refused
    with pytest.raises(ValueError):
        la._workspace(torch.empty(8, dtype=torch.uint8), 16, "cpu")
    ws, n = la._workspace(torch.empty(4, dtype=torch.float32), 16, "cpu")
    assert n == 16


def test_forward_noalloc_host_checks(lib):
    """The allocation-free forward validates like la_forward, and refuses a
    non-causal call whose sums exceed its scratch array, all before any HIP
    call (the pointers here are fake)."""
    f = lambda a: None if a is None else fake(a)

    def g(**kw):
        a = dict(q=0x10000, k=0x20000000, v=0x40000000, mask=None, sik=None, sikk=None, sok=None, sokk=None,
                 causal=1, fm=0, norm=1, eps=1e-6, out=0x60000000, B=2, T=100, H=4, Dk=64, Dv=64, dtype=1)
        a.update(kw)
        return lib.la_forward_noalloc(f(a["q"]), f(a["k"]), f(a["v"]), f(a["mask"]), f(a["sik"]), f(a["sikk"]),
                                      f(a["sok"]), f(a["sokk"]), a["causal"], a["fm"], a["norm"], a["eps"],
                                      f(a["out"]), a["B"], a["T"], a["H"], a["Dk"], a["Dv"], a["dtype"], None)

    big = 1 << 40
    assert g(dtype=7) == DTYPE
    assert g(q=None) == NULL_ARG
    assert g(causal=0, sik=big, sikk=2 * big) == STATE
    assert g(out=0x10000 + 64) == BAD_ARG
    # 1024 (batch, head) units at Dk = Dv = 128 need 1024 * 66048 bytes > 64 MiB
    assert g(causal=0, B=8, H=128, T=64, Dk=128, Dv=128, q=1 << 36, k=2 << 36, v=3 << 36,
             out=4 << 36) == WORKSPACE
    assert b"scratch" in lib.la_last_error_message()
