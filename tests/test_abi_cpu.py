"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad host arguments before anything is enqueued.
No call here reaches a kernel launch (no GPU is needed)."""
import ctypes
import os
import re

import pytest

import adapter_lora_serving_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_mi355x.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.lib_path()):
        from adapter_lora_serving_amd import build
        build.build()
    return L.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_\w+)\s*\(", text)))


def test_header_symbols_exported(lib):
    names = header_functions()
    assert "lora_apply_linear" in names and "lora_build_addressing" in names
    for n in names:
        assert hasattr(lib, n), n
    # the Python binding declares a signature for every exported entry point
    assert sorted(L.SIGNATURES) == names


def test_status_strings(lib):
    for code in range(6):
        assert lib.lora_status_string(code)
    assert lib.lora_status_string(99) == b"unknown status"
    assert b"gfx950" in lib.lora_version()


A16 = 0x10000        # an aligned fake device address (never dereferenced here)
MIS = 0x10008        # 8-byte aligned only


def _slices(*w):
    return (ctypes.c_int64 * len(w))(*w)


def test_shrink_validation(lib):
    f = lib.lora_shrink
    args = dict(dtype=1, x=A16, T=4, inf=64, a=A16, slots=2, S=1, R=16, order=A16, indptr=A16,
                ranks=A16, h=A16, ws=None, wsb=0, stream=None)

    def call(**kw):
        d = {**args, **kw}
        return f(d["dtype"], d["x"], d["T"], d["inf"], d["a"], d["slots"], d["S"], d["R"],
                 d["order"], d["indptr"], d["ranks"], d["h"], d["ws"], d["wsb"], d["stream"])

    assert call(dtype=7) == UNSUPPORTED
    assert call(T=-1) == INVALID
    assert call(slots=0) == UNSUPPORTED
    assert call(slots=8193) == UNSUPPORTED
    assert call(R=0) == UNSUPPORTED
    assert call(R=260) == UNSUPPORTED
    assert call(R=12) == ALIGN                 # bf16 rows must be multiples of 8
    assert call(S=9) == UNSUPPORTED
    assert call(S=8, R=136) == UNSUPPORTED      # S*R > 1024
    assert call(inf=0) == INVALID
    assert call(x=None) == INVALID
    assert call(order=None) == INVALID
    assert call(x=MIS) == ALIGN
    assert call(inf=60) == ALIGN
    assert call(T=0, x=None, a=None, h=None) == OK    # nothing to do: no launch
    # a lent workspace must hold the K parts and be 256-byte aligned
    need = lib.lora_shrink_workspace_bytes(4, 4096, 1, 16)
    assert need == 4 * 16 * 4 * 4                  # 4 parts of a [4, 16] float32 h
    assert call(inf=4096, ws=A16, wsb=need - 1) == WORKSPACE
    assert call(inf=4096, ws=A16 + 16, wsb=need) == ALIGN
    # a shallow `in` still takes 4 parts of >= 256; below 512 one part, no workspace
    assert lib.lora_shrink_workspace_bytes(4, 1024, 1, 16) == 4 * 16 * 4 * 4
    assert lib.lora_shrink_workspace_bytes(4, 256, 1, 16) == 0
    assert lib.lora_shrink_workspace_bytes(-1, 4096, 1, 16) == 0   # bad input


def test_expand_validation(lib):
    f = lib.lora_expand

    def call(dtype=1, y=A16, T=4, sl=(64, 32), h=A16, b=A16, slots=2, R=16, order=A16,
             indptr=A16, ranks=A16, scal=A16):
        arr = None if sl is None else _slices(*sl)
        return f(dtype, y, T, arr, 0 if sl is None else len(sl), h, b, slots, R, order, indptr,
                 ranks, scal, None)

    assert call(sl=None) == UNSUPPORTED
    assert call(sl=(64, 0)) == INVALID
    assert call(sl=(64, 36)) == ALIGN
    # f32 widths only need multiples of 4 (T=0: validated, nothing launched)
    assert call(dtype=0, sl=(64, 36), T=0) == OK
    assert call(dtype=0, sl=(64, 34), T=0) == ALIGN
    assert call(sl=(8,) * 9) == UNSUPPORTED
    assert call(scal=None) == INVALID
    assert call(y=MIS) == ALIGN
    assert call(T=0, y=None, h=None, b=None) == OK


def test_gather_validation(lib):
    f = lib.lora_gather_shrink
    assert f(1, A16, 4, 0, A16, 2, 16, A16, A16, A16, A16, None) == INVALID      # vocab 0
    assert f(1, None, 4, 100, A16, 2, 16, A16, A16, A16, A16, None) == INVALID   # ids
    assert f(1, A16, 4, 100, MIS, 2, 16, A16, A16, A16, A16, None) == ALIGN
    assert f(1, A16, 0, 100, None, 2, 16, A16, A16, A16, A16, None) == OK


def test_apply_linear_validation_and_workspace(lib):
    f = lib.lora_apply_linear
    need = lib.lora_apply_linear_workspace_bytes(256, 4096, 32, 3, 16)
    assert need >= 256 * 48 * 4
    assert lib.lora_apply_linear_workspace_bytes(-1, 4096, 32, 3, 16) == 0
    sl = _slices(4096, 1024, 1024)

    def call(ws=A16, nbytes=need, T=256, inf=4096, x=A16):
        return f(1, x, A16, T, inf, sl, 3, A16, A16, 32, 16, A16, A16, A16, A16, ws, nbytes, None)

    assert call(ws=None) == WORKSPACE
    assert call(nbytes=need - 1) == WORKSPACE
    assert call(ws=A16 + 16) == ALIGN            # workspace must be 256-byte aligned
    assert call(inf=4100) == ALIGN
    assert call(x=None) == INVALID
    assert call(T=0, ws=None) == OK


def test_addressing_validation(lib):
    f = lib.lora_build_addressing
    assert f(A16, -1, 4, A16, A16, None, 0, None) == INVALID
    assert f(A16, 4, 0, A16, A16, None, 0, None) == UNSUPPORTED
    assert f(A16, 4, 4, A16, None, None, 0, None) == INVALID
    assert f(None, 4, 4, A16, A16, None, 0, None) == INVALID
    # the two-pass workspace: one count per (1024-token block, key)
    need = lib.lora_build_addressing_workspace_bytes(8192, 16)
    assert need == 8 * 17 * 4
    assert lib.lora_build_addressing_workspace_bytes(1024, 16) == 0     # one block
    assert lib.lora_build_addressing_workspace_bytes(8192, 1024) == 0   # keys > 1024
    assert lib.lora_build_addressing_workspace_bytes(-1, 16) == 0
    assert f(A16, 8192, 16, A16, A16, A16, need - 1, None) == WORKSPACE
    assert f(A16, 8192, 16, A16, A16, A16 + 8, need, None) == ALIGN


def test_binding_refuses_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    with pytest.raises(L.LoraError):
        L.build_addressing(torch.zeros(4, dtype=torch.int32), 2)
