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
    for code in range(7):
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


def test_column_linear_validation(lib):
    """The base projection and the fused-epilogue call refuse bad host
    arguments before any launch: fp32, a slice width that is not a multiple
    of 256, `in` not a multiple of 8, a buffer of 2 GiB or more, null or
    misaligned pointers, a short or misaligned workspace."""
    f = lib.lora_column_linear
    sl = _slices(512, 256)
    assert f(0, A16, A16, A16, 300, 512, sl, 2, None) == UNSUPPORTED
    assert f(1, A16, A16, A16, 300, 512, _slices(504), 1, None) == UNSUPPORTED
    assert f(1, A16, A16, A16, 300, 512, _slices(500), 1, None) == ALIGN      # not 8-element rows
    assert f(1, A16, A16, A16, 300, 516, sl, 2, None) == UNSUPPORTED
    assert f(1, A16, A16, A16, 1 << 20, 512, _slices(1024), 1, None) == UNSUPPORTED   # y of 2 GiB
    assert f(1, A16, A16, A16, -1, 512, sl, 2, None) == INVALID
    assert f(1, None, A16, A16, 300, 512, sl, 2, None) == INVALID
    assert f(1, MIS, A16, A16, 300, 512, sl, 2, None) == ALIGN
    assert f(1, None, None, None, 0, 512, sl, 2, None) == OK      # nothing to do

    g = lib.lora_fused_column_linear
    need = lib.lora_fused_column_linear_workspace_bytes(300, 512, 2, 16)
    assert need >= 300 * 2 * 16 * 4
    assert lib.lora_fused_column_linear_workspace_bytes(-1, 512, 2, 16) == 0

    def call(dtype=1, x=A16, T=300, inf=512, widths=(512, 256), R=16, order=A16, ws=A16,
             nbytes=need):
        return g(dtype, x, A16, A16, T, inf, _slices(*widths), len(widths), A16, A16, 8, R,
                 order, A16, A16, A16, ws, nbytes, None)

    assert call(dtype=0) == UNSUPPORTED
    assert call(widths=(504,)) == UNSUPPORTED
    assert call(inf=516) == UNSUPPORTED
    assert call(R=0) == UNSUPPORTED
    assert call(x=None) == INVALID
    assert call(order=None) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(nbytes=need - 1) == WORKSPACE
    assert call(ws=A16 + 16) == ALIGN             # workspace must be 256-byte aligned
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


def test_apply_linear_path_predicate(lib):
    """The kernel family lora_apply_linear picks for a shape, queried on the
    host: fused for a small bf16 batch, the segment tiles for a large one,
    the vector kernels for fp32 and wherever a buffer the MFMA kernels read
    through 32-bit offsets (x, y, h, one slot's A or B) reaches 2 GiB."""
    VALU, FUSED, SEGMENT = 0, 1, 2
    f = lib.lora_apply_linear_path
    qkv = _slices(4096, 1024, 1024)
    assert f(1, 256, 4096, qkv, 3, 16) == FUSED
    assert f(1, 8192, 4096, _slices(14336, 14336), 2, 64) == SEGMENT
    assert f(0, 256, 4096, qkv, 3, 16) == VALU                    # fp32
    # h = T * S * R * 4 bytes: 2^21 tokens at R = 128 hold 1 GiB, at R = 256 2 GiB
    T = 1 << 21
    assert f(1, T, 8, _slices(16), 1, 128) == SEGMENT
    assert f(1, T, 8, _slices(16), 1, 256) == VALU
    assert f(1, T // 2, 8, _slices(16, 16), 2, 256) == VALU      # two slices of h
    assert f(1, T // 2, 8, _slices(16), 1, 256) == SEGMENT
    # y of 2 GiB (T * out * 2) and x of 2 GiB (T * in * 2)
    assert f(1, 1 << 16, 8, _slices(1 << 14), 1, 16) == VALU
    assert f(1, 1 << 16, 1 << 14, _slices(16), 1, 16) == VALU
    # bad arguments come back as a negated status
    assert f(7, 256, 4096, qkv, 3, 16) == -UNSUPPORTED
    assert f(1, -1, 4096, qkv, 3, 16) == -INVALID
    assert f(1, 256, 4096, qkv, 9, 16) == -UNSUPPORTED
    assert f(1, 256, 4096, _slices(12), 1, 16) == -ALIGN


def test_from_slots_validation_and_path(lib):
    """The one-launch form (addressing built in the same call) refuses bad
    host arguments before any launch, sizes its workspace as the apply's
    plus the addressing's, and is one launch exactly for the fused path of
    a batch of at most 1024 tokens over at most 63 slots."""
    qkv = _slices(4096, 1024, 1024)
    one = lib.lora_apply_linear_from_slots_one_launch
    assert one(1, 256, 4096, qkv, 3, 32, 16) == 1
    assert one(1, 1, 4096, qkv, 3, 63, 16) == 1
    assert one(1, 1023, 4096, qkv, 3, 32, 16) == 1
    assert one(1, 256, 4096, qkv, 3, 64, 16) == 0                 # the sort needs 64 keys or fewer
    assert one(1, 1024, 4096, qkv, 3, 32, 16) == 0                # segment path
    assert one(0, 256, 4096, qkv, 3, 32, 16) == 0                 # fp32: vector kernels
    assert one(1, 0, 4096, qkv, 3, 32, 16) == 0
    assert one(7, 256, 4096, qkv, 3, 32, 16) == -UNSUPPORTED
    assert one(1, 256, 4096, qkv, 3, 0, 16) == -UNSUPPORTED

    wsb = lib.lora_apply_linear_from_slots_workspace_bytes
    apply_need = lib.lora_apply_linear_workspace_bytes(256, 4096, 32, 3, 16)
    assert wsb(256, 4096, 32, 3, 16) == (apply_need + 255) // 256 * 256
    big = lib.lora_apply_linear_workspace_bytes(8192, 4096, 32, 3, 16)
    assert wsb(8192, 4096, 32, 3, 16) == (big + 255) // 256 * 256 + 8 * 33 * 4   # two-pass sort
    assert wsb(-1, 4096, 32, 3, 16) == 0
    need = wsb(256, 4096, 32, 3, 16)

    f = lib.lora_apply_linear_from_slots

    def call(dtype=1, x=A16, T=256, inf=4096, R=16, slot=A16, order=A16, indptr=A16, ranks=A16,
             ws=A16, nbytes=need):
        return f(dtype, x, A16, T, inf, qkv, 3, A16, A16, 32, R, slot, order, indptr, ranks,
                 A16, ws, nbytes, None)

    assert call(dtype=5) == UNSUPPORTED
    assert call(R=0) == UNSUPPORTED
    assert call(T=-1) == INVALID
    assert call(inf=0) == INVALID
    assert call(indptr=None) == INVALID
    assert call(slot=None) == INVALID
    assert call(order=None) == INVALID
    assert call(ranks=None) == INVALID
    assert call(x=None) == INVALID
    assert call(x=MIS) == ALIGN
    assert call(inf=4100) == ALIGN
    assert call(ws=None) == WORKSPACE
    assert call(nbytes=need - 1) == WORKSPACE
    assert call(ws=A16 + 16) == ALIGN


def test_from_experts_validation_and_path(lib):
    """The routed-expert one-launch form refuses bad host arguments before any
    launch, sizes its workspace as the apply's (over experts x slots pool
    entries) plus the expert addressing's, and is one launch exactly for the
    fused path of fewer than 1024 rows, at most 63 experts and 1023 pool
    entries."""
    gu = _slices(14336, 14336)
    one = lib.lora_apply_linear_from_experts_one_launch
    assert one(1, 512, 4096, gu, 2, 8, 32, 16) == 1
    assert one(1, 1023, 256, _slices(64), 1, 63, 16, 16) == 1
    assert one(1, 600, 256, _slices(64), 1, 1, 1023, 16) == 1
    assert one(1, 600, 256, _slices(64), 1, 64, 8, 16) == 0       # 65 bounds
    assert one(1, 600, 256, _slices(64), 1, 32, 32, 16) == 0      # 1024 pool entries
    assert one(1, 1024, 256, _slices(64), 1, 8, 16, 16) == 0      # segment tiles
    assert one(0, 512, 256, _slices(64), 1, 8, 16, 16) == 0       # fp32
    assert one(1, 0, 256, _slices(64), 1, 8, 16, 16) == 0
    assert one(1, 512, 256, _slices(64), 1, 0, 16, 16) == -UNSUPPORTED
    assert one(1, 512, 256, _slices(64), 1, 128, 128, 16) == -UNSUPPORTED   # > 8192 entries

    wsb = lib.lora_apply_linear_from_experts_workspace_bytes
    apply_need = lib.lora_apply_linear_workspace_bytes(512, 4096, 256, 2, 16)
    addr_need = lib.lora_build_addressing_experts_workspace_bytes(512, 8, 32)
    assert addr_need > 0
    assert wsb(512, 4096, 8, 32, 2, 16) == (apply_need + 255) // 256 * 256 + addr_need
    assert wsb(512, 4096, 0, 32, 2, 16) == 0
    assert wsb(-1, 4096, 8, 32, 2, 16) == 0
    need = wsb(512, 4096, 8, 32, 2, 16)

    f = lib.lora_apply_linear_from_experts

    def call(dtype=1, x=A16, T=512, inf=4096, E=8, S=32, R=16, rs=A16, offs=A16, order=A16,
             indptr=A16, ranks=A16, ws=A16, nbytes=need):
        return f(dtype, x, A16, T, inf, gu, 2, A16, A16, E, S, R, rs, offs, order, indptr, ranks,
                 A16, ws, nbytes, None)

    assert call(dtype=5) == UNSUPPORTED
    assert call(E=0) == UNSUPPORTED
    assert call(S=9000) == UNSUPPORTED
    assert call(R=0) == UNSUPPORTED
    assert call(T=-1) == INVALID
    assert call(indptr=None) == INVALID
    assert call(offs=None) == INVALID
    assert call(rs=None) == INVALID
    assert call(order=None) == INVALID
    assert call(ranks=None) == INVALID
    assert call(x=None) == INVALID
    assert call(x=MIS) == ALIGN
    assert call(ws=None) == WORKSPACE
    assert call(nbytes=need - 1) == WORKSPACE
    assert call(ws=A16 + 16) == ALIGN


def test_noalloc_limits_checked_on_host(lib):
    """lora_apply_linear_noalloc refuses sizes beyond its static scratch array
    (LORA_ERR_SCRATCH_LIMIT) and bad scalars (as lora_apply_linear does)
    before any HIP call, so these run without a GPU."""
    SCRATCH_LIMIT = 6
    assert lib.lora_noalloc_scratch_bytes() == 128 << 20
    f = lib.lora_apply_linear_noalloc
    qkv = _slices(4096, 1024, 1024)
    # h alone of 2^20 tokens x 48 columns x 4 bytes = 192 MiB
    assert lib.lora_apply_linear_workspace_bytes(1 << 20, 4096, 32, 3, 16) > 128 << 20
    assert f(1, A16, A16, 1 << 20, 4096, qkv, 3, A16, A16, 32, 16, A16, A16, A16, A16,
             None) == SCRATCH_LIMIT
    assert f(1, A16, A16, 256, 4096, qkv, 3, A16, A16, 32, 0, A16, A16, A16, A16,
             None) == UNSUPPORTED                                  # R = 0
    assert f(1, A16, A16, -5, 4096, qkv, 3, A16, A16, 32, 16, A16, A16, A16, A16,
             None) == INVALID                                      # T < 0
