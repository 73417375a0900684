"""Batched multi-LoRA delta on MI355X: Python binding of liblora_mi355x.so.

The functions here only marshal arguments (torch tensors -> device pointers,
torch's current HIP stream) and call the C ABI declared in
include/lora_mi355x.h; every step of the computation runs in the HIP kernels
of the library. There is no fallback: if the library is not built, or no GPU
is present, the calls raise.

Names and argument order follow the LoraBackend methods of the mstar
lora.backend page (shrink, gather_shrink, expand_fused, apply_linear_,
apply_), plus build_addressing for the per-step addressing that, per that
page's module overview, the shrink and the expand both take from the pool.
"""
from __future__ import annotations

import ctypes
import os
from collections import namedtuple
from typing import Optional, Sequence

__all__ = [
    "Addressing", "LoraError", "lib", "lib_path", "build_addressing", "shrink",
    "gather_shrink", "expand_", "expand_fused", "apply_linear_", "apply_linear_from_slots_",
    "from_slots_one_launch", "apply_linear_from_experts_", "from_experts_one_launch", "apply_",
    "Backend",
    "workspace_bytes", "STATUS", "column_linear", "fused_column_linear",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "liblora_mi355x.so")
_LIB = None

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "alignment", 4: "workspace",
          5: "HIP launch failed", 6: "scratch limit"}

Addressing = namedtuple("Addressing", ["token_order", "slot_indptr"])

# symbol -> (restype, argtypes); mirrors include/lora_mi355x.h
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
SIGNATURES = {
    "lora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "lora_version": (ctypes.c_char_p, []),
    "lora_build_addressing": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _P, _SZ, _P]),
    "lora_build_addressing_workspace_bytes": (_SZ, [_I64, _I32]),
    "lora_build_addressing_experts": (ctypes.c_int, [_P, _P, _I32, _I64, _I32, _P, _P, _P, _SZ,
                                                     _P]),
    "lora_build_addressing_experts_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "lora_shrink": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _P, _I32, _I32, _I32, _P, _P,
                                   _P, _P, _P, _SZ, _P]),
    "lora_shrink_workspace_bytes": (_SZ, [_I64, _I64, _I32, _I32]),
    "lora_gather_shrink": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _P, _I32, _I32, _P, _P,
                                          _P, _P, _P]),
    "lora_expand": (ctypes.c_int, [ctypes.c_int, _P, _I64, _P, _I32, _P, _P, _I32, _I32, _P, _P,
                                   _P, _P, _P]),
    "lora_apply_linear": (ctypes.c_int, [ctypes.c_int, _P, _P, _I64, _I64, _P, _I32, _P, _P,
                                         _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "lora_apply_linear_workspace_bytes": (_SZ, [_I64, _I64, _I32, _I32, _I32]),
    "lora_apply_linear_path": (ctypes.c_int, [ctypes.c_int, _I64, _I64, _P, _I32, _I32]),
    "lora_apply_linear_from_slots": (ctypes.c_int, [ctypes.c_int, _P, _P, _I64, _I64, _P, _I32,
                                                    _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                                    _SZ, _P]),
    "lora_apply_linear_from_slots_workspace_bytes": (_SZ, [_I64, _I64, _I32, _I32, _I32]),
    "lora_apply_linear_from_slots_one_launch": (ctypes.c_int, [ctypes.c_int, _I64, _I64, _P, _I32,
                                                               _I32, _I32]),
    "lora_apply_linear_from_experts": (ctypes.c_int, [ctypes.c_int, _P, _P, _I64, _I64, _P, _I32,
                                                      _P, _P, _I32, _I32, _I32, _P, _P, _P, _P,
                                                      _P, _P, _P, _SZ, _P]),
    "lora_apply_linear_from_experts_workspace_bytes": (_SZ, [_I64, _I64, _I32, _I32, _I32,
                                                             _I32]),
    "lora_apply_linear_from_experts_one_launch": (ctypes.c_int, [ctypes.c_int, _I64, _I64, _P,
                                                                 _I32, _I32, _I32, _I32]),
    "lora_apply_linear_noalloc": (ctypes.c_int, [ctypes.c_int, _P, _P, _I64, _I64, _P, _I32, _P,
                                                 _P, _I32, _I32, _P, _P, _P, _P, _P]),
    "lora_noalloc_scratch_bytes": (_SZ, []),
    "lora_column_linear": (ctypes.c_int, [ctypes.c_int, _P, _P, _P, _I64, _I64, _P, _I32, _P]),
    "lora_fused_column_linear": (ctypes.c_int, [ctypes.c_int, _P, _P, _P, _I64, _I64, _P, _I32,
                                                _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "lora_fused_column_linear_workspace_bytes": (_SZ, [_I64, _I64, _I32, _I32]),
}


class LoraError(RuntimeError):
    pass


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load the HIP library (after torch, so both use the same HIP runtime)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH):
            raise LoraError(f"{_LIB_PATH} is not built: run `python -m adapter_lora_serving_amd.build`"
                            " (the LoRA delta has no CPU or PyTorch fallback)")
        import torch  # noqa: F401  (loads torch's libamdhip64 first)
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int, what: str):
    if status != 0:
        msg = lib().lora_status_string(status).decode()
        raise LoraError(f"{what}: {msg} (status {status})")


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return 1
    if t.dtype == torch.float32:
        return 0
    raise LoraError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _dev(*tensors):
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise LoraError("all tensors must be on the GPU (no CPU fallback)")
        if not t.is_contiguous():
            raise LoraError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise LoraError("tensors on different devices")
    return dev


def _stream(dev) -> int:
    import torch
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _i32(t):
    import torch
    return t if t.dtype == torch.int32 else t.to(torch.int32)


def _addr(addressing):
    if isinstance(addressing, Addressing):
        return addressing.token_order, addressing.slot_indptr
    return addressing[0], addressing[1]


def build_addressing(token_slot, slots: int, out: Optional[Addressing] = None) -> Addressing:
    """Group a step's tokens by adapter slot on the device (no host sync)."""
    import torch
    token_slot = _i32(token_slot)
    dev = _dev(token_slot)
    T = token_slot.numel()
    if out is None:
        out = Addressing(torch.empty(T, dtype=torch.int32, device=dev),
                         torch.empty(slots + 1, dtype=torch.int32, device=dev))
    _dev(token_slot, *out)
    # the two-pass sort of a large batch takes a workspace (torch's caching
    # allocator; no initialisation needed)
    nws = int(lib().lora_build_addressing_workspace_bytes(T, slots))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    st = lib().lora_build_addressing(_ptr(token_slot), T, slots, _ptr(out.token_order),
                                     _ptr(out.slot_indptr), _ptr(ws), nws, _stream(dev))
    _check(st, "lora_build_addressing")
    return out


def build_addressing_experts(row_slot, expert_offsets, num_experts: int, slots: int,
                             out: Optional[Addressing] = None) -> Addressing:
    """Group the rows of an expert-sorted batch by (expert, slot) on the
    device; virtual slot k = expert * slots + slot (num_experts * slots of
    them)."""
    import torch
    row_slot = _i32(row_slot)
    expert_offsets = _i32(expert_offsets)
    dev = _dev(row_slot, expert_offsets)
    rows = row_slot.numel()
    if expert_offsets.numel() != num_experts + 1:
        raise LoraError("expert_offsets must hold num_experts + 1 entries")
    if out is None:
        out = Addressing(torch.empty(rows, dtype=torch.int32, device=dev),
                         torch.empty(num_experts * slots + 1, dtype=torch.int32, device=dev))
    _dev(row_slot, *out)
    nws = int(lib().lora_build_addressing_experts_workspace_bytes(rows, num_experts, slots))
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    st = lib().lora_build_addressing_experts(_ptr(row_slot), _ptr(expert_offsets), num_experts,
                                             rows, slots, _ptr(out.token_order),
                                             _ptr(out.slot_indptr), _ptr(ws), ws.numel(),
                                             _stream(dev))
    _check(st, "lora_build_addressing_experts")
    return out


def shrink(x, a, addressing, ranks, num_slices: int = 1, out=None):
    """h[t] = x[t] @ a[slot(t)]^T (float32 [T, num_slices*R])."""
    import torch
    order, indptr = _addr(addressing)
    ranks = _i32(ranks)
    dev = _dev(x, a, order, indptr, ranks)
    T, in_f = x.shape
    slots, SR, in_a = a.shape
    if in_a != in_f or SR % num_slices or a.dtype != x.dtype:
        raise LoraError("shape/dtype mismatch between x and a")
    R = SR // num_slices
    if out is None:
        out = torch.empty(T, SR, dtype=torch.float32, device=dev)
    # K-part workspace for long segments (from torch's caching allocator;
    # its contents need no initialisation)
    nws = int(lib().lora_shrink_workspace_bytes(T, in_f, num_slices, R))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    st = lib().lora_shrink(_dtype_code(x), _ptr(x), T, in_f, _ptr(a), slots, num_slices, R,
                           _ptr(order), _ptr(indptr), _ptr(ranks), _ptr(out),
                           _ptr(ws), nws, _stream(dev))
    _check(st, "lora_shrink")
    return out


def gather_shrink(ids, a, addressing, ranks, out=None):
    """h[t] = a[slot(t)][:, ids[t]] (float32 [T, R]); invalid ids give 0."""
    import torch
    order, indptr = _addr(addressing)
    ids = _i32(ids)
    ranks = _i32(ranks)
    dev = _dev(ids, a, order, indptr, ranks)
    T = ids.numel()
    slots, R, vocab = a.shape
    if out is None:
        out = torch.empty(T, R, dtype=torch.float32, device=dev)
    st = lib().lora_gather_shrink(_dtype_code(a), _ptr(ids), T, vocab, _ptr(a), slots, R,
                                  _ptr(order), _ptr(indptr), _ptr(ranks), _ptr(out), _stream(dev))
    _check(st, "lora_gather_shrink")
    return out


def _slices(out_slices: Sequence[int]):
    arr = (ctypes.c_int64 * len(out_slices))(*[int(w) for w in out_slices])
    return arr, len(out_slices)


def expand_(h, b, addressing, ranks, scalings, y, out_slices: Sequence[int]) -> None:
    """Add each token's LoRA delta into y in place: for every fused output
    slice i, the slot's scaling times the token's slice-i h columns (below
    the slot's rank) against the slot's B rows of that slice."""
    order, indptr = _addr(addressing)
    ranks = _i32(ranks)
    dev = _dev(h, b, order, indptr, ranks, scalings, y)
    T = y.shape[0]
    slots, out, R = b.shape
    if sum(out_slices) != out or y.shape[1] != out or b.dtype != y.dtype:
        raise LoraError("shape/dtype mismatch between y, b and out_slices")
    arr, S = _slices(out_slices)
    st = lib().lora_expand(_dtype_code(y), _ptr(y), T, ctypes.cast(arr, _P), S, _ptr(h), _ptr(b),
                           slots, R, _ptr(order), _ptr(indptr), _ptr(ranks), _ptr(scalings),
                           _stream(dev))
    _check(st, "lora_expand")


expand_fused = expand_

_WS = {}
_WS_RETIRED = []


def workspace_bytes(T: int, in_features: int, slots: int, num_slices: int, R: int) -> int:
    return int(lib().lora_apply_linear_workspace_bytes(T, in_features, slots, num_slices, R))


def _workspace(dev, nbytes: int):
    """The workspace lora_apply_linear gets when the caller passes none: one
    zero-filled buffer per (device, stream), reused from call to call (every
    completed call leaves the synchronisation counters at its start in a
    state the next call accepts, so no clearing is needed).

    A graph captured on a stream keeps the address of the workspace it was
    captured with. When a later call needs a larger one, the old buffer is
    kept alive (never freed while the process runs), so a graph that still
    uses it stays valid. Calls that share one workspace must not run at the
    same time: graphs captured on one stream and replayed concurrently on
    other streams should each be given a workspace of their own."""
    import torch
    key = (str(dev), torch.cuda.current_stream(dev).cuda_stream)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _WS_RETIRED.append(ws)
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _WS[key] = ws
    return ws


def apply_linear_(x, y, a, b, addressing, ranks, scalings, out_slices: Sequence[int],
                  workspace=None) -> None:
    """Shrink then expand into y for a linear target (fused where the library fuses)."""
    order, indptr = _addr(addressing)
    ranks = _i32(ranks)
    dev = _dev(x, y, a, b, order, indptr, ranks, scalings)
    T, in_f = x.shape
    slots, out, R = b.shape
    S = len(out_slices)
    if a.shape != (slots, S * R, in_f) or y.shape != (T, out) or sum(out_slices) != out:
        raise LoraError("shape mismatch in apply_linear_")
    need = workspace_bytes(T, in_f, slots, S, R)
    ws = _workspace(dev, need) if workspace is None else workspace
    arr, S = _slices(out_slices)
    st = lib().lora_apply_linear(_dtype_code(x), _ptr(x), _ptr(y), T, in_f, ctypes.cast(arr, _P), S,
                                 _ptr(a), _ptr(b), slots, R, _ptr(order), _ptr(indptr), _ptr(ranks),
                                 _ptr(scalings), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(dev))
    _check(st, "lora_apply_linear")


def apply_linear_from_slots_(x, y, a, b, token_slot, ranks, scalings, out_slices: Sequence[int],
                             out: Optional[Addressing] = None, workspace=None) -> Addressing:
    """Build the step's addressing from token_slot and apply a linear
    target's delta into y in the same call (one kernel launch for a small
    bf16 batch); returns the addressing for the step's later targets."""
    import torch
    token_slot = _i32(token_slot)
    ranks = _i32(ranks)
    dev = _dev(x, y, a, b, token_slot, ranks, scalings)
    T, in_f = x.shape
    slots, outw, R = b.shape
    S = len(out_slices)
    if (a.shape != (slots, S * R, in_f) or y.shape != (T, outw) or sum(out_slices) != outw
            or token_slot.numel() != T):
        raise LoraError("shape mismatch in apply_linear_from_slots_")
    if out is None:
        out = Addressing(torch.empty(T, dtype=torch.int32, device=dev),
                         torch.empty(slots + 1, dtype=torch.int32, device=dev))
    order, indptr = _addr(out)
    _dev(x, order, indptr)
    if (order.dtype != torch.int32 or indptr.dtype != torch.int32 or order.numel() != T
            or indptr.numel() != slots + 1):
        raise LoraError("the addressing to write must be int32 [T] and [slots + 1]")
    need = int(lib().lora_apply_linear_from_slots_workspace_bytes(T, in_f, slots, S, R))
    ws = _workspace(dev, need) if workspace is None else workspace
    arr, S = _slices(out_slices)
    st = lib().lora_apply_linear_from_slots(
        _dtype_code(x), _ptr(x), _ptr(y), T, in_f, ctypes.cast(arr, _P), S, _ptr(a), _ptr(b),
        slots, R, _ptr(token_slot), _ptr(order), _ptr(indptr), _ptr(ranks), _ptr(scalings),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    _check(st, "lora_apply_linear_from_slots")
    return out


def apply_linear_from_experts_(x, y, a, b, row_slot, expert_offsets, num_experts: int,
                               slots: int, ranks, scalings, out_slices: Sequence[int],
                               out: Optional[Addressing] = None, workspace=None) -> Addressing:
    """Build the expert addressing of an expert-sorted batch and apply a
    routed-expert target's delta into y in the same call (one kernel launch
    for a small bf16 batch); a, b, ranks and scalings are per pool entry
    expert * slots + slot. Returns the addressing for the step's later
    targets."""
    import torch
    row_slot = _i32(row_slot)
    expert_offsets = _i32(expert_offsets)
    ranks = _i32(ranks)
    dev = _dev(x, y, a, b, row_slot, expert_offsets, ranks, scalings)
    rows, in_f = x.shape
    K, outw, R = b.shape
    S = len(out_slices)
    if (K != num_experts * slots or a.shape != (K, S * R, in_f) or y.shape != (rows, outw)
            or sum(out_slices) != outw or row_slot.numel() != rows
            or expert_offsets.numel() != num_experts + 1):
        raise LoraError("shape mismatch in apply_linear_from_experts_")
    if out is None:
        out = Addressing(torch.empty(rows, dtype=torch.int32, device=dev),
                         torch.empty(K + 1, dtype=torch.int32, device=dev))
    order, indptr = _addr(out)
    _dev(x, order, indptr)
    if (order.dtype != torch.int32 or indptr.dtype != torch.int32 or order.numel() != rows
            or indptr.numel() != K + 1):
        raise LoraError("the addressing to write must be int32 [rows] and [experts * slots + 1]")
    need = int(lib().lora_apply_linear_from_experts_workspace_bytes(rows, in_f, num_experts,
                                                                     slots, S, R))
    ws = _workspace(dev, need) if workspace is None else workspace
    arr, S = _slices(out_slices)
    st = lib().lora_apply_linear_from_experts(
        _dtype_code(x), _ptr(x), _ptr(y), rows, in_f, ctypes.cast(arr, _P), S, _ptr(a), _ptr(b),
        num_experts, slots, R, _ptr(row_slot), _ptr(expert_offsets), _ptr(order), _ptr(indptr),
        _ptr(ranks), _ptr(scalings), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    _check(st, "lora_apply_linear_from_experts")
    return out


def from_experts_one_launch(dtype_code: int, rows: int, in_features: int,
                            out_slices: Sequence[int], num_experts: int, slots: int,
                            R: int) -> bool:
    """Whether apply_linear_from_experts_ is one kernel launch for these sizes."""
    arr, S = _slices(out_slices)
    r = int(lib().lora_apply_linear_from_experts_one_launch(dtype_code, rows, in_features,
                                                            ctypes.cast(arr, _P), S, num_experts,
                                                            slots, R))
    if r < 0:
        _check(-r, "lora_apply_linear_from_experts_one_launch")
    return r == 1


def from_slots_one_launch(dtype_code: int, T: int, in_features: int, out_slices: Sequence[int],
                          slots: int, R: int) -> bool:
    """Whether apply_linear_from_slots_ is one kernel launch for these sizes."""
    arr, S = _slices(out_slices)
    r = int(lib().lora_apply_linear_from_slots_one_launch(dtype_code, T, in_features,
                                                          ctypes.cast(arr, _P), S, slots, R))
    if r < 0:
        _check(-r, "lora_apply_linear_from_slots_one_launch")
    return r == 1


def apply_(x, y, a, b, addressing, ranks, scalings, out_slices: Sequence[int],
           embedding: bool = False):
    """Shrink (a gather for an embedding target, whose x is token ids) then
    expand into y; returns y."""
    if embedding:
        h = gather_shrink(x, a, addressing, ranks)
        expand_(h, b, addressing, ranks, scalings, y, out_slices)
    else:
        apply_linear_(x, y, a, b, addressing, ranks, scalings, out_slices)
    return y


def column_linear(x, w, out_slices: Sequence[int], y=None):
    """The base projection of a fused column linear layer, y = x @ W^T
    (W [out, in]: the shards stacked along the output dimension)."""
    import torch
    dev = _dev(x, w, y)
    T, in_f = x.shape
    out = int(sum(out_slices))
    if w.shape != (out, in_f) or x.dtype != w.dtype:
        raise LoraError("shape/dtype mismatch between x, w and out_slices")
    if y is None:
        y = torch.empty(T, out, dtype=x.dtype, device=dev)
    arr, S = _slices(out_slices)
    st = lib().lora_column_linear(_dtype_code(x), _ptr(x), _ptr(w), _ptr(y), T, in_f,
                                  ctypes.cast(arr, _P), S, _stream(dev))
    _check(st, "lora_column_linear")
    return y


def fused_column_linear(x, w, a, b, addressing, ranks, scalings, out_slices: Sequence[int],
                        y=None, workspace=None):
    """The base projection x @ W^T with each token's LoRA delta added in the
    product's epilogue (y written once); returns y."""
    import torch
    order, indptr = _addr(addressing)
    ranks = _i32(ranks)
    dev = _dev(x, w, a, b, order, indptr, ranks, scalings, y)
    T, in_f = x.shape
    slots, out, R = b.shape
    S = len(out_slices)
    if w.shape != (out, in_f) or a.shape != (slots, S * R, in_f) or sum(out_slices) != out:
        raise LoraError("shape mismatch in fused_column_linear")
    if y is None:
        y = torch.empty(T, out, dtype=x.dtype, device=dev)
    need = int(lib().lora_fused_column_linear_workspace_bytes(T, in_f, S, R))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    arr, S = _slices(out_slices)
    st = lib().lora_fused_column_linear(
        _dtype_code(x), _ptr(x), _ptr(w), _ptr(y), T, in_f, ctypes.cast(arr, _P), S, _ptr(a),
        _ptr(b), slots, R, _ptr(order), _ptr(indptr), _ptr(ranks), _ptr(scalings),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st, "lora_fused_column_linear")
    return y


class Backend:
    """The LoraBackend method surface of the lora.backend page, on MI355X."""

    def shrink(self, x, a, addressing, ranks, num_slices: int = 1):
        return shrink(x, a, addressing, ranks, num_slices)

    def gather_shrink(self, ids, a, addressing, ranks):
        return gather_shrink(ids, a, addressing, ranks)

    def expand_fused(self, h, b, addressing, ranks, scalings, y, out_slices):
        expand_(h, b, addressing, ranks, scalings, y, out_slices)

    def apply_linear_(self, x, y, a, b, addressing, ranks, scalings, out_slices):
        apply_linear_(x, y, a, b, addressing, ranks, scalings, out_slices)

    def apply_(self, x, y, a, b, addressing, ranks, scalings, out_slices, embedding=False):
        return apply_(x, y, a, b, addressing, ranks, scalings, out_slices, embedding)
