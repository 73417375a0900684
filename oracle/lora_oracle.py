"""CPU oracle for the batched multi-LoRA delta.

TEST INFRASTRUCTURE ONLY. Only the tests, the package entry's smoke check and
the benchmark's CPU-baseline leg may import or call this module. The product
path (the HIP library and its Python binding) never does, and this module
imports nothing from it: the two share no code. Inputs come from the seeded
generators in `workloads`, which hold none of the method's arithmetic.

Everything is evaluated in float64 on the exact input values (bf16 bit
patterns are decoded exactly; fp32 inputs are taken as given). The method
reaches the plain definition exactly (no approximation, no iteration), so the
oracle *is* that definition, written with explicit loops over slots and
slices; inside a loop the only library primitive is a float64 matrix product.

Sources (page title, section):
  * mstar.engine.resources.lora.backend, module overview: the shapes
    x [T, in], y [T, out], h [T, slices*R], a [slots, slices*R, in],
    b [slots, out, R], ranks / scalings [slots]; slice i reads
    h[:, i*R:(i+1)*R] and writes its own columns of y; an embedding target's
    shrink is a gather of A's column for the token id.
  * same page, LoraBackend.shrink: h[t] = x[t] @ a[slot(t)]^T; rows of rank-0
    slots and columns past a slot's rank are not read by the expand.
  * same page, LoraBackend.gather_shrink: h[t] = a[slot(t)][:, ids[t]]; an id
    outside [0, in) contributes nothing.
  * same page, LoraBackend.expand_fused: y[t, slice i] +=
    scalings[slot(t)] * h[t, slice i] @ b[slot(t), slice i]^T, in place.
  * same page, LoraBackend.apply_ / apply_linear_: shrink (or gather) then
    expand.
  * same page, shrink_reference: every token against every slot, then its own
    selected; zeros where the expand does not read (dead tokens, columns past
    a slot's rank).
  * mstar.model.components.linear, FusedColumnLinear: shards of a fused
    output sit along the output dimension in iteration order, so slice i
    starts at the sum of the widths before it.

Readings where the pages are silent (each is listed with its reason in the
design notes): a token is dead when its slot is outside [0, slots); ranks are
clamped to [0, R]; the addressing is a stable grouping by slot with dead
tokens appended in ascending order; entries of h the expand never reads are
zero.

Parity status: every function here is pinned by CPU tests against closed
forms, brute force, special cases and invariants (tests/test_oracle_pins.py);
none is "parity unpinned".
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# exact decoding of the input encodings
# ---------------------------------------------------------------------------

def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of an input array. bf16 arrives as uint16 bits: a
    bf16 number is the upper half of the fp32 with the same bits."""
    if dtype == "bf16":
        bits = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def _rank(ranks: np.ndarray, s: int, R: int) -> int:
    return int(min(max(int(ranks[s]), 0), R))


def _live(slot: int, slots: int) -> bool:
    return 0 <= slot < slots


# ---------------------------------------------------------------------------
# addressing: token_order / slot_indptr
# (lora.backend, module overview: the shrink and the expand both take the
#  per-step addressing from the adapter pool; shrink_reference and
#  expand_reference_ take token_order and slot_indptr)
# ---------------------------------------------------------------------------

def build_addressing(token_slot: Sequence[int], slots: int) -> Tuple[np.ndarray, np.ndarray]:
    """Group tokens by slot: a stable counting sort.

    slot_indptr[s]..slot_indptr[s+1] is the segment of token_order holding the
    tokens of slot s, in ascending token index. Dead tokens (slot outside
    [0, slots)) follow slot_indptr[slots], also ascending, so token_order is a
    permutation of [0, T)."""
    T = len(token_slot)
    key = [int(s) if _live(int(s), slots) else slots for s in token_slot]
    count = [0] * (slots + 1)
    for k in key:
        count[k] += 1
    start = [0] * (slots + 2)
    for k in range(slots + 1):
        start[k + 1] = start[k] + count[k]
    cursor = start[: slots + 1]
    order = [0] * T
    for t in range(T):
        order[cursor[key[t]]] = t
        cursor[key[t]] += 1
    return np.asarray(order, dtype=np.int32), np.asarray(start[: slots + 1], dtype=np.int32)


def expert_keys(row_slot: Sequence[int], expert_offsets: Sequence[int], num_experts: int,
                slots: int) -> np.ndarray:
    """Composite key of each row of an expert-sorted batch (page
    "spark_model/lora/expert_apply.rs", the experts injection shape: rows of
    the grouped GEMM sorted by expert, each with its token's slot): expert e
    holds rows [offsets[e], offsets[e+1]); key = e * slots + slot, or -1 for
    a dead row (slot outside [0, slots), or no expert)."""
    keys = np.full(len(row_slot), -1, dtype=np.int64)
    for e in range(num_experts):
        for r in range(int(expert_offsets[e]), int(expert_offsets[e + 1])):
            if 0 <= r < len(row_slot) and _live(int(row_slot[r]), slots):
                keys[r] = e * slots + int(row_slot[r])
    return keys


def build_addressing_experts(row_slot: Sequence[int], expert_offsets: Sequence[int],
                             num_experts: int, slots: int) -> Tuple[np.ndarray, np.ndarray]:
    """The addressing of those rows over num_experts * slots virtual slots:
    the stable counting sort of build_addressing on the composite keys."""
    return build_addressing(expert_keys(row_slot, expert_offsets, num_experts, slots),
                            num_experts * slots)


# ---------------------------------------------------------------------------
# shrink / gather_shrink / expand
# ---------------------------------------------------------------------------

def shrink(x: np.ndarray, a: np.ndarray, token_slot: np.ndarray, ranks: np.ndarray,
           num_slices: int, R: int) -> np.ndarray:
    """h[t, i*R + j] = x[t] . a[slot(t), i*R + j] for j < rank(slot(t)); every
    other entry is 0 (lora.backend, LoraBackend.shrink and shrink_reference).

    x: float64 [T, in]; a: float64 [slots, num_slices*R, in]."""
    T = x.shape[0]
    slots = a.shape[0]
    h = np.zeros((T, num_slices * R), dtype=np.float64)
    for s in range(slots):
        r = _rank(ranks, s, R)
        toks = np.nonzero(token_slot == s)[0]
        if r == 0 or len(toks) == 0:
            continue
        for i in range(num_slices):
            rows = a[s, i * R: i * R + r, :]          # [r, in]
            h[toks, i * R: i * R + r] = x[toks] @ rows.T
    return h


def gather_shrink(ids: np.ndarray, a: np.ndarray, token_slot: np.ndarray,
                  ranks: np.ndarray, R: int) -> np.ndarray:
    """h[t, j] = a[slot(t), j, ids[t]] for j < rank(slot(t)) and a valid id;
    0 otherwise (lora.backend, LoraBackend.gather_shrink). An embedding has a
    single output, so there is one slice."""
    T = len(ids)
    slots, _, vocab = a.shape
    h = np.zeros((T, R), dtype=np.float64)
    for t in range(T):
        s = int(token_slot[t])
        if not _live(s, slots):
            continue
        v = int(ids[t])
        if not (0 <= v < vocab):
            continue
        r = _rank(ranks, s, R)
        h[t, :r] = a[s, :r, v]
    return h


def expand(y0: np.ndarray, h: np.ndarray, b: np.ndarray, token_slot: np.ndarray,
           ranks: np.ndarray, scalings: np.ndarray, out_slices: Sequence[int],
           R: int) -> np.ndarray:
    """y[t, off_i + o] = y0[t, off_i + o] + scaling(slot(t)) *
    sum_{j < r} h[t, i*R + j] * b[slot(t), off_i + o, j]; rows of dead tokens
    and of rank-0 slots are returned unchanged (lora.backend,
    LoraBackend.expand_fused and expand_reference_; slice offsets from
    FusedColumnLinear's shard layout).

    Only columns j < r of h and b are touched."""
    y = np.array(y0, dtype=np.float64, copy=True)
    slots = b.shape[0]
    off = 0
    for i, w in enumerate(out_slices):
        w = int(w)
        for s in range(slots):
            r = _rank(ranks, s, R)
            toks = np.nonzero(token_slot == s)[0]
            if r == 0 or len(toks) == 0:
                continue
            hs = h[toks, i * R: i * R + r]            # [n, r]
            bs = b[s, off: off + w, :r]               # [w, r]
            y[np.ix_(toks, np.arange(off, off + w))] += float(scalings[s]) * (hs @ bs.T)
        off += w
    return y


def base_projection(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """The base layer's own output, y[t, o] = sum_c x[t, c] * w[o, c]: one
    product over the fused weight, whose shards (q, k, v or gate, up) are
    stacked along the output dimension in order (mstar.model.components.linear,
    FusedColumnLinear.forward). The LoRA delta is then added on top of it
    (expand, with this as y0), as when the expand runs inside the base
    projection's epilogue.

    x: float64 [T, in]; w: float64 [out, in]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


# ---------------------------------------------------------------------------
# second formulation: the pages' capture-safe reference
# ---------------------------------------------------------------------------

def shrink_all_slots(x: np.ndarray, a: np.ndarray, token_slot: np.ndarray,
                     ranks: np.ndarray, num_slices: int, R: int) -> np.ndarray:
    """shrink_reference's formulation (lora.backend, shrink_reference): every
    token against every slot, then each token's own slot selected, with zeros
    at dead tokens and past each slot's rank."""
    T = x.shape[0]
    slots = a.shape[0]
    full = np.einsum("tc,src->tsr", x, a)             # [T, slots, S*R]
    keep = np.zeros((slots, num_slices * R), dtype=bool)
    for s in range(slots):
        r = _rank(ranks, s, R)
        for i in range(num_slices):
            keep[s, i * R: i * R + r] = True
    h = np.zeros((T, num_slices * R), dtype=np.float64)
    for t in range(T):
        s = int(token_slot[t])
        if _live(s, slots):
            h[t] = np.where(keep[s], full[t, s], 0.0)
    return h


# ---------------------------------------------------------------------------
# brute force: scalar loops, for tiny sizes only
# ---------------------------------------------------------------------------

def apply_scalar(inp, y0, a, b, token_slot, ranks, scalings, out_slices, R,
                 embedding=False):
    """The whole delta as nested scalar Python loops (no array arithmetic)."""
    T = len(token_slot)
    slots = a.shape[0]
    y = [[float(v) for v in row] for row in np.asarray(y0, dtype=np.float64)]
    for t in range(T):
        s = int(token_slot[t])
        if not _live(s, slots):
            continue
        r = _rank(ranks, s, R)
        scale = float(scalings[s])
        off = 0
        for i, w in enumerate(out_slices):
            hrow = [0.0] * r
            for j in range(r):
                if embedding:
                    v = int(inp[t])
                    hrow[j] = float(a[s, j, v]) if 0 <= v < a.shape[2] else 0.0
                else:
                    acc = 0.0
                    for c in range(a.shape[2]):
                        acc += float(inp[t, c]) * float(a[s, i * R + j, c])
                    hrow[j] = acc
            for o in range(int(w)):
                acc = 0.0
                for j in range(r):
                    acc += hrow[j] * float(b[s, off + o, j])
                y[t][off + o] += scale * acc
            off += int(w)
    return np.asarray(y, dtype=np.float64)


# ---------------------------------------------------------------------------
# workload-level helpers (decoding + apply on a `workloads.Workload`)
# ---------------------------------------------------------------------------

def run_target(wl, tg) -> Tuple[np.ndarray, np.ndarray]:
    """(h, y) of one target of a generated workload, in float64."""
    a = decode(tg.a, wl.dtype)
    b = decode(tg.b, wl.dtype)
    y0 = decode(tg.y0, wl.dtype)
    if tg.embedding:
        h = gather_shrink(tg.ids, a, wl.token_slot, wl.ranks, wl.R)
    else:
        h = shrink(decode(tg.x, wl.dtype), a, wl.token_slot, wl.ranks, tg.num_slices, wl.R)
    y = expand(y0, h, b, wl.token_slot, wl.ranks, wl.scalings, tg.out_slices, wl.R)
    return h, y


def within_tolerance(gpu: np.ndarray, ref: np.ndarray, atol: float = 1e-2,
                     rtol: float = 1e-2) -> Tuple[bool, float]:
    """Graded bound |gpu - ref| <= atol + rtol*|ref|; returns (ok, max err/bound)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = atol + rtol * np.abs(ref)
    ratio = np.abs(gpu - ref) / bound
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    ok = bool(np.all(np.isfinite(gpu)) and np.all(ratio <= 1.0))
    return ok, worst
