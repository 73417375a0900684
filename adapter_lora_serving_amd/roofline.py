"""Algorithmic bytes and flops of one LoRA-delta call, for roofline reporting.

The byte count is what the method must move at minimum, not what a kernel
happens to move:
  * x rows of the tokens that are adapted (live, rank > 0): e*|L|*in
    (embedding target: the ids, 4*T);
  * A rows below the rank of every used slot, once: sum_s e*S*r_s*in
    (embedding target: the gathered elements, e*sum_{t in L} r_slot(t));
  * B columns below the rank of every used slot, once: sum_s e*out*r_s;
  * y read and written for every adapted token: 2*e*|L|*out;
  * the addressing and per-slot metadata: 4*T + 4*(slots+1) + 8*slots.
The intermediate h is excluded (it does not exist in the fused path).
flops = sum over adapted tokens of 2*r*(S*in + out) (embedding: 2*r*out).
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 matrix peak, vendor figure
FP32_VALU_PEAK_TFLOPS = 157.3   # fp32 vector peak (packed), vendor figure


def _ranks(ranks, R):
    return np.clip(np.asarray(ranks, dtype=np.int64), 0, R)


def lora_call_cost(T: int, in_features: int, out_slices: Sequence[int], R: int, slots: int,
                   ranks, token_slot, elem_bytes: int, embedding: bool = False,
                   ids: Optional[np.ndarray] = None) -> Tuple[int, int, Dict[str, int]]:
    """(bytes, flops, per-term bytes) of one call on one target."""
    S = len(out_slices)
    out = int(sum(out_slices))
    e = int(elem_bytes)
    r = _ranks(ranks, R)
    ts = np.asarray(token_slot, dtype=np.int64)
    live = (ts >= 0) & (ts < slots)
    rt = np.zeros(len(ts), dtype=np.int64)
    rt[live] = r[ts[live]]
    adapted = rt > 0
    if embedding:
        idv = np.asarray(ids, dtype=np.int64)
        adapted_y = adapted & (idv >= 0) & (idv < in_features)
    else:
        adapted_y = adapted
    used = np.unique(ts[adapted_y])
    terms = {}
    if embedding:
        terms["x"] = 4 * int(T)
        terms["a"] = e * int(rt[adapted_y].sum())
    else:
        terms["x"] = e * int(adapted.sum()) * int(in_features)
        terms["a"] = sum(e * S * int(r[s]) * int(in_features) for s in used)
    terms["b"] = sum(e * out * int(r[s]) for s in used)
    terms["y"] = 2 * e * int(adapted_y.sum()) * out
    terms["meta"] = 4 * int(T) + 4 * (int(slots) + 1) + 8 * int(slots)
    total = int(sum(terms.values()))
    if embedding:
        flops = int(2 * rt[adapted_y].sum() * out)
    else:
        flops = int(2 * rt[adapted].sum() * (S * int(in_features) + out))
    return total, flops, terms


def expert_row_slots(row_slot, expert_offsets, slots: int) -> np.ndarray:
    """Pool entry of every row of an expert-sorted batch, for the byte model:
    expert e owns rows [offsets[e], offsets[e+1]) and a row of slot s uses
    entry e * slots + s; rows outside the expert ranges or with a slot outside
    [0, slots) use none (-1)."""
    rs = np.asarray(row_slot, dtype=np.int64)
    offs = np.asarray(expert_offsets, dtype=np.int64)
    r = np.arange(len(rs))
    e = np.searchsorted(offs, r, side="right") - 1
    live = (r >= offs[0]) & (r < offs[-1]) & (rs >= 0) & (rs < slots)
    return np.where(live, e * slots + rs, -1)


def workload_cost(wl, tg) -> Tuple[int, int, Dict[str, int]]:
    """Cost of one target of a `workloads.Workload` (an expert-sorted batch
    takes each row's pool entry from its routing)."""
    e = 2 if wl.dtype == "bf16" else 4
    ts = wl.token_slot
    ex = getattr(wl, "experts", None)
    if ts is None and ex is not None:
        ts = expert_row_slots(ex["row_slot"], ex["offsets"], ex["slots"])
    return lora_call_cost(wl.T, tg.in_features, tg.out_slices, wl.R, wl.slots, wl.ranks,
                          ts, e, embedding=tg.embedding, ids=tg.ids)
