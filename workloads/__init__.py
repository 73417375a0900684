"""Seeded synthetic inputs for the batched multi-LoRA delta.

This module only draws inputs. It holds none of the method's arithmetic (no
shrink, gather, expand or addressing): the CPU oracle and the HIP path both
take their inputs from here and share nothing else.

Shapes follow the layouts on the mstar.engine.resources.lora.backend page
(module overview): x [T, in], y [T, out], a [slots, slices*R, in],
b [slots, out, R], ranks / scalings [slots]. For an embedding target x is
replaced by token ids and `in` is the vocabulary.

bf16 tensors are carried as uint16 bit patterns (numpy has no bf16); the
rounding from the fp32 draws is round-to-nearest-even. fp32 tensors are
float32 arrays. Draw order inside one workload is fixed: ranks, scalings,
token->slot, ids, then per target x, A, B, y0.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

__all__ = [
    "Target", "Workload", "f32_to_bf16_bits", "make_workload", "make_config",
    "CONFIG_NAMES", "poison_unread", "zipf_request_lengths", "permute_tokens",
    "take_tokens", "with_token_slot", "base_weight", "make_moe_experts", "make_router_fold", "make_tp_share",
]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return the bits.

    Inputs here are finite Gaussians; NaN/inf are not produced by the draws
    (poison NaNs are written as bit patterns directly)."""
    u = np.ascontiguousarray(a, dtype=np.float32).reshape(-1).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    step = 1 << 24
    for k in range(0, u.size, step):
        c = u[k:k + step]
        # finite inputs: c + 0x8000 stays below 2^32, so uint32 does not wrap
        out[k:k + step] = ((c + np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1)))
                           >> np.uint32(16)).astype(np.uint16)
    return out.reshape(np.shape(a))


@dataclass
class Target:
    """One LoRA target (a projection) of a workload."""
    name: str
    in_features: int            # `in` (the vocabulary for an embedding target)
    out_slices: tuple           # widths of the fused outputs, in layout order
    a: np.ndarray               # [slots, S*R, in]   (uint16 bf16 bits or float32)
    b: np.ndarray               # [slots, out, R]
    y0: np.ndarray              # [T, out]           initial y (base projection stand-in)
    x: Optional[np.ndarray] = None    # [T, in] for a linear target
    ids: Optional[np.ndarray] = None  # [T] int32 for an embedding target

    @property
    def embedding(self) -> bool:
        return self.ids is not None

    @property
    def num_slices(self) -> int:
        return len(self.out_slices)

    @property
    def out_features(self) -> int:
        return int(sum(self.out_slices))


@dataclass
class Workload:
    name: str
    dtype: str                  # "f32" or "bf16": the dtype of x, a, b, y
    T: int
    R: int
    slots: int
    ranks: np.ndarray           # int32 [slots]
    scalings: np.ndarray        # float32 [slots]
    token_slot: Optional[np.ndarray]  # int32 [T]; outside [0, slots) means "no adapter"
    targets: List[Target] = field(default_factory=list)
    seed: int = 0

    def target(self, name: Optional[str] = None) -> Target:
        if name is None:
            return self.targets[0]
        for t in self.targets:
            if t.name == name:
                return t
        raise KeyError(name)


def _cast(vals: np.ndarray, dtype: str) -> np.ndarray:
    vals = vals.astype(np.float32, copy=False)
    if dtype == "bf16":
        return f32_to_bf16_bits(vals)
    if dtype == "f32":
        return vals
    raise ValueError(dtype)


def _gauss(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return _cast(v, dtype)


def zipf_request_lengths(n_requests: int, total: int, exponent: float) -> np.ndarray:
    """Rank-frequency Zipf lengths: w_i = i^-exponent normalised to `total`,
    floored with a minimum of 1, then largest remainders take the leftover."""
    w = np.arange(1, n_requests + 1, dtype=np.float64) ** (-exponent)
    raw = w / w.sum() * total
    lens = np.maximum(np.floor(raw).astype(np.int64), 1)
    left = int(total - lens.sum())
    if left > 0:
        order = np.argsort(-(raw - np.floor(raw)), kind="stable")
        lens[order[:left]] += 1
    elif left < 0:  # only possible when the minimum of 1 overshoots
        order = np.argsort(-lens, kind="stable")
        for k in order[: -left]:
            lens[k] -= 1
    return lens


def make_workload(*, name: str, dtype: str, T: int, in_features: int,
                  out_slices: Sequence[int], R: int, slots: int,
                  ranks: Sequence[int], scalings: Sequence[float],
                  token_slot: np.ndarray, seed: int, rng: np.random.Generator,
                  ids: Optional[np.ndarray] = None, x_std: float = 1.0,
                  a_std: Optional[float] = None, b_std: Optional[float] = None,
                  y0_zero: bool = False, target_name: str = "t0") -> Workload:
    """Draw x (unless ids are given), A, B and y0 for one target and wrap it."""
    wl = Workload(name=name, dtype=dtype, T=T, R=R, slots=slots,
                  ranks=np.asarray(ranks, dtype=np.int32),
                  scalings=np.asarray(scalings, dtype=np.float32),
                  token_slot=np.asarray(token_slot, dtype=np.int32), seed=seed)
    wl.targets.append(_draw_target(rng, target_name, dtype, T, in_features,
                                   tuple(int(w) for w in out_slices), R, slots,
                                   ids=ids, x_std=x_std, a_std=a_std, b_std=b_std,
                                   y0_zero=y0_zero))
    return wl


def _draw_target(rng, name, dtype, T, in_features, out_slices, R, slots, *,
                 ids=None, x_std=1.0, a_std=None, b_std=None, y0_zero=False) -> Target:
    S = len(out_slices)
    out = int(sum(out_slices))
    a_std = (1.0 / np.sqrt(in_features)) if a_std is None else a_std
    b_std = (1.0 / np.sqrt(R)) if b_std is None else b_std
    x = None
    if ids is None:
        x = _gauss(rng, (T, in_features), x_std, dtype)
    a = _gauss(rng, (slots, S * R, in_features), a_std, dtype)
    b = _gauss(rng, (slots, out, R), b_std, dtype)
    if y0_zero:
        y0 = _cast(np.zeros((T, out), np.float32), dtype)
    else:
        y0 = _gauss(rng, (T, out), 1.0, dtype)
    return Target(name=name, in_features=in_features, out_slices=out_slices,
                  a=a, b=b, y0=y0, x=x,
                  ids=None if ids is None else np.asarray(ids, dtype=np.int32))


CONFIG_NAMES = {
    1: "tiny_fp32",
    2: "decode_bgmv_bf16",
    3: "prefill_sgmv_bf16",
    4: "embedding_gather_bf16",
    5: "skewed_mix_bf16",
}


ROUTER_FOLD = "router_fold_bf16"


def make_router_fold(seed: int = 0, *, T: int = 256, hidden: int = 4096, num_experts: int = 64,
                     slots: int = 32, dtype: str = "bf16", y0_zero: bool = False) -> Workload:
    """A router LoRA folded onto the routing logits before top-k: one linear
    target with a single out slice of num_experts columns on the router
    input. The pages give no sizes; this takes the decode batch of the
    qkv workload (T=256 one-token requests over 32 slots, ranks 8 or 16,
    scaling 2.0, x, A, B Gaussian as there) with 64 experts."""
    rng = np.random.default_rng(seed)
    ranks = rng.choice(np.array([8, 16]), size=slots)
    scal = np.full(slots, 2.0, np.float32)
    tslot = rng.integers(0, slots, size=T, dtype=np.int64)
    return make_workload(name=ROUTER_FOLD if dtype == "bf16" else "router_fold_f32", dtype=dtype,
                         T=T, in_features=hidden, out_slices=(num_experts,), R=16, slots=slots,
                         ranks=ranks, scalings=scal, token_slot=tslot, seed=seed, rng=rng,
                         y0_zero=y0_zero, target_name="router")


MOE_EXPERTS = "moe_experts_bf16"


def make_moe_experts(seed: int = 0, *, T: int = 256, experts: int = 8, topk: int = 2,
                     hidden: int = 4096, inter: int = 14336, slots: int = 32,
                     y0_zero: bool = False) -> Workload:
    """The routed-expert LoRA on the rows of an expert-sorted grouped GEMM.

    Routing: each of T tokens goes to `topk` distinct experts drawn uniformly;
    the (token, expert) rows are laid out sorted by expert (stably, by
    token), as the base grouped GEMM holds them, and every row carries its
    token's adapter slot. `wl.experts` holds that routing: row_slot [rows],
    expert_offsets [experts + 1] (expert e owns rows [offsets[e],
    offsets[e+1])), and the number of experts and of base slots.

    Adapter pool: one LoRA per (expert, slot), stored at pool index
    expert * slots + slot (experts * slots entries: A, B, ranks, scalings);
    a slot's rank and scaling are the same for every expert. Which pool entry
    a row uses is left to the method (its addressing); `wl.token_slot` is
    None here.

    Targets: the expert gate/up projection (in = hidden, out slices (inter,
    inter)), whose delta goes in before the activation, and the expert down
    projection (in = inter, out = hidden), whose delta goes in after the down
    product. The pages give no sizes: an 8-expert, top-2 MoE with 4096
    hidden and 14336 intermediate, over the decode recipe's 256 tokens and 32
    slots (ranks 8 or 16, scaling 2)."""
    rng = np.random.default_rng(seed)
    base_ranks = rng.choice(np.array([8, 16]), size=slots)
    tok_slot = rng.integers(0, slots, size=T, dtype=np.int64)
    route = np.stack([rng.choice(experts, size=topk, replace=False) for _ in range(T)])
    tok = np.repeat(np.arange(T), topk)
    ex = route.reshape(-1)
    order = np.argsort(ex, kind="stable")
    tok, ex = tok[order], ex[order]
    offsets = np.concatenate([[0], np.cumsum(np.bincount(ex, minlength=experts))])
    row_slot = tok_slot[tok]
    rows = len(row_slot)
    vslots = experts * slots
    R = 16
    wl = Workload(name=MOE_EXPERTS, dtype="bf16", T=rows, R=R, slots=vslots,
                  ranks=np.tile(base_ranks, experts).astype(np.int32),
                  scalings=np.full(vslots, 2.0, np.float32), token_slot=None, seed=seed)
    wl.targets.append(_draw_target(rng, "expert_gate_up", "bf16", rows, hidden, (inter, inter),
                                   R, vslots, y0_zero=y0_zero))
    wl.targets.append(_draw_target(rng, "expert_down", "bf16", rows, inter, (hidden,), R,
                                   vslots, y0_zero=y0_zero))
    wl.experts = dict(experts=experts, slots=slots, row_slot=row_slot.astype(np.int32),
                      offsets=offsets.astype(np.int32))
    return wl


def base_weight(wl: Workload, tg: Target) -> np.ndarray:
    """The base projection's weight W [out, in] of a linear target (the
    shards of its out slices stacked in order), N(0, 1/in) so that x @ W^T is
    of unit scale like y0, in the workload's dtype. Drawn from a generator of
    its own, seeded by the workload's seed and the target's position, so the
    workload's other draws are the same with or without it."""
    idx = next(k for k, t in enumerate(wl.targets) if t is tg)
    rng = np.random.default_rng([int(wl.seed), 7919, idx])
    return _gauss(rng, (tg.out_features, tg.in_features), 1.0 / np.sqrt(tg.in_features),
                  wl.dtype)


def with_token_slot(wl: Workload, token_slot: np.ndarray) -> Workload:
    """The same workload with the given per-token slot array (for instance the
    pool index of every row of an expert-sorted batch, which the method's
    own addressing gives)."""
    out = dataclasses.replace(wl, targets=list(wl.targets),
                              token_slot=np.asarray(token_slot, dtype=np.int32))
    if hasattr(wl, "experts"):
        out.experts = wl.experts
    return out


TP_SHARES = ("tp8_qkv_decode", "tp8_prefill")


def make_tp_share(name: str, seed: int = 0) -> Workload:
    """One GPU's share of a tensor-parallel projection at TP = 8, at its real
    shape: column-parallel targets keep x and A whole and take an eighth of
    every out slice (B's rows); row-parallel targets take an eighth of `in`
    (x's columns and A's). tp8_qkv_decode: the qkv decode workload with out
    slices (512, 128, 128). tp8_prefill: the prefill workload with an
    intermediate width of 1792, so gate/up is the column share (1792, 1792)
    and down the row share (in 1792)."""
    if name == "tp8_qkv_decode":
        wl = make_config(2, seed, out_slices=(4096 // 8, 1024 // 8, 1024 // 8))
    elif name == "tp8_prefill":
        wl = make_config(3, seed, inter=14336 // 8)
    else:
        raise ValueError(f"unknown share {name}")
    wl.name = name + "_bf16"
    return wl


def make_config(k: int, seed: int = 0, *, y0_zero: bool = False, **over) -> Workload:
    """The five synthetic workloads of the hot path, seeded.

    `over` shrinks a config for fast tests (keys: T, in_features, out_slices,
    vocab, slots). The readings behind each recipe (Zipf lengths, request to
    slot draw, scalings where none are given) are listed in the design notes.
    """
    rng = np.random.default_rng(seed)
    if k == 1:
        T = over.get("T", 64)
        in_f = over.get("in_features", 256)
        ranks = [8, 4, 0, 8]
        scal = [16.0 / r if r else 0.0 for r in ranks]
        tslot = rng.integers(0, 4, size=T, dtype=np.int64)
        return make_workload(name=CONFIG_NAMES[1], dtype="f32", T=T, in_features=in_f,
                             out_slices=over.get("out_slices", (256,)), R=8, slots=4,
                             ranks=ranks, scalings=scal, token_slot=tslot, seed=seed,
                             rng=rng, y0_zero=y0_zero, target_name="linear")
    if k == 2:
        T = over.get("T", 256)
        slots = over.get("slots", 32)
        in_f = over.get("in_features", 4096)
        ranks = rng.choice(np.array([8, 16]), size=slots)
        scal = np.full(slots, 2.0, np.float32)
        tslot = rng.integers(0, slots, size=T, dtype=np.int64)
        return make_workload(name=CONFIG_NAMES[2], dtype="bf16", T=T, in_features=in_f,
                             out_slices=over.get("out_slices", (4096, 1024, 1024)), R=16,
                             slots=slots, ranks=ranks, scalings=scal, token_slot=tslot,
                             seed=seed, rng=rng, y0_zero=y0_zero, target_name="qkv")
    if k == 3:
        T = over.get("T", 8192)
        n_req = over.get("requests", 16)
        slots = over.get("slots", 16)
        hidden = over.get("in_features", 4096)
        inter = over.get("inter", 14336)
        R = 64
        ranks = np.full(slots, 64, np.int32)
        scal = np.full(slots, 16.0 / 64, np.float32)
        lens = zipf_request_lengths(n_req, T, 1.1)
        lens = lens[rng.permutation(n_req)]
        req_slot = rng.integers(0, slots, size=n_req, dtype=np.int64)
        tslot = np.repeat(req_slot, lens)
        wl = Workload(name=CONFIG_NAMES[3], dtype="bf16", T=T, R=R, slots=slots,
                      ranks=ranks, scalings=scal, token_slot=tslot.astype(np.int32),
                      seed=seed)
        wl.targets.append(_draw_target(rng, "gate_up", "bf16", T, hidden, (inter, inter),
                                       R, slots, y0_zero=y0_zero))
        wl.targets.append(_draw_target(rng, "down", "bf16", T, inter, (hidden,), R, slots,
                                       y0_zero=y0_zero))
        return wl
    if k == 4:
        T = over.get("T", 4096)
        vocab = over.get("vocab", 128256)
        hidden = over.get("out_features", 4096)
        ranks = [32, 16, 8, 0, 32, 16, 8, 32]
        scal = [16.0 / r if r else 0.0 for r in ranks]
        tslot = rng.integers(0, 8, size=T, dtype=np.int64)
        ids = rng.integers(0, vocab, size=T, dtype=np.int64)
        n_img = int(round(0.05 * T))
        ids[rng.choice(T, size=n_img, replace=False)] = -1
        return make_workload(name=CONFIG_NAMES[4], dtype="bf16", T=T, in_features=vocab,
                             out_slices=(hidden,), R=32, slots=8, ranks=ranks,
                             scalings=scal, token_slot=tslot, seed=seed, rng=rng,
                             ids=ids.astype(np.int32), y0_zero=y0_zero,
                             a_std=over.get("a_std"), target_name="embed")
    if k == 5:
        T = over.get("T", 4096)
        slots = over.get("slots", 128)
        in_f = over.get("in_features", 5120)
        R = 128
        ranks = rng.choice(np.array([0, 8, 16, 32, 64, 128]), size=slots)
        scal = rng.uniform(0.5, 4.0, size=slots).astype(np.float32)
        perm = rng.permutation(slots)
        p = np.arange(1, slots + 1, dtype=np.float64) ** -1.2
        p /= p.sum()
        pop = rng.choice(slots, size=T, p=p)
        tslot = perm[pop]
        return make_workload(name=CONFIG_NAMES[5], dtype="bf16", T=T, in_features=in_f,
                             out_slices=over.get("out_slices", (5120, 1024, 1024)), R=R,
                             slots=slots, ranks=ranks, scalings=scal, token_slot=tslot,
                             seed=seed, rng=rng, y0_zero=y0_zero, target_name="qkv")
    raise ValueError(f"unknown config {k}")


def poison_unread(wl: Workload) -> Workload:
    """Write NaN into every region the method never reads: A rows at or past a
    slot's rank (per slice), B columns at or past it, and all of A and B for
    rank-0 slots. Returns a new workload; the input is untouched."""
    nan = BF16_NAN if wl.dtype == "bf16" else np.float32(np.nan)
    out = Workload(**{**wl.__dict__, "targets": []})
    for tg in wl.targets:
        a = tg.a.copy()
        b = tg.b.copy()
        for s in range(wl.slots):
            r = int(min(max(int(wl.ranks[s]), 0), wl.R))
            for i in range(tg.num_slices):
                a[s, i * wl.R + r:(i + 1) * wl.R, :] = nan
            b[s, :, r:] = nan
        out.targets.append(Target(**{**tg.__dict__, "a": a, "b": b}))
    return out


def permute_tokens(wl: Workload, perm: np.ndarray) -> Workload:
    """Reorder the tokens of a workload (x, ids, y0 rows and token->slot)."""
    out = Workload(**{**wl.__dict__, "targets": [],
                      "token_slot": wl.token_slot[perm].copy()})
    for tg in wl.targets:
        out.targets.append(Target(**{
            **tg.__dict__,
            "y0": tg.y0[perm].copy(),
            "x": None if tg.x is None else tg.x[perm].copy(),
            "ids": None if tg.ids is None else tg.ids[perm].copy()}))
    return out


def take_tokens(wl: Workload, idx: np.ndarray) -> Workload:
    """Sub-batch of the given token rows (same slots, adapters and targets)."""
    idx = np.asarray(idx)
    out = Workload(**{**wl.__dict__, "targets": [], "T": int(len(idx)),
                      "token_slot": wl.token_slot[idx].copy()})
    for tg in wl.targets:
        out.targets.append(Target(**{
            **tg.__dict__,
            "y0": tg.y0[idx].copy(),
            "x": None if tg.x is None else tg.x[idx].copy(),
            "ids": None if tg.ids is None else tg.ids[idx].copy()}))
    return out
