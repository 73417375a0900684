"""GPU parity of lora_apply_linear_from_slots, the call that builds a step's
addressing and applies the first target in one launch (for a small bf16
batch over at most 63 slots; elsewhere the addressing kernel runs first).

Bars, on every case: the addressing it writes equals the oracle's, bit for
bit; y equals what build_addressing followed by apply_linear_ gives, bit for
bit (the same tokens reach the same tile rows, so the arithmetic is the
same); y is within |gpu - oracle| <= 1e-2 + 1e-2*|oracle| of the oracle.
"""
import sys

import numpy as np
import pytest

import adapter_lora_serving_amd as L
import oracle as O
import workloads as W
from gpu_util import GpuTarget, assert_tol, f64, torch
from test_gpu_parity import EDGE, SMALL, _custom, _random_shape

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _one_launch(wl, tg):
    code = 1 if wl.dtype == "bf16" else 0
    return L.from_slots_one_launch(code, wl.T, tg.in_features, tg.out_slices, wl.slots, wl.R)


def _check(wl, tg, what, expect_one=None):
    """Runs the one-call form and the two-call form on the same inputs and
    checks both bars; returns whether the one-call form was one launch."""
    t = torch()
    g = GpuTarget(wl, tg)
    one = _one_launch(wl, tg)
    if expect_one is not None:
        assert one == expect_one, f"{what}: one launch = {one}"
    y1 = g.y0.clone()
    addr1 = L.apply_linear_from_slots_(g.x, y1, g.a, g.b, g.token_slot, g.ranks, g.scal,
                                       tg.out_slices)
    t.cuda.synchronize()
    _, _, y2 = g.run(fused=True)
    order, indptr = O.build_addressing(np.asarray(wl.token_slot), wl.slots)
    assert np.array_equal(addr1.token_order.cpu().numpy(), order), f"{what}: token_order"
    assert np.array_equal(addr1.slot_indptr.cpu().numpy(), indptr), f"{what}: slot_indptr"
    assert t.equal(y1, y2), f"{what}: y differs from the two-call form"
    _, y_ref = O.run_target(wl, tg)
    assert_tol(f64(y1), y_ref, what)
    return one


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_full_one_launch(seed):
    log(f"from_slots decode full seed {seed}")
    wl = W.make_config(2, seed)
    _check(wl, wl.targets[0], f"decode seed {seed}", expect_one=True)


LINEAR = [(1, None), (2, None), (3, "gate_up"), (3, "down"), (5, None)]
ONE = {1: False, 2: True, 3: False, 5: True}   # fp32; T=256; T=1024 (segment tiles); T=768


@pytest.mark.parametrize("k,name", LINEAR)
def test_configs_small(k, name):
    log(f"from_slots config {k} {name}")
    wl = W.make_config(k, 0, **SMALL[k])
    _check(wl, wl.target(name), f"config {k} {name}", expect_one=ONE[k])


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_cases(case):
    log(f"from_slots edge {case}")
    wl = _custom(7, **EDGE[case])
    _check(wl, wl.targets[0], case)


def _random_small(seed):
    """A seeded batch inside the one-launch limits (T <= 1023, slots <= 63),
    skewed so that some segments pass 16 tokens (the 16-token prefill items)
    while the rest stay on the decode pieces."""
    rng = np.random.default_rng(2000 + seed)
    T = int(rng.integers(1, 1024))
    S = int(rng.integers(1, 4))
    widths = tuple(16 * int(rng.integers(1, 41)) for _ in range(S))
    R = int(rng.choice([8, 16, 32, 64]))
    slots = int(rng.integers(1, 64))
    ranks = [int(rng.integers(0, R + 1)) for _ in range(slots)]
    return dict(T=T, in_f=8 * int(rng.integers(1, 97)), out_slices=widths, R=R, slots=slots,
                ranks=ranks, dead=float(rng.choice([0.0, 0.1])),
                skew=float(rng.choice([0.0, 1.2, 2.0])))


@pytest.mark.parametrize("seed", range(16))
def test_random_one_launch(seed):
    case = _random_small(seed)
    log(f"from_slots random {seed}: T={case['T']} in={case['in_f']} out={case['out_slices']} "
        f"R={case['R']} slots={case['slots']}")
    wl = _custom(seed, **case)
    _check(wl, wl.targets[0], f"random small {seed}", expect_one=True)


@pytest.mark.parametrize("seed", range(8))
def test_random_any(seed):
    case = _random_shape(seed)
    log(f"from_slots random any {seed}: T={case['T']} slots={case['slots']}")
    wl = _custom(seed, **case)
    _check(wl, wl.targets[0], f"random any {seed}")


LIMITS = {
    # the largest one-launch batch and key count, long segments (prefill items)
    "T1023_slots63": dict(T=1023, in_f=256, out_slices=(128, 64), R=16, slots=63,
                          ranks=[16, 8, 0] * 21, dead=0.05),
    "T1000_slots3": dict(T=1000, in_f=264, out_slices=(96,), R=32, slots=3, ranks=[32, 5, 17]),
    "T1_slot0": dict(T=1, in_f=64, out_slices=(16,), R=8, slots=1, ranks=[8]),
    "T15_slots2": dict(T=15, in_f=128, out_slices=(32, 16), R=8, slots=2, ranks=[8, 3]),
    "mixed_16_17": dict(T=600, in_f=512, out_slices=(256,), R=16, slots=40, ranks=[16] * 40,
                        skew=1.0),
    # past the limits: the addressing kernel first, then the apply
    "slots64": dict(T=300, in_f=256, out_slices=(64,), R=16, slots=64, ranks=[16, 8] * 32),
    "T1024": dict(T=1024, in_f=256, out_slices=(64,), R=16, slots=8, ranks=[16] * 8),
    "T3000_twopass": dict(T=3000, in_f=128, out_slices=(32,), R=8, slots=20, ranks=[8] * 20,
                          dead=0.1),
}


@pytest.mark.parametrize("case", sorted(LIMITS))
def test_limits(case):
    log(f"from_slots limits {case}")
    wl = _custom(11, **LIMITS[case])
    expect = not (case.startswith("slots64") or case.startswith("T1024")
                  or case.startswith("T3000"))
    _check(wl, wl.targets[0], case, expect_one=expect)


def test_T0_writes_empty_addressing():
    t = torch()
    wl = _custom(3, T=8, in_f=64, out_slices=(16,), R=8, slots=5, ranks=[8] * 5)
    g = GpuTarget(wl, wl.targets[0])
    x0 = g.x[:0]
    y0 = g.y0[:0]
    out = L.Addressing(t.empty(0, dtype=t.int32, device="cuda:0"),
                       t.full((6,), 77, dtype=t.int32, device="cuda:0"))
    L.apply_linear_from_slots_(x0, y0, g.a, g.b, g.token_slot[:0], g.ranks, g.scal, (16,),
                               out=out)
    t.cuda.synchronize()
    assert out.slot_indptr.cpu().tolist() == [0] * 6


def test_addressing_serves_later_targets():
    """The addressing the first call writes drives the step's next target
    exactly as build_addressing's would."""
    log("from_slots: addressing reused by a second target")
    t = torch()
    wl = W.make_config(2, 4)
    tg = wl.targets[0]
    g = GpuTarget(wl, tg)
    y1 = g.y0.clone()
    addr = L.apply_linear_from_slots_(g.x, y1, g.a, g.b, g.token_slot, g.ranks, g.scal,
                                      tg.out_slices)
    y_next = g.y0.clone()
    L.apply_linear_(g.x, y_next, g.a, g.b, addr, g.ranks, g.scal, tg.out_slices)
    _, _, y_ref = g.run(fused=True)
    t.cuda.synchronize()
    assert t.equal(y_next, y_ref)


def test_graph_replays_equal_eager():
    """Captured once, replayed three times with eager work and
    synchronisations between: y and the addressing equal the eager call's
    on every replay."""
    log("from_slots graph replay")
    t = torch()
    wl = _custom(5, T=700, in_f=512, out_slices=(256, 64), R=32, slots=40,
                 ranks=[32, 16, 5, 0] * 10, skew=1.2, dead=0.05)
    tg = wl.targets[0]
    g = GpuTarget(wl, tg)
    y_e = g.y0.clone()
    a_e = L.apply_linear_from_slots_(g.x, y_e, g.a, g.b, g.token_slot, g.ranks, g.scal,
                                     tg.out_slices)
    t.cuda.synchronize()
    y_g = g.y0.clone()
    out = L.Addressing(t.empty(wl.T, dtype=t.int32, device="cuda:0"),
                       t.empty(wl.slots + 1, dtype=t.int32, device="cuda:0"))
    ws = t.zeros(L.lib().lora_apply_linear_from_slots_workspace_bytes(
        wl.T, tg.in_features, wl.slots, tg.num_slices, wl.R), dtype=t.uint8, device="cuda:0")
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    graph = t.cuda.CUDAGraph()
    with t.cuda.stream(s):
        with t.cuda.graph(graph, stream=s):
            L.apply_linear_from_slots_(g.x, y_g, g.a, g.b, g.token_slot, g.ranks, g.scal,
                                       tg.out_slices, out=out, workspace=ws)
    t.cuda.synchronize()
    for rep in range(3):
        y_g.copy_(g.y0)
        out.token_order.fill_(-5)
        out.slot_indptr.fill_(-5)
        _ = (g.x.float().sum() * 0).item()     # eager work between replays
        t.cuda.synchronize()
        graph.replay()
        t.cuda.synchronize()
        assert t.equal(y_g, y_e), f"replay {rep}: y"
        assert t.equal(out.token_order, a_e.token_order), f"replay {rep}: token_order"
        assert t.equal(out.slot_indptr, a_e.slot_indptr), f"replay {rep}: slot_indptr"
