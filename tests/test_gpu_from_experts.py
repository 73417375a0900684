"""GPU parity of lora_apply_linear_from_experts, the call that builds a
routed-expert step's addressing (by expert and slot) and applies the first
expert target in one launch (fewer than 1024 rows, at most 63 experts and
1023 pool entries; elsewhere the addressing kernels run first).

Bars, on every case: the addressing it writes equals the oracle's, bit for
bit; y equals what build_addressing_experts followed by apply_linear_ gives,
bit for bit; y is within |gpu - oracle| <= 1e-2 + 1e-2*|oracle| of the
oracle, whose rows take their pool entries from oracle.expert_keys.
"""
import sys

import numpy as np
import pytest

import adapter_lora_serving_amd as L
import oracle as O
import workloads as W
from gpu_util import GpuTarget, assert_tol, f64, torch

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev_i32(a):
    return torch().from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")


def _check(wl, tg, what, expect_one=None):
    t = torch()
    e = wl.experts
    g = GpuTarget(wl, tg)
    one = L.from_experts_one_launch(1, wl.T, tg.in_features, tg.out_slices, e["experts"],
                                    e["slots"], wl.R)
    if expect_one is not None:
        assert one == expect_one, f"{what}: one launch = {one}"
    rs, offs = _dev_i32(e["row_slot"]), _dev_i32(e["offsets"])
    y1 = g.y0.clone()
    addr1 = L.apply_linear_from_experts_(g.x, y1, g.a, g.b, rs, offs, e["experts"], e["slots"],
                                         g.ranks, g.scal, tg.out_slices)
    addr2 = L.build_addressing_experts(rs, offs, e["experts"], e["slots"])
    y2 = g.y0.clone()
    L.apply_linear_(g.x, y2, g.a, g.b, addr2, g.ranks, g.scal, tg.out_slices)
    t.cuda.synchronize()
    order, indptr = O.build_addressing_experts(e["row_slot"], e["offsets"], e["experts"],
                                               e["slots"])
    assert np.array_equal(addr1.token_order.cpu().numpy(), order), f"{what}: token_order"
    assert np.array_equal(addr1.slot_indptr.cpu().numpy(), indptr), f"{what}: slot_indptr"
    assert t.equal(y1, y2), f"{what}: y differs from the two-call form"
    keys = O.expert_keys(e["row_slot"], e["offsets"], e["experts"], e["slots"])
    keyed = W.with_token_slot(wl, keys)
    _, y_ref = O.run_target(keyed, keyed.target(tg.name))
    assert_tol(f64(y1), y_ref, what)
    return one


_MOE = {}


def _moe(size):
    if size not in _MOE:
        over = dict(T=256, experts=8, hidden=1024, inter=2048) if size == "reduced" else {}
        _MOE[size] = W.make_moe_experts(5, **over)
    return _MOE[size]


@pytest.mark.parametrize("target", ["expert_gate_up", "expert_down"])
@pytest.mark.parametrize("size", ["reduced", "bench"])
def test_moe_one_launch(size, target):
    log(f"from_experts moe {size} {target}")
    wl = _moe(size)
    _check(wl, wl.target(target), f"moe {size} {target}", expect_one=True)


def _routing(seed, T, experts, slots, hidden, inter, dead_rows=True, bad_slots=True,
             empty=True, topk=2):
    """A seeded expert-sorted batch; optionally rows before the first and
    after the last expert bound (dead), slots outside [0, slots) (dead) and
    experts that own no rows."""
    wl = W.make_moe_experts(seed, T=T, experts=experts, topk=topk, hidden=hidden, inter=inter,
                            slots=slots)
    rng = np.random.default_rng(7000 + seed)
    e = wl.experts
    rows = wl.T
    rs = e["row_slot"].copy()
    offs = e["offsets"].astype(np.int64).copy()
    if bad_slots:
        k = rng.random(rows) < 0.05
        rs[k] = rng.choice(np.array([-1, slots, slots + 7]), size=int(k.sum()))
    if empty and experts > 2:   # one expert's rows go to its neighbour
        j = int(rng.integers(1, experts))
        offs[j] = offs[j - 1]
        offs = np.maximum.accumulate(offs)
    if dead_rows and rows > 8:
        offs[0] = min(3, int(offs[1]))
        offs[-1] = max(rows - 2, int(offs[-2]))
    e["row_slot"] = rs.astype(np.int32)
    e["offsets"] = offs.astype(np.int32)
    return wl


def _random_case(seed):
    rng = np.random.default_rng(3000 + seed)
    experts = int(rng.integers(1, 33))
    slots = int(rng.integers(1, max(2, 1023 // experts) + 1))
    slots = min(slots, 1023 // experts)
    topk = int(rng.integers(1, min(experts, 4) + 1))
    T = int(rng.integers(1, 1023 // topk + 1))   # rows <= 1023: the fused path
    hidden = 16 * int(rng.integers(1, 33))
    inter = 16 * int(rng.integers(1, 33))
    return dict(T=T, experts=experts, slots=slots, hidden=hidden, inter=inter, topk=topk)


@pytest.mark.parametrize("seed", range(12))
def test_random_one_launch(seed):
    c = _random_case(seed)
    log(f"from_experts random {seed}: {c}")
    wl = _routing(seed, **c)
    target = "expert_gate_up" if seed % 2 == 0 else "expert_down"
    _check(wl, wl.target(target), f"random {seed}", expect_one=True)


def _ranked(seed, R):
    """A seeded expert-sorted batch at rank R: the routing of a small MoE
    (with dead rows, bad slots and an empty expert), and adapters drawn at
    rank R with per-entry ranks in [0, R] (0 and R included)."""
    base = _routing(seed, T=160, experts=4, slots=8, hidden=64, inter=64, topk=2)
    e = base.experts
    K = e["experts"] * e["slots"]
    rng = np.random.default_rng(9000 + seed)
    ranks = rng.integers(0, R + 1, size=K)
    ranks[0], ranks[1] = 0, R
    keys = O.expert_keys(e["row_slot"], e["offsets"], e["experts"], e["slots"])
    wl = W.make_workload(name="experts_ranked", dtype="bf16", T=base.T, in_features=264,
                         out_slices=(128, 48), R=R, slots=K, ranks=ranks,
                         scalings=rng.uniform(0.5, 2.0, size=K), token_slot=keys, seed=seed,
                         rng=rng, target_name="expert_gate_up")
    wl.experts = e
    return wl


@pytest.mark.parametrize("R", [8, 32, 64, 128, 256])
def test_rank_buckets_one_launch(R):
    """Every rank bucket of the fused kernel's expert mode (1, 2, 4, 8 and 16
    rank tiles)."""
    log(f"from_experts rank {R}")
    wl = _ranked(40 + R, R)
    _check(wl, wl.targets[0], f"rank {R}", expect_one=True)


LIMITS = {
    # 63 experts, 1008 pool entries; 1022 rows; 1 row
    "E63": dict(T=300, experts=63, slots=16, hidden=128, inter=256, topk=2),
    "rows1022": dict(T=511, experts=8, slots=32, hidden=256, inter=128, topk=2),
    "E1_slots1023": dict(T=200, experts=1, slots=1023, hidden=64, inter=64, topk=1),
    "rows1": dict(T=1, experts=2, slots=4, hidden=64, inter=64, topk=1, dead_rows=False),
    "one_long_entry": dict(T=400, experts=2, slots=1, hidden=128, inter=128, topk=1,
                           bad_slots=False, empty=False),
    # past the limits: the addressing kernels first (1024 rows and more take
    # the segment tiles)
    "E64": dict(T=300, experts=64, slots=8, hidden=128, inter=128, topk=2),
    "K1024": dict(T=300, experts=32, slots=32, hidden=128, inter=128, topk=2),
    "rows1024": dict(T=512, experts=8, slots=16, hidden=128, inter=128, topk=2),
}


@pytest.mark.parametrize("case", sorted(LIMITS))
def test_limits(case):
    log(f"from_experts limits {case}")
    wl = _routing(11, **LIMITS[case])
    expect = case not in ("E64", "K1024", "rows1024")
    for target in ("expert_gate_up", "expert_down"):
        _check(wl, wl.target(target), f"{case} {target}", expect_one=expect)


def test_zero_rows_writes_empty_addressing():
    t = torch()
    wl = _moe("reduced")
    tg = wl.target("expert_down")
    g = GpuTarget(wl, tg)
    e = wl.experts
    out = L.Addressing(t.empty(0, dtype=t.int32, device="cuda:0"),
                       t.full((e["experts"] * e["slots"] + 1,), 77, dtype=t.int32,
                              device="cuda:0"))
    L.apply_linear_from_experts_(g.x[:0], g.y0[:0], g.a, g.b, _dev_i32(np.zeros(0)),
                                 _dev_i32(np.zeros(e["experts"] + 1)), e["experts"], e["slots"],
                                 g.ranks, g.scal, tg.out_slices, out=out)
    t.cuda.synchronize()
    assert out.slot_indptr.cpu().tolist() == [0] * (e["experts"] * e["slots"] + 1)


def test_graph_replays_equal_eager():
    """Captured once, replayed three times with eager work and
    synchronisations between: y and the addressing equal the eager call's
    on every replay."""
    log("from_experts graph replay")
    t = torch()
    wl = _routing(21, T=300, experts=8, slots=16, hidden=256, inter=512)
    tg = wl.target("expert_gate_up")
    g = GpuTarget(wl, tg)
    e = wl.experts
    rs, offs = _dev_i32(e["row_slot"]), _dev_i32(e["offsets"])
    y_e = g.y0.clone()
    a_e = L.apply_linear_from_experts_(g.x, y_e, g.a, g.b, rs, offs, e["experts"], e["slots"],
                                       g.ranks, g.scal, tg.out_slices)
    t.cuda.synchronize()
    K = e["experts"] * e["slots"]
    out = L.Addressing(t.empty(wl.T, dtype=t.int32, device="cuda:0"),
                       t.empty(K + 1, dtype=t.int32, device="cuda:0"))
    ws = t.zeros(L.lib().lora_apply_linear_from_experts_workspace_bytes(
        wl.T, tg.in_features, e["experts"], e["slots"], tg.num_slices, wl.R), dtype=t.uint8,
        device="cuda:0")
    y_g = g.y0.clone()
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    graph = t.cuda.CUDAGraph()
    with t.cuda.stream(s):
        with t.cuda.graph(graph, stream=s):
            L.apply_linear_from_experts_(g.x, y_g, g.a, g.b, rs, offs, e["experts"], e["slots"],
                                         g.ranks, g.scal, tg.out_slices, out=out, workspace=ws)
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
