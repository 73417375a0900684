"""Pins for the CPU oracle: each check ties it to something other than itself.

The pages print no numeric example, so the pins are: a hand-derived worked
example (tests/golden/worked_example.json), closed forms, special cases that
reduce to a plain dense matrix chain, a second formulation (the pages'
every-slot-then-select reference), scalar brute force, invariants stated by the
pages (rank-0 slots untouched, out-of-range ids contribute nothing, columns
past a rank are never read, rows are independent) and the matrix-rank bound a
low-rank update must obey. A mutation test at the end plants plausible
mistakes into copies of the oracle and checks that some pin catches each one.
"""
import inspect
import json
import os
import types

import numpy as np
import pytest

import oracle.lora_oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


# ---------------------------------------------------------------------------
# small random problems (float64 straight away; no bf16 involved)
# ---------------------------------------------------------------------------

def rand_problem(seed, T=37, in_f=19, out_slices=(7, 5, 3), R=6, slots=5,
                 ranks=None, dead_frac=0.15):
    rng = np.random.default_rng(seed)
    S = len(out_slices)
    out = sum(out_slices)
    ranks = rng.integers(0, R + 1, size=slots) if ranks is None else np.asarray(ranks)
    scal = rng.uniform(0.25, 3.0, size=slots)
    tslot = rng.integers(0, slots, size=T)
    dead = rng.random(T) < dead_frac
    tslot[dead] = rng.choice([-1, slots, slots + 3], size=int(dead.sum()))
    x = rng.standard_normal((T, in_f))
    a = rng.standard_normal((slots, S * R, in_f))
    b = rng.standard_normal((slots, out, R))
    y0 = rng.standard_normal((T, out))
    return types.SimpleNamespace(T=T, in_f=in_f, out_slices=tuple(out_slices), R=R,
                                 slots=slots, ranks=ranks.astype(np.int64), scal=scal,
                                 tslot=tslot.astype(np.int64), x=x, a=a, b=b, y0=y0)


def run(impl, p):
    h = impl.shrink(p.x, p.a, p.tslot, p.ranks, len(p.out_slices), p.R)
    return impl.expand(p.y0, h, p.b, p.tslot, p.ranks, p.scal, p.out_slices, p.R)


# ---------------------------------------------------------------------------
# pin checks, parametrised by the implementation so the mutation test can
# run them against planted mistakes
# ---------------------------------------------------------------------------

def check_worked_example(impl):
    g = json.load(open(GOLD))
    L = g["linear"]
    a = np.array(L["a"], float)
    b = np.array(L["b"], float)
    x = np.array(L["x"], float)
    y0 = np.array(L["y0"], float)
    ts = np.array(L["token_slot"])
    ranks = np.array(L["ranks"])
    order, indptr = impl.build_addressing(ts, L["slots"])
    assert order.tolist() == L["expect_token_order"]
    assert indptr.tolist() == L["expect_slot_indptr"]
    h = impl.shrink(x, a, ts, ranks, len(L["out_slices"]), L["R"])
    assert np.array_equal(h, np.array(L["expect_h"], float))
    y = impl.expand(y0, h, b, ts, ranks, np.array(L["scalings"]), L["out_slices"], L["R"])
    assert np.array_equal(y, np.array(L["expect_y"], float))
    E = g["embedding"]
    he = impl.gather_shrink(np.array(E["ids"]), np.array(E["a"], float),
                            np.array(E["token_slot"]), np.array(E["ranks"]), E["R"])
    assert np.array_equal(he, np.array(E["expect_h"], float))


def check_addressing_vs_argsort(impl):
    rng = np.random.default_rng(11)
    for trial in range(30):
        slots = int(rng.integers(1, 9))
        T = int(rng.integers(0, 200))
        ts = rng.integers(-2, slots + 2, size=T)
        order, indptr = impl.build_addressing(ts, slots)
        key = np.where((ts >= 0) & (ts < slots), ts, slots)
        assert np.array_equal(order, np.argsort(key, kind="stable"))
        assert np.array_equal(indptr, np.searchsorted(np.sort(key), np.arange(slots + 1)))


def check_closed_form_single_slot(impl):
    # one slot, every token live, full rank: per slice the delta is the dense
    # chain s * X @ A_i^T @ B_i^T written into columns [off_i, off_i + w_i)
    rng = np.random.default_rng(3)
    T, in_f, R, out_slices = 9, 11, 4, (6, 2, 5)
    S = len(out_slices)
    x = rng.standard_normal((T, in_f))
    a = rng.standard_normal((1, S * R, in_f))
    b = rng.standard_normal((1, sum(out_slices), R))
    y0 = rng.standard_normal((T, sum(out_slices)))
    s = 1.75
    ts = np.zeros(T, int)
    h = impl.shrink(x, a, ts, np.array([R]), S, R)
    y = impl.expand(y0, h, b, ts, np.array([R]), np.array([s]), out_slices, R)
    off = 0
    for i, w in enumerate(out_slices):
        Ai = a[0, i * R:(i + 1) * R]
        Bi = b[0, off:off + w]
        dense = s * (x @ Ai.T) @ Bi.T
        np.testing.assert_allclose(y[:, off:off + w] - y0[:, off:off + w], dense,
                                   rtol=1e-12, atol=1e-12)
        off += w


def check_rank0_and_dead_rows_untouched(impl):
    p = rand_problem(5, ranks=[0, 3, 0, 6, 2])
    y = run(impl, p)
    untouched = (p.tslot < 0) | (p.tslot >= p.slots)
    untouched |= np.isin(p.tslot, [0, 2])
    assert untouched.any()
    assert np.array_equal(y[untouched], p.y0[untouched])
    assert not np.array_equal(y[~untouched], p.y0[~untouched])


def check_gather_is_onehot_shrink(impl):
    rng = np.random.default_rng(7)
    T, vocab, R, slots = 40, 13, 5, 4
    a = rng.standard_normal((slots, R, vocab))
    ranks = np.array([5, 0, 2, 4])
    ts = rng.integers(-1, slots + 1, size=T)
    ids = rng.integers(-3, vocab + 3, size=T)
    onehot = np.zeros((T, vocab))
    ok = (ids >= 0) & (ids < vocab)
    onehot[np.nonzero(ok)[0], ids[ok]] = 1.0
    hg = impl.gather_shrink(ids, a, ts, ranks, R)
    hs = impl.shrink(onehot, a, ts, ranks, 1, R)
    assert np.array_equal(hg, hs)


def check_out_of_range_ids(impl):
    rng = np.random.default_rng(8)
    vocab, R, slots = 10, 3, 2
    a = rng.standard_normal((slots, R, vocab))
    b = rng.standard_normal((slots, 4, R))
    bad = np.array([-1, vocab, vocab + 7, np.iinfo(np.int32).min, np.iinfo(np.int32).max])
    ts = np.array([0, 1, 0, 1, 0])
    h = impl.gather_shrink(bad, a, ts, np.array([3, 2]), R)
    assert np.array_equal(h, np.zeros_like(h))
    y0 = rng.standard_normal((5, 4))
    y = impl.expand(y0, h, b, ts, np.array([3, 2]), np.array([1.0, 2.0]), (4,), R)
    assert np.array_equal(y, y0)


def check_permutation_invariance(impl):
    p = rand_problem(9)
    y = run(impl, p)
    perm = np.random.default_rng(1).permutation(p.T)
    q = types.SimpleNamespace(**{**p.__dict__, "x": p.x[perm], "tslot": p.tslot[perm],
                                 "y0": p.y0[perm]})
    np.testing.assert_allclose(run(impl, q), y[perm], rtol=1e-13, atol=1e-13)


def check_row_independence(impl):
    p = rand_problem(10)
    y = run(impl, p)
    k = p.T // 3
    parts = []
    for sl in (slice(0, k), slice(k, p.T)):
        q = types.SimpleNamespace(**{**p.__dict__, "x": p.x[sl], "tslot": p.tslot[sl],
                                     "y0": p.y0[sl], "T": len(p.x[sl])})
        parts.append(run(impl, q))
    np.testing.assert_allclose(np.concatenate(parts), y, rtol=1e-13, atol=1e-13)


def check_scaling_linearity(impl):
    p = rand_problem(12)
    y1 = run(impl, p)
    q = types.SimpleNamespace(**{**p.__dict__, "scal": 2.0 * p.scal})
    y2 = run(impl, q)
    np.testing.assert_allclose(y2 - p.y0, 2.0 * (y1 - p.y0), rtol=1e-12, atol=1e-12)


def check_poison_never_read(impl):
    p = rand_problem(13, ranks=[0, 2, 6, 3, 1])
    y = run(impl, p)
    a = p.a.copy()
    b = p.b.copy()
    for s in range(p.slots):
        r = int(p.ranks[s])
        for i in range(len(p.out_slices)):
            a[s, i * p.R + r:(i + 1) * p.R] = np.nan
        b[s, :, r:] = np.nan
    q = types.SimpleNamespace(**{**p.__dict__, "a": a, "b": b})
    yq = run(impl, q)
    assert np.all(np.isfinite(yq))
    assert np.array_equal(yq, y)


def check_all_slots_formulation(impl):
    p = rand_problem(14)
    S = len(p.out_slices)
    h1 = impl.shrink(p.x, p.a, p.tslot, p.ranks, S, p.R)
    h2 = O.shrink_all_slots(p.x, p.a, p.tslot, p.ranks, S, p.R)
    np.testing.assert_allclose(h1, h2, rtol=1e-12, atol=1e-12)


def check_scalar_brute_force(impl):
    p = rand_problem(15, T=12, in_f=7, out_slices=(3, 4), R=3, slots=3)
    y = run(impl, p)
    ys = O.apply_scalar(p.x, p.y0, p.a, p.b, p.tslot, p.ranks, p.scal, p.out_slices, p.R)
    np.testing.assert_allclose(y, ys, rtol=1e-12, atol=1e-12)
    rng = np.random.default_rng(2)
    a = rng.standard_normal((3, 3, 9))
    ids = rng.integers(-2, 11, size=12)
    h = impl.gather_shrink(ids, a, p.tslot, p.ranks, 3)
    ye = impl.expand(p.y0[:, :5], h, p.b[:, :5], p.tslot, p.ranks, p.scal, (5,), 3)
    yse = O.apply_scalar(ids, p.y0[:, :5], a, p.b[:, :5], p.tslot, p.ranks, p.scal, (5,),
                         3, embedding=True)
    np.testing.assert_allclose(ye, yse, rtol=1e-12, atol=1e-12)


def check_low_rank_bound(impl):
    # for one slot and one slice the delta over that slot's tokens is a product
    # through an r-dimensional space: its matrix rank is at most r
    p = rand_problem(16, T=80, in_f=30, out_slices=(25, 20), R=8, slots=3,
                     ranks=[3, 8, 5], dead_frac=0.0)
    y = run(impl, p)
    d = y - p.y0
    off = 0
    for w in p.out_slices:
        for s in range(p.slots):
            rows = np.nonzero(p.tslot == s)[0]
            sv = np.linalg.svd(d[np.ix_(rows, np.arange(off, off + w))], compute_uv=False)
            r = int(p.ranks[s])
            assert np.sum(sv > 1e-9 * sv[0]) == r, (s, r, sv[:10])
        off += w


PINS = [check_worked_example, check_addressing_vs_argsort, check_closed_form_single_slot,
        check_rank0_and_dead_rows_untouched, check_gather_is_onehot_shrink,
        check_out_of_range_ids, check_permutation_invariance, check_row_independence,
        check_scaling_linearity, check_poison_never_read, check_all_slots_formulation,
        check_scalar_brute_force, check_low_rank_bound]


@pytest.mark.parametrize("pin", PINS, ids=[f.__name__ for f in PINS])
def test_oracle_pin(pin):
    pin(O)


# ---------------------------------------------------------------------------
# the oracle on generated workloads (bf16 decode + the same pins at real dtypes)
# ---------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8,
                                  3.3895e38, 1e-40, 0.0, -0.0], np.float32)])
    ours = W.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # and the oracle's exact decode returns torch's widening of the same bits
    back = O.decode(ours, "bf16")
    tb = torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(back, tb)


def test_generators_deterministic():
    a = W.make_config(2, seed=1, T=32, in_features=64, slots=4)
    b = W.make_config(2, seed=1, T=32, in_features=64, slots=4)
    c = W.make_config(2, seed=2, T=32, in_features=64, slots=4)
    for f in ("x", "a", "b", "y0"):
        assert np.array_equal(getattr(a.targets[0], f), getattr(b.targets[0], f))
    assert not np.array_equal(a.targets[0].x, c.targets[0].x)
    assert np.array_equal(a.token_slot, b.token_slot)


def test_config_recipes():
    c3 = W.make_config(3, seed=0, T=8192, requests=16, in_features=8, inter=8)
    # 16 contiguous requests with the rank-frequency Zipf(1.1) lengths
    runs = np.flatnonzero(np.diff(np.r_[-1, np.arange(8192)]))  # noqa: F841
    lens = W.zipf_request_lengths(16, 8192, 1.1)
    assert lens.tolist() == [2704, 1262, 808, 589, 460, 377, 318, 275, 241, 215, 193,
                             176, 161, 148, 137, 128]
    assert c3.T == 8192 and [t.name for t in c3.targets] == ["gate_up", "down"]
    c4 = W.make_config(4, seed=0, T=4096, vocab=64, out_features=8)
    assert int((c4.targets[0].ids == -1).sum()) == 205
    assert c4.scalings.tolist() == [0.5, 1.0, 2.0, 0.0, 0.5, 1.0, 2.0, 0.5]
    c5 = W.make_config(5, seed=0, T=4096, in_features=8, out_slices=(8, 4, 4))
    assert set(np.unique(c5.ranks)) <= {0, 8, 16, 32, 64, 128}
    assert 0.5 <= c5.scalings.min() and c5.scalings.max() <= 4.0
    counts = np.bincount(c5.token_slot, minlength=128)
    assert counts.max() > 700        # skewed: P(top rank) ~ 0.27


@pytest.mark.parametrize("k", [1, 2, 4, 5])
def test_oracle_poison_on_configs(k):
    small = {1: {}, 2: dict(T=64, in_features=128, slots=8, out_slices=(64, 32, 16)),
             4: dict(T=256, vocab=300, out_features=64),
             5: dict(T=128, in_features=96, slots=16, out_slices=(48, 16, 16))}[k]
    wl = W.make_config(k, seed=0, **small)
    pw = W.poison_unread(wl)
    for tg, ptg in zip(wl.targets, pw.targets):
        h1, y1 = O.run_target(wl, tg)
        h2, y2 = O.run_target(pw, ptg)
        assert np.all(np.isfinite(y2))
        assert np.array_equal(y1, y2)
        assert np.array_equal(h1, h2)


# ---------------------------------------------------------------------------
# mutation test: plant a mistake into a copy of one oracle function and make
# sure at least one pin fails
# ---------------------------------------------------------------------------

MUTANTS = [
    ("expand", "off += w", "off += w - 1"),                               # slice offset
    ("expand", "float(scalings[s]) *", ""),                               # dropped scaling
    ("expand", "+= float(scalings[s])", "-= float(scalings[s])"),         # sign
    ("expand", "float(scalings[s])", "float(scalings[0])"),               # wrong slot's scaling
    ("expand", "bs = b[s, off: off + w, :r]", "bs = b[s, off: off + w, 1:r + 1]"),  # past rank
    ("expand", "hs @ bs.T", "hs[::-1] @ bs.T"),                           # rows swapped
    ("shrink", "a[s, i * R: i * R + r, :]", "a[s, i * r: i * r + r, :]"),  # slice stride
    ("shrink", "r = _rank(ranks, s, R)", "r = R"),                        # ignores rank
    ("shrink", "x[toks] @ rows.T", "x[toks][:, ::-1] @ rows.T"),          # transposed operand
    ("gather_shrink", "0 <= v < vocab", "v < vocab"),                     # -1 wraps
    ("gather_shrink", "h[t, :r] = a[s, :r, v]", "h[t, :r] = a[s, v % a.shape[1], :r]"),
    ("build_addressing", "for t in range(T):", "for t in reversed(range(T)):"),  # unstable
    ("build_addressing", "if _live(int(s), slots) else slots", "if _live(int(s), slots) else 0"),
]


def _mutant(fn_name, old, new):
    src = inspect.getsource(getattr(O, fn_name))
    assert old in src, (fn_name, old)
    ns = dict(vars(O))
    exec(src.replace(old, new, 1), ns)
    m = types.SimpleNamespace(**{k: getattr(O, k) for k in
                                 ("build_addressing", "shrink", "gather_shrink", "expand")})
    setattr(m, fn_name, ns[fn_name])
    return m


@pytest.mark.parametrize("mut", MUTANTS, ids=[f"{m[0]}:{m[2][:24]}" for m in MUTANTS])
def test_pins_catch_planted_mistake(mut):
    impl = _mutant(*mut)
    caught = []
    for pin in PINS:
        try:
            pin(impl)
        except Exception:  # an assertion or a shape error both mean "caught"
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {mut}"


# ---------------------------------------------------------------------------
# the routed-expert addressing (page "spark_model/lora/expert_apply.rs", the
# experts injection shape): composite key of (expert, slot) per row of an
# expert-sorted batch, then the stable grouping of the addressing
# ---------------------------------------------------------------------------

GOLD_EXPERT = os.path.join(os.path.dirname(__file__), "golden", "expert_keys.json")


def _experts_addressing(impl, row_slot, offs, E, slots):
    return impl.build_addressing(impl.expert_keys(row_slot, offs, E, slots), E * slots)


def check_expert_keys_golden(impl):
    """The hand-worked example: rows before expert_offsets[0] and at or after
    expert_offsets[E], an empty expert, and slots outside [0, slots)."""
    g = json.load(open(GOLD_EXPERT))
    keys = impl.expert_keys(g["row_slot"], g["expert_offsets"], g["num_experts"], g["slots"])
    assert np.asarray(keys).tolist() == g["expect_keys"]
    order, indptr = _experts_addressing(impl, g["row_slot"], g["expert_offsets"],
                                        g["num_experts"], g["slots"])
    assert order.tolist() == g["expect_token_order"]
    assert indptr.tolist() == g["expect_slot_indptr"]


def check_expert_vs_sorted(impl):
    """Brute force: Python's sorted by (expert, slot, row), dead rows (bad slot,
    or outside [offsets[0], offsets[E])) last by row; expert bounds drawn so
    that rows fall outside them at both ends."""
    rng = np.random.default_rng(11)
    for rows, E, slots in ((1, 1, 1), (40, 3, 5), (300, 8, 16), (97, 5, 3)):
        cuts = np.sort(rng.integers(0, rows + 1, size=E + 1))
        offs = cuts.astype(np.int32)                 # offs[0] > 0 and offs[E] < rows mostly
        if rows > 4:
            offs[0], offs[-1] = min(offs[0], 2) + 1, max(offs[-1], rows - 3) - 1
            offs = np.maximum.accumulate(offs)
        row_slot = rng.integers(-1, slots + 1, size=rows)
        order, indptr = _experts_addressing(impl, row_slot, offs, E, slots)
        expert = [next((e for e in range(E) if offs[e] <= r < offs[e + 1]), None)
                  for r in range(rows)]
        live = [expert[r] is not None and 0 <= row_slot[r] < slots for r in range(rows)]
        want = sorted(range(rows), key=lambda r: (0, expert[r], int(row_slot[r]), r) if live[r]
                      else (1, 0, 0, r))
        assert order.tolist() == want
        for e in range(E):
            for sl in range(slots):
                k = e * slots + sl
                assert int(indptr[k + 1] - indptr[k]) == sum(
                    1 for r in range(rows) if live[r] and expert[r] == e and row_slot[r] == sl)
        assert int(indptr[-1]) == sum(live)


EXPERT_PINS = [check_expert_keys_golden, check_expert_vs_sorted]


@pytest.mark.parametrize("pin", EXPERT_PINS, ids=[f.__name__ for f in EXPERT_PINS])
def test_expert_pin(pin):
    pin(O)


EXPERT_MUTANTS = [
    # rows outside every expert range default to expert 0 instead of dead
    ("expert_keys", "keys = np.full(len(row_slot), -1, dtype=np.int64)",
     "keys = np.where((np.asarray(row_slot) >= 0) & (np.asarray(row_slot) < slots), "
     "np.asarray(row_slot), -1).astype(np.int64)"),
    # an expert's range taken as closed at its end
    ("expert_keys", "int(expert_offsets[e + 1])", "int(expert_offsets[e + 1]) + 1"),
    # expert and slot transposed in the key
    ("expert_keys", "keys[r] = e * slots + int(row_slot[r])",
     "keys[r] = int(row_slot[r]) * num_experts + e"),
    # a bad slot not treated as dead
    ("expert_keys", "_live(int(row_slot[r]), slots)", "int(row_slot[r]) < slots"),
]


def _expert_mutant(fn_name, old, new):
    src = inspect.getsource(getattr(O, fn_name))
    assert old in src, (fn_name, old)
    ns = dict(vars(O))
    exec(src.replace(old, new, 1), ns)
    return types.SimpleNamespace(expert_keys=ns["expert_keys"],
                                 build_addressing=O.build_addressing)


@pytest.mark.parametrize("mut", EXPERT_MUTANTS, ids=[f"{m[0]}:{m[2][:28]}" for m in EXPERT_MUTANTS])
def test_expert_pins_catch_planted_mistake(mut):
    impl = _expert_mutant(*mut)
    caught = []
    for pin in EXPERT_PINS:
        try:
            pin(impl)
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {mut}"


# ---------------------------------------------------------------------------
# the workload-level helpers every GPU parity test goes through
# ---------------------------------------------------------------------------

def _worked_example_workload():
    """The hand-worked linear example as a generated workload (float32: every
    value in it is exact in fp32)."""
    g = json.load(open(GOLD))
    L = g["linear"]
    f32 = lambda v: np.asarray(v, dtype=np.float32)  # noqa: E731
    wl = W.Workload(name="worked", dtype="f32", T=len(L["token_slot"]), R=L["R"],
                    slots=L["slots"], ranks=np.asarray(L["ranks"], np.int32),
                    scalings=f32(L["scalings"]), token_slot=np.asarray(L["token_slot"], np.int32))
    wl.targets.append(W.Target(name="t", in_features=len(L["x"][0]),
                               out_slices=tuple(L["out_slices"]), a=f32(L["a"]), b=f32(L["b"]),
                               y0=f32(L["y0"]), x=f32(L["x"])))
    E = g["embedding"]
    we = W.Workload(name="worked_emb", dtype="f32", T=len(E["token_slot"]), R=E["R"],
                    slots=E["slots"], ranks=np.asarray(E["ranks"], np.int32),
                    scalings=np.ones(E["slots"], np.float32),
                    token_slot=np.asarray(E["token_slot"], np.int32))
    a = f32(E["a"])
    we.targets.append(W.Target(name="e", in_features=a.shape[2], out_slices=(1,), a=a,
                               b=np.ones((E["slots"], 1, E["R"]), np.float32),
                               y0=np.zeros((len(E["token_slot"]), 1), np.float32),
                               ids=np.asarray(E["ids"], np.int32)))
    return g, wl, we


def check_run_target_worked_example(impl):
    """run_target (decode, shrink or gather, then expand) reproduces the
    hand-worked h and y; the embedding target's y is the sum of its h row
    (b = 1, scaling 1, y0 = 0)."""
    g, wl, we = _worked_example_workload()
    h, y = impl.run_target(wl, wl.targets[0])
    assert np.array_equal(h, np.array(g["linear"]["expect_h"], float))
    assert np.array_equal(y, np.array(g["linear"]["expect_y"], float))
    he, ye = impl.run_target(we, we.targets[0])
    want = np.array(g["embedding"]["expect_h"], float)
    assert np.array_equal(he, want)
    assert np.array_equal(ye[:, 0], want.sum(axis=1))


def check_run_target_decodes_bf16(impl):
    """The bf16 path of run_target decodes the bit patterns exactly: the same
    example written as bf16 bits (all its values are exact in bf16) gives the
    same h and y."""
    g, wl, _ = _worked_example_workload()
    tg = wl.targets[0]
    bits = {k: W.f32_to_bf16_bits(getattr(tg, k)) for k in ("a", "b", "y0", "x")}
    wb = W.Workload(**{**wl.__dict__, "dtype": "bf16", "targets": []})
    wb.targets.append(W.Target(**{**tg.__dict__, **bits}))
    h, y = impl.run_target(wb, wb.targets[0])
    assert np.array_equal(h, np.array(g["linear"]["expect_h"], float))
    assert np.array_equal(y, np.array(g["linear"]["expect_y"], float))


def check_within_tolerance(impl):
    O = impl  # noqa: N806  (the checks below read as calls of the oracle)
    ref = np.array([0.0, 1.0, -2.0, 100.0])
    # just inside the bound 1e-2 + 1e-2 |ref| passes, just past it fails
    bound = 1e-2 + 1e-2 * np.abs(ref)
    ok, worst = O.within_tolerance(ref + 0.999 * bound, ref)
    assert ok and abs(worst - 0.999) < 1e-9
    ok, worst = O.within_tolerance(ref - 0.999 * bound, ref)
    assert ok and abs(worst - 0.999) < 1e-9
    ok, worst = O.within_tolerance(ref + 1.001 * bound, ref)
    assert not ok and worst > 1.0
    ok, worst = O.within_tolerance(ref - 1.001 * bound, ref)
    assert not ok and worst > 1.0
    # a single element past the bound fails; the worst ratio names it
    gpu = ref.copy()
    gpu[3] += 3.0 * bound[3]
    ok, worst = O.within_tolerance(gpu, ref)
    assert not ok and abs(worst - 3.0) < 1e-9
    # NaN or inf in the result never passes
    for bad in (np.nan, np.inf, -np.inf):
        gpu = ref.copy()
        gpu[1] = bad
        assert not O.within_tolerance(gpu, ref)[0]
    # tighter bounds are honoured
    assert O.within_tolerance(ref + 5e-6, ref, atol=1e-5, rtol=1e-5)[0]
    assert not O.within_tolerance(ref + 5e-4, ref, atol=1e-5, rtol=1e-5)[0]
    # empty input passes trivially
    assert O.within_tolerance(np.zeros(0), np.zeros(0)) == (True, 0.0)


HELPER_PINS = [check_run_target_worked_example, check_run_target_decodes_bf16,
               check_within_tolerance]


@pytest.mark.parametrize("pin", HELPER_PINS, ids=[f.__name__ for f in HELPER_PINS])
def test_helper_pin(pin):
    pin(O)


HELPER_MUTANTS = [
    ("run_target", "y0 = decode(tg.y0, wl.dtype)", "y0 = 0.0 * decode(tg.y0, wl.dtype)"),
    ("run_target", "tg.num_slices, wl.R)", "1, wl.R)"),
    ("run_target", "wl.scalings, tg.out_slices", "np.ones_like(wl.scalings), tg.out_slices"),
    ("run_target", "b = decode(tg.b, wl.dtype)", "b = decode(tg.b, \"f32\")"),
    ("within_tolerance", "np.abs(gpu - ref)", "(gpu - ref)"),
    ("within_tolerance", "rtol * np.abs(ref)", "rtol * np.abs(gpu)"),
    ("within_tolerance", "ratio <= 1.0", "ratio <= 1.5"),
    ("within_tolerance", "np.nanmax(ratio)", "np.nanmean(ratio)"),
]


@pytest.mark.parametrize("mut", HELPER_MUTANTS, ids=[f"{m[0]}:{m[2][:28]}" for m in HELPER_MUTANTS])
def test_helper_pins_catch_planted_mistake(mut):
    fn_name, old, new = mut
    src = inspect.getsource(getattr(O, fn_name))
    assert old in src, mut
    ns = dict(vars(O))
    exec(src.replace(old, new, 1), ns)
    impl = types.SimpleNamespace(run_target=O.run_target, within_tolerance=O.within_tolerance)
    setattr(impl, fn_name, ns[fn_name])
    caught = []
    for pin in HELPER_PINS:
        try:
            pin(impl)
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {mut}"


# ---------------------------------------------------------------------------
# the base projection (mstar.model.components.linear, FusedColumnLinear) and
# the delta added on top of it: the merged-weight closed form
# ---------------------------------------------------------------------------

def test_base_projection_brute_force_and_identity():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((5, 7))
    w = rng.standard_normal((6, 7))
    y = O.base_projection(x, w)
    for t in range(5):
        for o in range(6):
            assert abs(y[t, o] - sum(x[t, c] * w[o, c] for c in range(7))) < 1e-12
    assert np.array_equal(O.base_projection(x, np.eye(7)), x)
    # shards stacked along the output dimension give their columns in order
    wq, wk = rng.standard_normal((4, 7)), rng.standard_normal((2, 7))
    yq, yk = O.base_projection(x, wq), O.base_projection(x, wk)
    assert np.array_equal(O.base_projection(x, np.vstack([wq, wk])), np.hstack([yq, yk]))


def test_base_plus_delta_is_merged_weight():
    """For one slot at full rank, the base projection plus the LoRA delta is
    the projection through the merged weight W_i + s * B_i @ A_i per slice
    (the closed form of a LoRA-adapted linear layer)."""
    rng = np.random.default_rng(22)
    T, in_f, R, out_slices = 9, 13, 3, (5, 4, 6)
    S = len(out_slices)
    out = sum(out_slices)
    x = rng.standard_normal((T, in_f))
    w = rng.standard_normal((out, in_f))
    a = rng.standard_normal((1, S * R, in_f))
    b = rng.standard_normal((1, out, R))
    s = 0.75
    ts = np.zeros(T, int)
    h = O.shrink(x, a, ts, np.array([R]), S, R)
    y = O.expand(O.base_projection(x, w), h, b, ts, np.array([R]), np.array([s]), out_slices, R)
    merged = w.copy()
    off = 0
    for i, wd in enumerate(out_slices):
        merged[off:off + wd] += s * b[0, off:off + wd] @ a[0, i * R:(i + 1) * R]
        off += wd
    np.testing.assert_allclose(y, x @ merged.T, rtol=1e-12, atol=1e-12)


def test_moe_workload_through_the_oracle():
    """The routed-expert workload carries routing and pool only; with each
    row's pool entry from oracle.expert_keys it runs through the oracle, and
    every live row's entry is (its expert, its token's slot)."""
    wl = W.make_moe_experts(3, T=24, experts=4, hidden=32, inter=48, slots=5)
    assert wl.token_slot is None
    e = wl.experts
    keys = O.expert_keys(e["row_slot"], e["offsets"], e["experts"], e["slots"])
    kw = W.with_token_slot(wl, keys)
    assert kw.experts is e and kw.slots == 4 * 5 and kw.T == 48
    expert = np.searchsorted(e["offsets"], np.arange(kw.T), side="right") - 1
    assert np.array_equal(keys, expert * 5 + e["row_slot"])
    for name in ("expert_gate_up", "expert_down"):
        tg = kw.target(name)
        h, y = O.run_target(kw, tg)
        assert np.all(np.isfinite(y)) and y.shape == (48, tg.out_features)
