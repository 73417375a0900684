"""GPU parity of the base projection with the LoRA delta in its epilogue
(lora_fused_column_linear) and of the base projection alone
(lora_column_linear), through the C ABI, against the oracle: the fp64 base
product (oracle.base_projection, pinned by the merged-weight closed form)
with the delta added on top (oracle.expand of oracle.shrink). Bar:
|gpu - oracle| <= 1e-2 + 1e-2 |oracle| elementwise."""
import sys

import numpy as np
import pytest

import adapter_lora_serving_amd as L
import oracle as O
import workloads as W
from gpu_util import GpuTarget, assert_tol, dev, f64, torch

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _reference(wl, tg, w, rows=None):
    """oracle y = x @ W^T + delta, on all rows or the given ones."""
    sub = wl if rows is None else W.take_tokens(wl, rows)
    stg = sub.target(tg.name)
    x = O.decode(stg.x, wl.dtype)
    base = O.base_projection(x, O.decode(w, wl.dtype))
    h = O.shrink(x, O.decode(stg.a, wl.dtype), sub.token_slot, sub.ranks, stg.num_slices, sub.R)
    return O.expand(base, h, O.decode(stg.b, wl.dtype), sub.token_slot, sub.ranks, sub.scalings,
                    stg.out_slices, sub.R)


def _run(wl, tg, w, fused=True):
    g = GpuTarget(wl, tg)
    wd = dev(w, wl.dtype)
    addr = g.addressing()
    if fused:
        y = L.fused_column_linear(g.x, wd, g.a, g.b, addr, g.ranks, g.scal, tg.out_slices)
    else:
        y = L.column_linear(g.x, wd, tg.out_slices)
        L.apply_linear_(g.x, y, g.a, g.b, addr, g.ranks, g.scal, tg.out_slices)
    torch().cuda.synchronize()
    return f64(y)


CASES = {
    # the decode qkv batch, whole
    "decode_qkv": (2, {}, None),
    # prefill: 1024 tokens in 16 requests, gate/up (two 1024-wide slices) and down
    "prefill_gate_up": (3, dict(T=1024, in_features=512, inter=1024), "gate_up"),
    "prefill_down": (3, dict(T=1024, in_features=1024, inter=512), "down"),
    # the skewed 128-adapter mix, ragged T, three slices of 512 / 256 / 256
    "skewed_ragged": (5, dict(T=700, in_features=640, slots=32, out_slices=(512, 256, 256)), None),
}


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("case", sorted(CASES))
def test_fused_column_linear(case, fused):
    log(f"fused column linear {case} fused={fused}")
    k, over, name = CASES[case]
    wl = W.make_config(k, 1, **over)
    tg = wl.target(name)
    w = W.base_weight(wl, tg)
    y = _run(wl, tg, w, fused)
    assert_tol(y, _reference(wl, tg, w), case)


def test_column_linear_base_only():
    """The base projection alone equals oracle.base_projection."""
    wl = W.make_config(3, 2, T=600, in_features=768, inter=1280)
    tg = wl.target("gate_up")
    w = W.base_weight(wl, tg)
    g = GpuTarget(wl, tg)
    y = L.column_linear(g.x, dev(w, "bf16"), tg.out_slices)
    torch().cuda.synchronize()
    ref = O.base_projection(O.decode(tg.x, "bf16"), O.decode(w, "bf16"))
    assert_tol(f64(y), ref, "base only")


def test_fused_column_linear_edges():
    """Dead tokens and rank-0 slots get the base projection only; NaN in
    every never-read A row / B column changes nothing, bit for bit; `in` not
    a multiple of the 64-deep K step."""
    rng = np.random.default_rng(3)
    T, in_f, R, slots = 333, 200, 32, 6
    ts = rng.integers(0, slots, size=T)
    ts[rng.random(T) < 0.1] = -1
    wl = W.make_workload(name="edges", dtype="bf16", T=T, in_features=in_f,
                         out_slices=(256, 512), R=R, slots=slots,
                         ranks=[32, 0, 7, 16, 1, 25], scalings=rng.uniform(0.5, 2, slots),
                         token_slot=ts, seed=3, rng=rng)
    tg = wl.targets[0]
    w = W.base_weight(wl, tg)
    y = _run(wl, tg, w)
    ref = _reference(wl, tg, w)
    assert_tol(y, ref, "edges")
    base = O.base_projection(O.decode(tg.x, "bf16"), O.decode(w, "bf16"))
    plain = (ts < 0) | np.isin(ts, [1])
    assert_tol(y[plain], base[plain], "dead and rank-0 rows")
    pw = W.poison_unread(wl)
    y2 = _run(pw, pw.targets[0], w)
    assert np.all(np.isfinite(y2)) and np.array_equal(y, y2)


@pytest.mark.slow
def test_fused_column_linear_prefill_full_sampled():
    """The full prefill gate/up shape (8192 tokens, in 4096, out 2 x 14336)
    that the benchmark times; the oracle checks sampled rows (the first and
    last token of every segment plus random ones): each row's output depends
    on that row alone."""
    log("fused column linear, full prefill gate/up, sampled rows")
    wl = W.make_config(3, 0)
    tg = wl.target("gate_up")
    w = W.base_weight(wl, tg)
    y = _run(wl, tg, w)
    order, indptr = O.build_addressing(wl.token_slot, wl.slots)
    pick = {0, wl.T - 1}
    for s in range(wl.slots):
        if indptr[s + 1] > indptr[s]:
            pick.update([int(order[indptr[s]]), int(order[indptr[s + 1] - 1])])
    pick.update(np.random.default_rng(4).choice(wl.T, size=40, replace=False).tolist())
    idx = np.array(sorted(pick))
    assert_tol(y[idx], _reference(wl, tg, w, rows=idx), "full prefill gate/up")


def test_fused_column_linear_graph_equals_eager():
    """The addressing build and the fused call recorded in one hipGraph
    (a batch over 1024 tokens, so the shrink's K parts live in the
    workspace), replayed with new x and new token slots: every replay equals
    eager execution on the same inputs bit for bit, and two eager calls are
    bit-identical."""
    t = torch()
    wl = W.make_config(3, 4, T=1100, in_features=512, inter=768)
    tg = wl.target("gate_up")
    w = dev(W.base_weight(wl, tg), "bf16")
    g = GpuTarget(wl, tg)
    T, out = wl.T, sum(tg.out_slices)
    ts = g.token_slot.clone()
    x = g.x.clone()
    addr = L.build_addressing(ts, wl.slots)
    y = t.empty(T, out, dtype=t.bfloat16, device="cuda:0")
    need = int(L.lib().lora_fused_column_linear_workspace_bytes(T, tg.in_features,
                                                               tg.num_slices, wl.R))
    ws = t.empty(need, dtype=t.uint8, device="cuda:0")

    def step():
        L.build_addressing(ts, wl.slots, out=addr)
        L.fused_column_linear(x, w, g.a, g.b, addr, g.ranks, g.scal, tg.out_slices, y=y,
                              workspace=ws)

    step()
    t.cuda.synchronize()
    y_first = y.clone()
    step()
    t.cuda.synchronize()
    assert t.equal(y, y_first), "two eager calls differ"

    graph = t.cuda.CUDAGraph()
    st = t.cuda.Stream()
    with t.cuda.stream(st):
        with t.cuda.graph(graph, stream=st):
            step()
    t.cuda.synchronize()
    rng = np.random.default_rng(21)
    for rep in range(3):
        log(f"fused linear graph replay {rep}")
        new_x = W.f32_to_bf16_bits(rng.standard_normal((T, tg.in_features), dtype=np.float32))
        new_ts = rng.integers(-1, wl.slots, size=T).astype(np.int32)
        x.copy_(dev(new_x, "bf16"))
        ts.copy_(t.from_numpy(new_ts))
        t.cuda.synchronize()
        graph.replay()
        t.cuda.synchronize()
        y_graph = y.clone()
        a_e = L.build_addressing(t.from_numpy(new_ts).to("cuda:0"), wl.slots)
        y_e = L.fused_column_linear(dev(new_x, "bf16"), w, g.a, g.b, a_e, g.ranks, g.scal,
                                    tg.out_slices)
        t.cuda.synchronize()
        assert t.equal(addr.token_order, a_e.token_order)
        assert t.equal(y_graph, y_e), f"replay {rep}"


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("seed", range(8))
def test_random_fused_column_linear(seed, fused):
    """Seeded random shapes for the base projection with the delta in its
    epilogue (and for our GEMM followed by lora_apply_linear): T, `in`, 1-3
    slices of 256-multiples, rank, slots, ranks, dead tokens and skew drawn."""
    rng = np.random.default_rng(4000 + seed)
    T = int(rng.choice([int(rng.integers(1, 1024)), int(rng.integers(1024, 1800))]))
    in_f = 8 * int(rng.integers(1, 97))
    S = int(rng.integers(1, 4))
    widths = tuple(256 * int(rng.integers(1, 4)) for _ in range(S))
    R = int(rng.choice([8, 16, 32, 64, 128]))
    slots = int(rng.integers(1, 40))
    ranks = [int(rng.integers(0, R + 1)) for _ in range(slots)]
    p = 1.0 / np.arange(1, slots + 1) ** float(rng.choice([0.0, 1.2]))
    ts = rng.choice(slots, size=T, p=p / p.sum())
    ts[rng.random(T) < 0.05] = -1
    log(f"random fused linear {seed} fused={fused}: T={T} in={in_f} out={widths} R={R} "
        f"slots={slots}")
    wl = W.make_workload(name="random_fused_linear", dtype="bf16", T=T, in_features=in_f,
                         out_slices=widths, R=R, slots=slots, ranks=ranks,
                         scalings=rng.uniform(0.5, 2.0, size=slots), token_slot=ts, seed=seed,
                         rng=rng)
    tg = wl.targets[0]
    w = W.base_weight(wl, tg)
    y = _run(wl, tg, w, fused)
    assert_tol(y, _reference(wl, tg, w), f"random fused linear {seed}")
