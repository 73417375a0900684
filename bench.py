#!/usr/bin/env python3
"""Throughput of the batched multi-LoRA delta on one MI355X.

A step is one pass of the whole hot path over one batch: the device-side
addressing build, then the fused shrink + expand (lora_apply_linear) of a
linear target, or gather_shrink + expand of an embedding target. Where the
library does both in one launch (lora_apply_linear_from_slots: a bf16 batch
of at most 1024 tokens over at most 63 slots) the step is that one call,
which also writes the addressing for the step's later targets; an
expert-sorted batch likewise (lora_apply_linear_from_experts: fewer than 1024
rows, at most 63 experts and 1023 pool entries). The default
workload is the decode BGMV batch: T=256 tokens, one per request, in=4096,
fused q/k/v out_slices (4096, 1024, 1024), 32 adapter slots with ranks in
{8, 16} (R=16), scaling 2, bf16, seeded synthetic data. `--config 3|4|5`
times the prefill, embedding and skewed-mix batches the same way.

Timing: the inputs of `--sets` independent buffer sets are resident in HBM
(more than 1 GiB in total, so the 256 MB Infinity Cache cannot serve them);
step i uses set i mod sets. The K timed steps are recorded once in a hipGraph
(through torch.cuda.CUDAGraph) and replayed once between two synchronisations,
so host launch overhead is not measured. The dominant kernel's average launch
duration: the step's own where it is one launch, else HIP events around a
second graph that launches only the apply (lora_apply_linear, or
gather_shrink + expand) K times on the same stream. The addressing alone,
the apply alone and (for a one-launch step) the two-launch step are timed
the same way and reported beside it.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402
from adapter_lora_serving_amd.roofline import BF16_MFMA_PEAK_TFLOPS, HBM_PEAK_GBS, workload_cost  # noqa: E402

PROFILE_DIR = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "adapter_lora_serving_amd", "csrc")


def kernel_sources():
    """Every device and launch source of the library (all of csrc/)."""
    return sorted(n for n in os.listdir(CSRC)
                  if n.endswith((".hip", ".h", ".cpp")))


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the device and launch sources with comments and blank space
    removed, so that a comment edit does not invalidate recorded counters."""
    import re
    h = hashlib.sha256()
    for name in kernel_sources():
        p = os.path.join(CSRC, name)
        if os.path.exists(p):
            text = open(p, encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
            text = "\n".join(l.strip() for l in text.splitlines() if l.strip())
            h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the kernel sources as they are now; else None. `workload` is the
    workload name, with the target appended for a multi-target workload."""
    p = os.path.join(PROFILE_DIR, f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def host_info():
    """CPU model, the CPUs this process may run on, and the BLAS build the
    oracle's matrix products use (threads, library, version)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    blas = {}
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            i = max(info, key=lambda d: int(d.get("num_threads", 1)))
            blas = {"library": i.get("internal_api"), "version": i.get("version"),
                    "threads": int(i.get("num_threads", 1)),
                    "threading": i.get("threading_layer"),
                    "arch": i.get("architecture")}
    except Exception:
        pass
    return model, affinity, blas


def cpu_baseline(wl, tg, budget_s: float):
    """The fp64 CPU oracle as it stands, on the same batch, for ~budget_s."""
    import oracle as O
    model, affinity, blas = host_info()
    threads = blas.get("threads", affinity)
    ex = getattr(wl, "experts", None)
    if wl.token_slot is None and ex is not None:
        # rows of an expert-sorted batch: the oracle's own key of each row
        wl = W.with_token_slot(wl, O.expert_keys(ex["row_slot"], ex["offsets"], ex["experts"],
                                                 ex["slots"]))
    runs = 0
    t0 = time.perf_counter()
    while True:
        O.run_target(wl, tg)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": round(wl.T * runs / el, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"the full {wl.T}-token batch of the same workload, {runs} oracle runs "
                      f"(fp64 NumPy, bf16 decode included) in {el:.1f} s",
            "cpu_model": model, "affinity_cpus": int(affinity), "blas": blas}


def _graph_timer(torch, stream):
    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for i in range(n):
                    fn(i)
        torch.cuda.synchronize()
        return g

    def timed(g):
        g.replay()
        torch.cuda.synchronize()
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            st.record(stream)
            g.replay()
            en.record(stream)
        torch.cuda.synchronize()
        return st.elapsed_time(en)

    return capture, timed


def run_fused_linear(args, torch, L, dev):
    """The base projection of a linear target with the LoRA delta fused into
    its epilogue (lora_fused_column_linear: the shrink into the workspace,
    then the MFMA GEMM whose epilogue adds the delta), against the same GEMM
    followed by lora_apply_linear, and against the library GEMM (torch.matmul,
    hipBLASLt) followed by lora_apply_linear. A step is one addressing build
    plus one fused call."""
    config = args.config if args.config != 2 or args.target else 3
    wl = W.make_config(config, seed=0)
    tg = wl.target(args.target or ("gate_up" if config == 3 else None))
    w_host = W.base_weight(wl, tg)
    alg_bytes_lora, lora_flops, _ = workload_cost(wl, tg)
    T, in_f, out = wl.T, tg.in_features, tg.out_features
    base_flops = 2 * T * in_f * out
    flops = base_flops + lora_flops
    # minimum HBM bytes of the fused call: x, W, A and B of the used slots,
    # y written once, metadata
    e = 2
    min_bytes = e * (T * in_f + out * in_f + T * out) + alg_bytes_lora - 2 * e * T * out - e * T * in_f

    def d(arr):
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(dev)

    ranks = torch.from_numpy(wl.ranks).to(dev)
    scal = torch.from_numpy(wl.scalings).to(dev)
    ts = torch.from_numpy(wl.token_slot.astype(np.int32)).to(dev)
    set_bytes = e * (T * in_f + out * in_f + T * out) + (tg.a.size + tg.b.size) * e
    n_sets = args.sets or int(min(16, max(2, math.ceil(1.1 * 2 ** 30 / set_bytes))))
    eprint(f"fused_linear {wl.name}/{tg.name}: T={T} in={in_f} out={tg.out_slices} R={wl.R} "
           f"slots={wl.slots}; {base_flops / 1e9:.1f} GFLOP base + {lora_flops / 1e9:.2f} GFLOP "
           f"delta; {n_sets} buffer sets x {set_bytes / 1e6:.0f} MB")
    x0, w0, a0, b0 = d(tg.x), d(w_host), d(tg.a), d(tg.b)
    sets = []
    for i in range(n_sets):
        s = dict(x=x0.clone(), w=w0.clone(), a=a0.clone(), b=b0.clone(),
                 y=torch.empty(T, out, dtype=torch.bfloat16, device=dev), ts=ts.clone())
        s["addr"] = L.build_addressing(s["ts"], wl.slots)
        sets.append(s)
    del x0, w0, a0, b0
    need = int(L.lib().lora_fused_column_linear_workspace_bytes(T, in_f, tg.num_slices, wl.R))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    wsa = torch.zeros(L.workspace_bytes(T, in_f, wl.slots, tg.num_slices, wl.R),
                      dtype=torch.uint8, device=dev)

    def fused(i):
        s = sets[i % n_sets]
        L.fused_column_linear(s["x"], s["w"], s["a"], s["b"], s["addr"], ranks, scal,
                              tg.out_slices, y=s["y"], workspace=ws)

    def step(i):
        s = sets[i % n_sets]
        L.build_addressing(s["ts"], wl.slots, out=s["addr"])
        fused(i)

    def base_only(i):
        s = sets[i % n_sets]
        L.column_linear(s["x"], s["w"], tg.out_slices, y=s["y"])

    def unfused(i):
        s = sets[i % n_sets]
        L.column_linear(s["x"], s["w"], tg.out_slices, y=s["y"])
        L.apply_linear_(s["x"], s["y"], s["a"], s["b"], s["addr"], ranks, scal, tg.out_slices,
                        workspace=wsa)

    def lib_base(i):
        s = sets[i % n_sets]
        torch.matmul(s["x"], s["w"].t(), out=s["y"])

    def lib_unfused(i):
        lib_base(i)
        s = sets[i % n_sets]
        L.apply_linear_(s["x"], s["y"], s["a"], s["b"], s["addr"], ranks, scal, tg.out_slices,
                        workspace=wsa)

    legs = [("step", step), ("fused", fused)]
    if not args.no_compare:
        legs += [("base", base_only), ("unfused", unfused), ("lib_base", lib_base),
                 ("lib_unfused", lib_unfused)]
    for i in range(args.warmup):
        for _, fn in legs[1:] if len(legs) > 2 else legs:
            fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    capture, timed = _graph_timer(torch, stream)
    K = args.steps
    ms = {}
    for name, fn in legs:
        g = capture(fn, K)
        ms[name] = timed(g) / K
        del g
    us = {k: round(v * 1e3, 2) for k, v in ms.items()}
    tf = flops / (ms["fused"] * 1e-3) / 1e12
    tf_base = base_flops / (ms["base"] * 1e-3) / 1e12 if "base" in ms else None
    eprint(f"per call (us): {us}; fused {tf:.0f} TFLOP/s, base GEMM alone {tf_base} TFLOP/s")
    result = {
        "metric": "LoRA-delta tokens/sec + achieved HBM GB/s (decode) / MFMA util (prefill)",
        "value": round(T / (ms["step"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms["step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian inputs and base weights, no trained adapters)",
        "config": {"workload": "fused_linear_" + wl.name, "target": tg.name, "T": T,
                   "in": in_f, "out_slices": list(tg.out_slices), "R": wl.R,
                   "slots": wl.slots, "buffer_sets": n_sets},
        "roofline": {
            "bound": "mfma",
            "kernel": "lora_fused_column_linear",
            "achieved": round(tf, 1),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(f"fused_linear_{wl.name}_{tg.name}"),
            "algorithmic_flops_per_launch": int(flops),
            "min_hbm_bytes_per_launch": int(min_bytes),
            "avg_launch_us": us["fused"],
        },
        "per_call_us": {"fused (shrink + GEMM with the delta in its epilogue)": us["fused"],
                        "GEMM alone (lora_column_linear)": us.get("base"),
                        "GEMM then lora_apply_linear": us.get("unfused"),
                        "torch.matmul alone": us.get("lib_base"),
                        "torch.matmul then lora_apply_linear": us.get("lib_unfused")},
        "gemm_tflops": None if tf_base is None else round(tf_base, 1),
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="synthetic workload 1-5 (default 2)")
    ap.add_argument("--target", default=None, help="target name for multi-target workloads")
    ap.add_argument("--workload", choices=["router_fold", "tp8_qkv_decode", "tp8_prefill",
                                           "moe_experts", "fused_linear"],
                    default=None,
                    help="a workload beyond the five configs: router_fold (a router LoRA "
                         "folded onto 64 routing logits, decode batch); tp8_qkv_decode, "
                         "tp8_prefill (one GPU's share of a TP=8 projection; --target "
                         "gate_up or down for the latter); moe_experts (the routed-expert "
                         "LoRA on 512 expert-sorted rows, its addressing by (expert, slot); "
                         "--target expert_gate_up or expert_down); fused_linear (the base "
                         "projection x @ W^T of --config/--target with the LoRA delta in its "
                         "epilogue, lora_fused_column_linear; default config 3 gate_up)")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets (0: enough for >1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="fused_linear: time the fused call only (for profiling its kernels)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import adapter_lora_serving_amd as L

    if not torch.cuda.is_available():
        eprint("bench.py needs a GPU: the LoRA delta has no CPU path")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.workload == "fused_linear":
        return run_fused_linear(args, torch, L, dev)
    if args.workload == "router_fold":
        wl = W.make_router_fold(0)
    elif args.workload == "moe_experts":
        wl = W.make_moe_experts(0)
    elif args.workload in W.TP_SHARES:
        wl = W.make_tp_share(args.workload, 0)
    else:
        wl = W.make_config(args.config, seed=0)
    tg = wl.target(args.target)
    alg_bytes, alg_flops, terms = workload_cost(wl, tg)
    eb = 2 if wl.dtype == "bf16" else 4
    x_bytes = tg.ids.size * 4 if tg.embedding else tg.x.size * eb
    set_bytes = x_bytes + (tg.a.size + tg.b.size + tg.y0.size) * eb
    n_sets = args.sets or int(min(64, max(2, math.ceil(1.1 * 2 ** 30 / set_bytes))))
    eprint(f"workload {wl.name}/{tg.name}: T={wl.T} in={tg.in_features} out={tg.out_slices} "
           f"R={wl.R} slots={wl.slots}; algorithmic {alg_bytes / 1e6:.2f} MB/call "
           f"{terms}; {n_sets} buffer sets x {set_bytes / 1e6:.1f} MB")

    def d(arr):
        if wl.dtype == "bf16":
            return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(arr).to(dev)

    ranks = torch.from_numpy(wl.ranks).to(dev)
    scal = torch.from_numpy(wl.scalings).to(dev)
    ts_host = (None if wl.token_slot is None
               else torch.from_numpy(wl.token_slot.astype(np.int32)))
    sets = []
    if tg.embedding:
        x0 = torch.from_numpy(tg.ids.astype(np.int32)).to(dev)
    else:
        x0 = d(tg.x)
    a0, b0, y0 = d(tg.a), d(tg.b), d(tg.y0)
    ex = getattr(wl, "experts", None)

    def addressing(s, out=None):
        if ex is None:
            return L.build_addressing(s["ts"], wl.slots, out=out)
        # rows of an expert-sorted batch: grouped by (expert, slot) on the device
        return L.build_addressing_experts(s["rs"], s["offs"], ex["experts"], ex["slots"], out=out)

    for i in range(n_sets):
        s = dict(x=x0.clone(), a=a0.clone(), b=b0.clone(), y=y0.clone(),
                 ts=None if ts_host is None else ts_host.to(dev))
        if ex is not None:
            s["rs"] = torch.from_numpy(ex["row_slot"]).to(dev)
            s["offs"] = torch.from_numpy(ex["offsets"]).to(dev)
        s["addr"] = addressing(s)
        sets.append(s)
    del x0, a0, b0, y0
    if tg.embedding:
        h = torch.empty(wl.T, wl.R, dtype=torch.float32, device=dev)
    else:
        need = L.workspace_bytes(wl.T, tg.in_features, wl.slots, tg.num_slices, wl.R)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)

    def apply_only(i):
        s = sets[i % n_sets]
        if tg.embedding:
            L.gather_shrink(s["x"], s["a"], s["addr"], ranks, out=h)
            L.expand_(h, s["b"], s["addr"], ranks, scal, s["y"], tg.out_slices)
        else:
            L.apply_linear_(s["x"], s["y"], s["a"], s["b"], s["addr"], ranks, scal,
                            tg.out_slices, workspace=ws)

    # The first linear target of a small batch builds the step's addressing
    # in its own launch (lora_apply_linear_from_slots): the step is then one
    # kernel, which also writes token_order and slot_indptr for the step's
    # later targets. Elsewhere the addressing kernel runs first.
    # (lora_apply_linear_from_experts likewise for an expert-sorted batch)
    code = 1 if wl.dtype == "bf16" else 0
    if tg.embedding:
        one_launch = False
    elif ex is None:
        one_launch = L.from_slots_one_launch(code, wl.T, tg.in_features, tg.out_slices,
                                             wl.slots, wl.R)
    else:
        one_launch = L.from_experts_one_launch(code, wl.T, tg.in_features, tg.out_slices,
                                               ex["experts"], ex["slots"], wl.R)
    if one_launch:
        if ex is None:
            need_fs = int(L.lib().lora_apply_linear_from_slots_workspace_bytes(
                wl.T, tg.in_features, wl.slots, tg.num_slices, wl.R))
        else:
            need_fs = int(L.lib().lora_apply_linear_from_experts_workspace_bytes(
                wl.T, tg.in_features, ex["experts"], ex["slots"], tg.num_slices, wl.R))
        ws_fs = torch.zeros(max(need_fs, 256), dtype=torch.uint8, device=dev)

    def step_two_launch(i):
        s = sets[i % n_sets]
        addressing(s, out=s["addr"])
        apply_only(i)

    def step(i):
        if not one_launch:
            return step_two_launch(i)
        s = sets[i % n_sets]
        if ex is None:
            L.apply_linear_from_slots_(s["x"], s["y"], s["a"], s["b"], s["ts"], ranks, scal,
                                       tg.out_slices, out=s["addr"], workspace=ws_fs)
        else:
            L.apply_linear_from_experts_(s["x"], s["y"], s["a"], s["b"], s["rs"], s["offs"],
                                         ex["experts"], ex["slots"], ranks, scal,
                                         tg.out_slices, out=s["addr"], workspace=ws_fs)

    def addr_only(i):
        s = sets[i % n_sets]
        addressing(s, out=s["addr"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for i in range(n):
                    fn(i)
        torch.cuda.synchronize()
        return g

    K = args.steps
    g_step = capture(step, K)
    g_apply = capture(apply_only, K)
    g_addr = capture(addr_only, K)
    g_two = capture(step_two_launch, K) if one_launch else None

    def timed(g):
        g.replay()                     # untimed replay: graph upload, caches of the code
        torch.cuda.synchronize()
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            st.record(stream)
            g.replay()
            en.record(stream)
        torch.cuda.synchronize()
        return st.elapsed_time(en)     # ms

    ms_total = timed(g_step)
    ms_step = ms_total / K
    ms_apply = timed(g_apply) / K
    ms_addr = timed(g_addr) / K
    ms_two = timed(g_two) / K if one_launch else None
    # the dominant kernel: the step's one launch (it also reads the slot ids,
    # counted in the metadata term, and the expert bounds, and writes the
    # addressing), else the apply
    if one_launch:
        ms_kernel = ms_step
        kernel_bytes = alg_bytes + 4 * wl.T + 4 * (wl.slots + 1)
        if ex is not None:
            kernel_bytes += 4 * (ex["experts"] + 1)
    else:
        ms_kernel = ms_apply
        kernel_bytes = alg_bytes

    # sanity denominator: a plain device copy of 1 GiB
    src = torch.empty(2 ** 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    for _ in range(5):
        dst.copy_(src)
    en.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * src.numel() * 4 / (st.elapsed_time(en) * 1e-3) / 1e9
    del src, dst

    # the same number of bytes moved by a plain device copy (half read, half
    # written), rotated over buffers that exceed the Infinity Cache, timed the
    # same way: what a kernel with no dependences achieves at this size
    half = max(1, int(alg_bytes // 2) // 16)
    n_pairs = int(min(64, max(2, math.ceil(1.1 * 2 ** 30 / (2 * half * 16)))))
    pairs = [(torch.zeros(half, 4, dtype=torch.float32, device=dev),
              torch.empty(half, 4, dtype=torch.float32, device=dev)) for _ in range(n_pairs)]
    torch.cuda.synchronize()
    g_copy = capture(lambda i: pairs[i % n_pairs][1].copy_(pairs[i % n_pairs][0]), K)
    ms_copy = timed(g_copy) / K
    del g_copy, pairs

    # the per-launch floor on this stream: the same graph timing around K
    # launches of a one-element fill, a kernel with no work of its own
    one = torch.zeros(1, dtype=torch.float32, device=dev)
    g_nop = capture(lambda i: one.fill_(1.0), K)
    ms_nop = timed(g_nop) / K
    del g_nop, one

    achieved = kernel_bytes / (ms_kernel * 1e-3) / 1e9
    tokens_per_s = wl.T / (ms_step * 1e-3)
    eprint(f"step {ms_step * 1e3:.2f} us ({'one launch' if one_launch else 'two launches'}; "
           f"{achieved:.0f} GB/s algorithmic); addressing alone {ms_addr * 1e3:.2f} us, apply "
           f"alone {ms_apply * 1e3:.2f} us"
           + (f", addressing then apply {ms_two * 1e3:.2f} us" if one_launch else "")
           + f"; device copy {copy_gbs:.0f} GB/s; a copy of the same bytes "
           f"{ms_copy * 1e3:.2f} us; an empty launch {ms_nop * 1e3:.2f} us")

    result = {
        "metric": "LoRA-delta tokens/sec + achieved HBM GB/s (decode) / MFMA util (prefill)",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Gaussian inputs, no trained adapters)",
        "config": {"workload": wl.name, "target": tg.name, "T": wl.T,
                   "in": tg.in_features, "out_slices": list(tg.out_slices), "R": wl.R,
                   "slots": wl.slots, "buffer_sets": n_sets},
        "roofline": {
            "bound": "hbm",
            "kernel": ("lora_gather_shrink + lora_expand" if tg.embedding else
                       "lora_apply_linear" if not one_launch else
                       "lora_apply_linear_from_slots" if ex is None else
                       "lora_apply_linear_from_experts"),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(wl.name if len(wl.targets) == 1
                                        else f"{wl.name}_{tg.name}"),
            "algorithmic_bytes_per_launch": int(kernel_bytes),
            "avg_launch_us": round(ms_kernel * 1e3, 3),
        },
        "mfma_util": round(alg_flops / (ms_kernel * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12), 5),
        "addressing_us": round(ms_addr * 1e3, 3),
        "apply_only_us": round(ms_apply * 1e3, 3),
        "addressing_then_apply_us": round((ms_two if one_launch else ms_step) * 1e3, 3),
        "device_copy_gbs": round(copy_gbs, 1),
        "device_copy_same_bytes_us": round(ms_copy * 1e3, 3),
        "empty_launch_us": round(ms_nop * 1e3, 3),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, tg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
