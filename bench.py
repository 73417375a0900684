#!/usr/bin/env python3
"""Throughput of the batched multi-LoRA delta on one MI355X.

A step is one pass of the whole hot path over one batch: the device-side
addressing build, then the fused shrink + expand (lora_apply_linear) of a
linear target, or gather_shrink + expand of an embedding target. The default
workload is the decode BGMV batch: T=256 tokens, one per request, in=4096,
fused q/k/v out_slices (4096, 1024, 1024), 32 adapter slots with ranks in
{8, 16} (R=16), scaling 2, bf16, seeded synthetic data. `--config 3|4|5`
times the prefill, embedding and skewed-mix batches the same way.

Timing: the inputs of `--sets` independent buffer sets are resident in HBM
(more than 1 GiB in total, so the 256 MB Infinity Cache cannot serve them);
step i uses set i mod sets. The K timed steps are recorded once in a hipGraph
(through torch.cuda.CUDAGraph) and replayed once between two synchronisations,
so host launch overhead is not measured. The dominant kernel's average launch
duration comes from HIP events around a second graph that launches only the
apply (lora_apply_linear, or gather_shrink + expand) K times on the same
stream.

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
KERNEL_SOURCES = ["lora_common.h", "lora_kernels.h", "fused.hip", "sgmv.hip", "shrink.hip", "expand.hip",
                  "lora_api.cpp"]


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the device and launch sources with comments and blank space
    removed, so that a comment edit does not invalidate recorded counters."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "adapter_lora_serving_amd", "csrc")
    for name in KERNEL_SOURCES:
        p = os.path.join(csrc, name)
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


def cpu_baseline(wl, tg, budget_s: float):
    """The fp64 CPU oracle as it stands, on the same batch, for ~budget_s."""
    import oracle as O
    threads = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
    except Exception:
        pass
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
                      f"(fp64 NumPy, bf16 decode included) in {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="synthetic workload 1-5 (default 2)")
    ap.add_argument("--target", default=None, help="target name for multi-target workloads")
    ap.add_argument("--workload", choices=["router_fold", "tp8_qkv_decode", "tp8_prefill",
                                           "moe_experts"],
                    default=None,
                    help="a workload beyond the five configs: router_fold (a router LoRA "
                         "folded onto 64 routing logits, decode batch); tp8_qkv_decode, "
                         "tp8_prefill (one GPU's share of a TP=8 projection; --target "
                         "gate_up or down for the latter); moe_experts (the routed-expert "
                         "LoRA on 512 expert-sorted rows, its addressing by (expert, slot))")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets (0: enough for >1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import adapter_lora_serving_amd as L

    if not torch.cuda.is_available():
        eprint("bench.py needs a GPU: the LoRA delta has no CPU path")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

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
    ts_host = torch.from_numpy(wl.token_slot.astype(np.int32))
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
        s = dict(x=x0.clone(), a=a0.clone(), b=b0.clone(), y=y0.clone(), ts=ts_host.to(dev))
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

    def step(i):
        s = sets[i % n_sets]
        addressing(s, out=s["addr"])
        apply_only(i)

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

    achieved = alg_bytes / (ms_apply * 1e-3) / 1e9
    tokens_per_s = wl.T / (ms_step * 1e-3)
    eprint(f"step {ms_step * 1e3:.2f} us (addressing {ms_addr * 1e3:.2f} us, apply "
           f"{ms_apply * 1e3:.2f} us/launch = {achieved:.0f} GB/s algorithmic); device copy "
           f"{copy_gbs:.0f} GB/s; a copy of the same bytes {ms_copy * 1e3:.2f} us")

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
            "kernel": "lora_gather_shrink + lora_expand" if tg.embedding else "lora_apply_linear",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(wl.name if len(wl.targets) == 1
                                        else f"{wl.name}_{tg.name}"),
            "algorithmic_bytes_per_launch": int(alg_bytes),
            "avg_launch_us": round(ms_apply * 1e3, 3),
        },
        "mfma_util": round(alg_flops / (ms_apply * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12), 5),
        "addressing_us": round(ms_addr * 1e3, 3),
        "device_copy_gbs": round(copy_gbs, 1),
        "device_copy_same_bytes_us": round(ms_copy * 1e3, 3),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, tg, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
