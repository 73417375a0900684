"""lora_apply_linear_noalloc (workspace in the library's static scratch
array) against lora_apply_linear (caller workspace) through the C ABI: two
calls in a row, the second on a smaller batch of another shape, each equal
bit for bit to lora_apply_linear on the same inputs and within the graded
bound of the oracle."""
import ctypes
import sys

import numpy as np
import pytest

import adapter_lora_serving_amd as L
import oracle as O
import workloads as W
from gpu_util import GpuTarget, assert_tol, f64, torch

pytestmark = pytest.mark.gpu


def _noalloc(g, y, addr):
    t = torch()
    tg, wl = g.tg, g.wl
    arr = (ctypes.c_int64 * tg.num_slices)(*tg.out_slices)
    return L.lib().lora_apply_linear_noalloc(
        1, g.x.data_ptr(), y.data_ptr(), wl.T, tg.in_features, ctypes.cast(arr, ctypes.c_void_p),
        tg.num_slices, g.a.data_ptr(), g.b.data_ptr(), wl.slots, wl.R,
        addr.token_order.data_ptr(), addr.slot_indptr.data_ptr(), g.ranks.data_ptr(),
        g.scal.data_ptr(), t.cuda.current_stream().cuda_stream)


def test_noalloc_matches_apply_linear():
    t = torch()
    cases = [
        ("decode qkv, 256 tokens", W.make_config(2, 4)),
        ("smaller: 40 tokens, 2 slices, 8 slots", W.make_config(
            2, 5, T=40, in_features=1024, slots=8, out_slices=(512, 256))),
    ]
    for what, wl in cases:
        print(f"noalloc case: {what}", flush=True)
        sys.stdout.flush()
        tg = wl.targets[0]
        g = GpuTarget(wl, tg)
        addr = g.addressing()
        y_na = g.y0.clone()
        assert _noalloc(g, y_na, addr) == 0
        need = L.workspace_bytes(wl.T, tg.in_features, wl.slots, tg.num_slices, wl.R)
        ws = t.zeros(need, dtype=t.uint8, device="cuda:0")
        y_ws = g.y0.clone()
        L.apply_linear_(g.x, y_ws, g.a, g.b, addr, g.ranks, g.scal, tg.out_slices, workspace=ws)
        t.cuda.synchronize()
        assert t.equal(y_na, y_ws), what
        _, y_ref = O.run_target(wl, tg)
        assert_tol(f64(y_na), y_ref, what)
