"""Helpers for the GPU parity tests: move generated workloads to the device,
run the HIP path through the binding, and compare with the oracle."""
import numpy as np

import adapter_lora_serving_amd as L


def torch():
    import torch as _t
    return _t


def dev(arr, dtype):
    """numpy input (uint16 bf16 bits / float32 / int32) -> torch tensor on cuda:0."""
    t = torch()
    if dtype == "bf16":
        return t.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(t.bfloat16).to("cuda:0")
    return t.from_numpy(np.ascontiguousarray(arr)).to("cuda:0")


def f64(t):
    return t.detach().to(torch().float64).cpu().numpy()


class GpuTarget:
    """Device copies of one workload target, ready for the binding."""

    def __init__(self, wl, tg):
        t = torch()
        self.wl, self.tg = wl, tg
        self.token_slot = (None if wl.token_slot is None
                           else t.from_numpy(wl.token_slot.astype(np.int32)).to("cuda:0"))
        self.ranks = t.from_numpy(wl.ranks.astype(np.int32)).to("cuda:0")
        self.scal = t.from_numpy(wl.scalings.astype(np.float32)).to("cuda:0")
        self.a = dev(tg.a, wl.dtype)
        self.b = dev(tg.b, wl.dtype)
        self.y0 = dev(tg.y0, wl.dtype)
        self.x = None if tg.x is None else dev(tg.x, wl.dtype)
        self.ids = None if tg.ids is None else t.from_numpy(tg.ids.astype(np.int32)).to("cuda:0")

    def addressing(self):
        return L.build_addressing(self.token_slot, self.wl.slots)

    def run(self, fused=True, addr=None, y=None):
        """Returns (addressing, h or None, y)."""
        addr = self.addressing() if addr is None else addr
        y = self.y0.clone() if y is None else y
        h = None
        if self.tg.embedding:
            h = L.gather_shrink(self.ids, self.a, addr, self.ranks)
            L.expand_(h, self.b, addr, self.ranks, self.scal, y, self.tg.out_slices)
        elif fused:
            L.apply_linear_(self.x, y, self.a, self.b, addr, self.ranks, self.scal,
                            self.tg.out_slices)
        else:
            h = L.shrink(self.x, self.a, addr, self.ranks, self.tg.num_slices)
            L.expand_(h, self.b, addr, self.ranks, self.scal, y, self.tg.out_slices)
        torch().cuda.synchronize()
        return addr, h, y


def unread_mask(wl, num_slices):
    """bool [T, S*R]: entries of h the expand never reads."""
    T, R = wl.T, wl.R
    m = np.ones((T, num_slices * R), dtype=bool)
    for t in range(T):
        s = int(wl.token_slot[t])
        if 0 <= s < wl.slots:
            r = int(min(max(int(wl.ranks[s]), 0), R))
            for i in range(num_slices):
                m[t, i * R:i * R + r] = False
    return m


def assert_tol(gpu, ref, what="", atol=1e-2, rtol=1e-2):
    from oracle import within_tolerance
    ok, worst = within_tolerance(gpu, ref, atol=atol, rtol=rtol)
    assert ok, f"{what}: max |gpu-oracle|/({atol:g}+{rtol:g}|oracle|) = {worst:.3f}"
    return worst
