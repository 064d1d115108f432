"""Where each part of the model waits between passes: residency tiers.

"Why Weight Offloading Slows Inference" (section "Keeping some weights
close", Table 1) keeps some weights resident on the GPU or unpacked in RAM so
that they skip part of the read -> unpack -> copy path, and asks which weights
deserve the scarce space; "Memory requirements of language model inference on
a consumer GPU" (its conclusions) frames that as choosing, under GPU and
system-memory budgets, which weights stay in each tier. With the unpack on the
GPU, a unit (the embedding, a decoder layer, the head) can wait in one of four
places; every pass over the model (the weights one generated token needs)
then costs it:

  G   restored BF16 in HBM           nothing                      S bytes of HBM
  Gc  compressed in HBM              restore                      S_disk of HBM
  H   compressed in pinned RAM       copy (S_disk) + restore      S_disk of RAM
  D   compressed on disk             read + copy + restore        nothing

`plan` fills the budgets greedily by time saved per byte; `TieredPass` runs
one pass over a plan with the same overlap as the disk pipeline (a reader
thread ahead for D units, a copy stream for H and D units, restores on the
compute stream) and returns its wall time. Units restored each pass share two
output buffers; a pass ends with every unit restored once, in order.
"""
from __future__ import annotations

import time
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from . import afx
from .store import Store, _out_slot

TIERS = ("G", "Gc", "H", "D")


@dataclass
class Rates:
    """Measured costs: bytes per second of the read and the copy, seconds of
    restore per unit."""

    read_Bps: float
    copy_Bps: float
    restore_s: list


def unit_cost_s(tier: str, stored: int, restore_s: float, r: Rates) -> float:
    """Per-pass time of one unit in a tier if its steps ran back to back."""
    if tier == "G":
        return 0.0
    if tier == "Gc":
        return restore_s
    if tier == "H":
        return stored / r.copy_Bps + restore_s
    return stored / r.read_Bps + stored / r.copy_Bps + restore_s


def plan(store: Store, gpu_budget: int, host_budget: int, r: Rates) -> list:
    """Greedy tier choice: every unit starts on disk; repeatedly take the
    promotion (to a tier with more memory) that saves the most time per added
    byte of its memory, while the budget allows. GPU bytes count restored
    units at 2 bytes per value and compressed ones at their stored size."""
    n = len(store.units)
    stored = [u.bytes for u in store.units]
    full = [2 * sum(_out_slot(int(np.prod(t.shape))) for t in u.tensors) for u in store.units]
    tier = ["D"] * n
    gpu_used = host_used = 0

    def mem(t, i):
        return {"G": (full[i], 0), "Gc": (stored[i], 0), "H": (0, stored[i]), "D": (0, 0)}[t]

    while True:
        best = None
        for i in range(n):
            g0, h0 = mem(tier[i], i)
            c0 = unit_cost_s(tier[i], stored[i], r.restore_s[i], r)
            for t in TIERS[:TIERS.index(tier[i])]:
                g1, h1 = mem(t, i)
                dg, dh = g1 - g0, h1 - h0
                if gpu_used + dg > gpu_budget or host_used + dh > host_budget:
                    continue
                saved = c0 - unit_cost_s(t, stored[i], r.restore_s[i], r)
                added = max(dg, 0) + max(dh, 0)
                if saved <= 0:
                    continue
                score = saved / max(added, 1)
                if best is None or score > best[0]:
                    best = (score, i, t, dg, dh)
        if best is None:
            return tier
        _, i, t, dg, dh = best
        tier[i] = t
        gpu_used += dg
        host_used += dh


class TieredPass:
    """Hold a store's units in the tiers of a plan and run passes over them."""

    def __init__(self, store: Store, tiers: list, device="cuda", threads: int = 16, direct: bool = True):
        import torch

        self.torch = torch
        self.store = store
        self.tiers = list(tiers)
        self.dev = torch.device(device)
        self.threads = threads
        self.direct = direct
        units = store.units
        streamed = [i for i, t in enumerate(self.tiers) if t != "G"]
        moved = [i for i, t in enumerate(self.tiers) if t in ("H", "D")]
        max_vals = max([sum(_out_slot(int(np.prod(t.shape))) for t in units[i].tensors) for i in streamed] or [1])
        max_moved = max([units[i].bytes for i in moved] or [1])
        self.out = [torch.empty(max_vals, dtype=torch.int16, device=self.dev) for _ in range(2)]
        self.blob = [torch.empty(max_moved, dtype=torch.uint8, device=self.dev) for _ in range(2)]
        self.stage = [torch.empty(max_moved, dtype=torch.uint8, pin_memory=True)
                      for _ in range(3 if "D" in self.tiers else 0)]
        self.copy_stream = torch.cuda.Stream(self.dev)  # default priority
        self.resident_out = {}  # G: restored once, kept
        self.resident_blob = {}  # Gc: compressed in HBM
        self.host_blob = {}  # H: compressed in pinned RAM
        self.infos = {}
        for i, t in enumerate(self.tiers):
            u = units[i]
            if t == "D":
                continue
            host = torch.empty(u.bytes, dtype=torch.uint8, pin_memory=True)
            afx.afx_file_read(store.path, u.offset, u.bytes, host.data_ptr(), threads, direct)
            self.infos[i] = [afx.afx_query(host.data_ptr() + tt.offset, tt.bytes) for tt in u.tensors]
            if t == "H":
                self.host_blob[i] = host
                continue
            dev_blob = host.to(self.dev)
            if t == "Gc":
                self.resident_blob[i] = dev_blob
                continue
            out = torch.empty(sum(_out_slot(int(info.n_elems)) for info in self.infos[i]), dtype=torch.int16,
                              device=self.dev)
            afx.afx_decode_layer_async(self._jobs(i, dev_blob.data_ptr(), out.data_ptr()),
                                       torch.cuda.current_stream(self.dev).cuda_stream)
            torch.cuda.synchronize(self.dev)
            self.resident_out[i] = out
        torch.cuda.synchronize(self.dev)

    def _jobs(self, i, blob_ptr, out_ptr):
        oo, jobs = 0, []
        for info, t in zip(self.infos[i], self.store.units[i].tensors):
            m = int(info.n_elems)
            jobs.append((info, blob_ptr + t.offset, out_ptr + 2 * oo, 2 * m))
            oo += _out_slot(m)
        return afx.make_jobs(jobs)

    def hbm_bytes(self) -> int:
        held = [*self.resident_out.values(), *self.resident_blob.values(), *self.out, *self.blob]
        return sum(t.numel() * t.element_size() for t in held)

    def run(self, on_unit=None) -> float:
        """One pass; returns its wall time in seconds. ``on_unit(i, out)``
        sees every unit's restored values (it synchronizes: off the clock)."""
        torch = self.torch
        units = self.store.units
        n = len(units)
        main = torch.cuda.current_stream(self.dev)
        disk = [i for i in range(n) if self.tiers[i] == "D"]
        slot = {i: k for k, i in enumerate(disk)}
        copied = {i: torch.cuda.Event() for i in range(n) if self.tiers[i] in ("H", "D")}
        decoded = [torch.cuda.Event() for _ in range(n)]
        reader = ThreadPoolExecutor(max_workers=1)

        def read(k):
            i = disk[k]
            if k >= 3:
                copied[disk[k - 3]].synchronize()  # its staging buffer has been copied out
            u, h = units[i], self.stage[k % 3]
            afx.afx_file_read(self.store.path, u.offset, u.bytes, h.data_ptr(), self.threads, self.direct)
            return [afx.afx_query(h.data_ptr() + t.offset, t.bytes) for t in u.tensors]

        torch.cuda.synchronize(self.dev)
        t0 = time.perf_counter()
        futs = {k: reader.submit(read, k) for k in range(min(3, len(disk)))}
        b = 0  # ring position of the restored outputs and moved blobs
        last_use = [None, None]  # the unit that used each ring position last
        try:
            for i, u in enumerate(units):
                t = self.tiers[i]
                if t == "G":
                    if on_unit is not None:
                        on_unit(i, self.resident_out[i])
                    continue
                if t == "D":
                    k = slot[i]
                    self.infos[i] = futs.pop(k).result()
                    src = self.stage[k % 3]
                elif t == "H":
                    src = self.host_blob[i]
                if t in ("H", "D"):
                    with torch.cuda.stream(self.copy_stream):
                        if last_use[b] is not None:
                            self.copy_stream.wait_event(decoded[last_use[b]])  # blob slot b is free
                        self.blob[b][:u.bytes].copy_(src[:u.bytes], non_blocking=True)
                        copied[i].record(self.copy_stream)
                    if t == "D" and slot[i] + 3 < len(disk):
                        futs[slot[i] + 3] = reader.submit(read, slot[i] + 3)
                    main.wait_event(copied[i])
                    blob_ptr = self.blob[b].data_ptr()
                else:
                    blob_ptr = self.resident_blob[i].data_ptr()
                afx.afx_decode_layer_async(self._jobs(i, blob_ptr, self.out[b].data_ptr()), main.cuda_stream)
                decoded[i].record(main)
                last_use[b] = i
                if on_unit is not None:
                    decoded[i].synchronize()
                    on_unit(i, self.out[b])
                b ^= 1
            torch.cuda.synchronize(self.dev)
        finally:
            reader.shutdown(wait=True)
        return time.perf_counter() - t0
