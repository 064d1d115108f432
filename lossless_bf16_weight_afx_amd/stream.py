"""Layer-by-layer restore of a compressed model held in pinned host memory.

"Memory requirements of language model inference on a consumer GPU"
(section "Loading one part of the model at a time") runs a model larger than
the GPU by loading one part, using it and releasing it before the next;
"Why Weight Offloading Slows Inference" (section "Loading during
computation", Figure 2) hides the loading of layer i+1 behind the work on
layer i. Here the parts are the model's units (embedding, each decoder
layer, output head with the final norm), stored compressed in pinned host
memory. Two device buffers alternate: while unit i is restored on the
compute stream, unit i+1's compressed bytes are copied on a side stream.

The restore itself is libafx's afx_decode_layer_async (one launch per unit);
this module only moves buffers and orders streams with events.
"""
from __future__ import annotations

import time
from dataclasses import dataclass, field

import numpy as np

from . import afx, synth

ALIGN = 256


def _align(v: int) -> int:
    return (v + ALIGN - 1) // ALIGN * ALIGN


def _out_slot(n: int) -> int:
    """Elements reserved for an n-element output (keeps every output 256-byte aligned)."""
    return (n + 127) // 128 * 128


@dataclass
class Unit:
    """One streamed part: its tensors' blobs packed in one pinned buffer."""

    name: str
    specs: list
    host: object  # torch uint8 tensor in pinned memory holding all blobs
    offsets: list  # byte offset of each tensor's blob in `host`
    infos: list  # afx_info of each blob
    n_values: int
    blob_bytes: int
    raw: list = field(default_factory=list)  # original bits (optional, for checks)


def build_unit(name: str, specs, threads: int = 0, keep_raw: bool = False) -> Unit:
    """Generate the unit's tensors and encode them into one pinned buffer."""
    import torch

    xs, plans = [], []
    for sp in specs:
        x = synth.generate(sp, threads=threads or None)
        xs.append(x)
        plans.append(afx.afx_encode_plan(x, threads))
    offsets, off = [], 0
    for plan in plans:
        offsets.append(off)
        off = _align(off + plan[2])
    host = torch.empty(max(off, ALIGN), dtype=torch.uint8, pin_memory=True)
    base = host.data_ptr()
    infos = []
    for sp, x, o, plan in zip(specs, xs, offsets, plans):
        nbytes = plan[2]
        n = afx.afx_encode(x, sp.shape, threads=threads, out=(base + o, nbytes), plan=plan)
        assert n == nbytes
        infos.append(afx.afx_query(base + o, nbytes))
    return Unit(name, list(specs), host, offsets, infos, sum(x.size for x in xs), off,
                raw=xs if keep_raw else [])


def build_model(units_specs, threads: int = 0, keep_raw: bool = False, progress=None) -> list:
    out = []
    for i, specs in enumerate(units_specs):
        t0 = time.time()
        name = specs[0].name.split(".")[0] if len(specs) == 1 else specs[0].name.rsplit(".", 1)[0]
        u = build_unit(name, specs, threads, keep_raw)
        out.append(u)
        if progress:
            progress(f"[store] unit {i + 1}/{len(units_specs)} {u.name}: {u.n_values} values, "
                     f"{u.blob_bytes} B compressed, {time.time() - t0:.1f}s")
    return out


class Streamer:
    """Double-buffered copy-then-restore of a list of units on one GPU."""

    def __init__(self, units, device="cuda"):
        import torch

        self.torch = torch
        self.units = units
        self.dev = torch.device(device)
        max_blob = max(u.blob_bytes for u in units)
        max_vals = max(sum(_out_slot(int(i.n_elems)) for i in u.infos) for u in units)
        self.blob = [torch.empty(max_blob, dtype=torch.uint8, device=self.dev) for _ in range(2)]
        self.out = [torch.empty(max_vals, dtype=torch.int16, device=self.dev) for _ in range(2)]
        self.copy_stream = torch.cuda.Stream(self.dev)  # default priority
        self.jobs = []
        for u in units:
            per_buf = []
            for b in range(2):
                oo, js = 0, []
                for info, off in zip(u.infos, u.offsets):
                    n = int(info.n_elems)
                    js.append((info, self.blob[b].data_ptr() + off, self.out[b].data_ptr() + 2 * oo, 2 * n))
                    oo += _out_slot(n)
                per_buf.append(afx.make_jobs(js))
            self.jobs.append(per_buf)

    def run(self, on_unit=None, snapshot=None) -> dict:
        """Stream every unit once. ``on_unit(i, unit, out_tensor)`` is called
        after unit i is restored (it synchronizes; use only off the clock).
        ``snapshot`` (a list of device int16 tensors, one of unit_slots(u)
        elements per unit) receives a device-to-device copy of every unit's
        restored output, ordered after its restore on the compute stream with
        no host wait, so a pass that runs free (copies overlapping restores)
        can be checked unit by unit afterwards."""
        torch = self.torch
        n = len(self.units)
        main = torch.cuda.current_stream(self.dev)
        ev = lambda: torch.cuda.Event(enable_timing=True)
        copied = [ev() for _ in range(n)]
        dec_start = [ev() for _ in range(n)]
        decoded = [ev() for _ in range(n)]
        start = ev()
        torch.cuda.synchronize(self.dev)
        start.record(main)
        self.copy_stream.wait_event(start)
        for i, u in enumerate(self.units):
            b = i % 2
            with torch.cuda.stream(self.copy_stream):
                if i >= 2:
                    self.copy_stream.wait_event(decoded[i - 2])  # buffer b is free again
                self.blob[b][:u.blob_bytes].copy_(u.host[:u.blob_bytes], non_blocking=True)
                copied[i].record(self.copy_stream)
            main.wait_event(copied[i])
            dec_start[i].record(main)
            afx.afx_decode_layer_async(self.jobs[i][b], main.cuda_stream)
            decoded[i].record(main)
            if snapshot is not None:
                # on the compute stream: the restore of unit i + 2 into the
                # same buffer is ordered after this read
                snapshot[i].copy_(self.out[b][:snapshot[i].numel()], non_blocking=True)
            if on_unit is not None:
                decoded[i].synchronize()
                on_unit(i, u, self.out[b])
        torch.cuda.synchronize(self.dev)
        e2e_ms = start.elapsed_time(decoded[-1])
        dec_ms = [s.elapsed_time(e) for s, e in zip(dec_start, decoded)]
        return {"e2e_ms": e2e_ms, "decode_ms": dec_ms, "restored_bytes": 2 * sum(u.n_values for u in self.units),
                "blob_bytes": sum(u.blob_bytes for u in self.units)}

    def link_copy_ms(self) -> float:
        """Time plain pinned-to-device copies of every unit's compressed bytes."""
        torch = self.torch
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(self.dev)
        s.record(self.copy_stream)
        with torch.cuda.stream(self.copy_stream):
            for i, u in enumerate(self.units):
                self.blob[i % 2][:u.blob_bytes].copy_(u.host[:u.blob_bytes], non_blocking=True)
        e.record(self.copy_stream)
        torch.cuda.synchronize(self.dev)
        return s.elapsed_time(e)


def unit_slots(u: Unit) -> int:
    """Output elements a unit occupies (every tensor's output 256-byte aligned)."""
    return sum(_out_slot(int(i.n_elems)) for i in u.infos)


def check_unit_regen(u: Unit, out, threads: int = 0) -> bool:
    """Bit-exact check of a restored unit against its original bits,
    generated again from the unit's seeded specs one tensor at a time (host
    memory stays at one tensor)."""
    import torch

    off, ok = 0, True
    for sp in u.specs:
        x = synth.generate(sp, threads=threads or None)
        ref = torch.from_numpy(x.view(np.int16)).to(out.device)
        ok &= bool(torch.equal(out[off:off + x.size], ref))
        del ref, x
        off += _out_slot(sp.numel)
    return ok


def check_unit(u: Unit, out) -> bool:
    """Bit-exact check of a restored unit against its original bits."""
    import torch

    off, ok = 0, True
    for x in u.raw:
        ref = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(out.device)
        ok &= bool(torch.equal(out[off:off + x.size], ref))
        off += _out_slot(x.size)
    return ok


def resident_decode(units, steps: int = 3, device="cuda", check: bool = False, reference=None,
                    warmup: int = 1, per_unit: bool = False, threads: int = 0) -> dict:
    """Restore the whole model with every unit's compressed bytes already in
    HBM, into one output region per unit (the restored model, ~29.5 GB, and
    the compressed one, ~20.5 GB, both fit in HBM): one afx_decode_layer_async
    call per unit, back to back on one stream. (Packing several layers into
    each 32-tensor launch is slower: mid-sized tensors then get too few or too
    many whole workgroups.)

    Returns milliseconds per whole-model pass (``steps`` passes between two
    events, after ``warmup`` passes) and, with ``check``, whether every unit
    came back bit-exact: against ``reference`` (a list of device int16
    tensors, one per unit, of unit_slots(u) elements, e.g. the snapshots of a
    checked streamed pass) when given, else against the raw bits kept in the
    units, else against bits generated again from the units' specs. With
    ``per_unit`` one more pass records an event between every two units and
    reports each unit's milliseconds."""
    import torch

    dev = torch.device(device)
    blobs = [u.host[:u.blob_bytes].to(dev) for u in units]
    slots = [unit_slots(u) for u in units]
    out = torch.empty(sum(slots), dtype=torch.int16, device=dev)
    calls, base = [], 0
    for k, u in enumerate(units):
        oo, jobs = base, []
        for info, off in zip(u.infos, u.offsets):
            n = int(info.n_elems)
            jobs.append((info, blobs[k].data_ptr() + off, out.data_ptr() + 2 * oo, 2 * n))
            oo += _out_slot(n)
        base += slots[k]
        calls.append(afx.make_jobs(jobs))
    s = torch.cuda.current_stream(dev)
    for arr in calls:  # first pass: the checked one
        afx.afx_decode_layer_async(arr, s.cuda_stream)
    torch.cuda.synchronize(dev)
    exact = None
    if check:
        exact, base = True, 0
        for k, u in enumerate(units):
            got = out[base:base + slots[k]]
            if reference is not None:
                exact &= bool(torch.equal(got, reference[k][:slots[k]]))
            elif u.raw:
                exact &= check_unit(u, got)
            else:
                exact &= check_unit_regen(u, got, threads)
            base += slots[k]
    for _ in range(max(0, warmup - 1)):
        for arr in calls:
            afx.afx_decode_layer_async(arr, s.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        for arr in calls:
            afx.afx_decode_layer_async(arr, s.cuda_stream)
    e1.record(s)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    unit_ms = None
    if per_unit:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
        evs[0].record(s)
        for k, arr in enumerate(calls):
            afx.afx_decode_layer_async(arr, s.cuda_stream)
            evs[k + 1].record(s)
        torch.cuda.synchronize(dev)
        unit_ms = [evs[k].elapsed_time(evs[k + 1]) for k in range(len(calls))]
    del blobs, out
    launches = sum((len(a) + afx.MAX_JOBS_PER_LAUNCH - 1) // afx.MAX_JOBS_PER_LAUNCH for a in calls)
    return {"ms": ms, "launches": launches, "bit_exact": exact, "unit_ms": unit_ms}
