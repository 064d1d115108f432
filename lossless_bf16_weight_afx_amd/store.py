"""A compressed model on disk, and its restore: read -> copy -> unpack.

"Why Weight Offloading Slows Inference" (section "The path from storage to
the GPU", Figure 1; section "Three steps for each weight", Eq. (1)) takes a
stored weight from the SSD into RAM, unpacks it and copies it over PCIe, and
prices the three steps as S_disk / b_disk + t_unpack + S / b_PCIe; the page
measures its reads with the page cache cleared. Here the compressed bytes
travel (RAM and PCIe carry S_disk, not S) and the unpack runs on the GPU, so
the three steps are read (S_disk / b_disk), copy (S_disk / b_link) and restore
(t_unpack). Section "Loading during computation" (Figure 2) overlaps the
loading of one part with the work on the one before; `DiskStreamer` keeps the
three steps of consecutive units in flight at once.

Store file ("AFXS", version 1), little-endian:
  [0, 4096)   magic "AFXS", u32 version 1, u64 index offset, u64 index bytes,
              u64 file bytes, zeros
  units       each unit's blobs packed at 256-byte offsets, the unit starting
              at a 4096-byte offset and padded to a multiple of 4096 bytes (a
              direct read of a unit then reads nothing around it)
  index       UTF-8 JSON at a 4096-byte offset: {"format": "afx-store",
              "version": 1, "units": [{"name", "offset", "bytes", "tensors":
              [{"name", "shape", "offset" (in the unit), "bytes"}]}]}
The restore itself is libafx's afx_decode_layer_async; the reads are libafx's
afx_file_read. This module only lays out files and orders the three steps.
"""
from __future__ import annotations

import json
import os
import struct
import time
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from . import afx, synth

MAGIC = b"AFXS"
VERSION = 1
PAGE = 4096
BLOB_ALIGN = 256
HEADER = struct.Struct("<4sIQQQ")


def _up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


@dataclass
class StoreTensor:
    name: str
    shape: tuple
    offset: int  # in the unit
    bytes: int


@dataclass
class StoreUnit:
    name: str
    offset: int  # in the file, multiple of 4096
    bytes: int  # multiple of 4096
    tensors: list

    @property
    def n_values(self) -> int:
        return sum(int(np.prod(t.shape)) for t in self.tensors)


@dataclass
class Store:
    path: str
    units: list
    file_bytes: int

    @property
    def blob_bytes(self) -> int:
        return sum(t.bytes for u in self.units for t in u.tensors)

    @property
    def restored_bytes(self) -> int:
        return 2 * sum(u.n_values for u in self.units)


def unit_name(specs) -> str:
    return specs[0].name.split(".")[0] if len(specs) == 1 else specs[0].name.rsplit(".", 1)[0]


def write_store(path: str, units_specs, threads: int = 0, progress=None) -> Store:
    """Generate and encode every unit (synthetic inputs) and write the store.
    The file is synced and its pages dropped from the page cache afterwards."""
    units, off = [], PAGE
    fd = os.open(path, os.O_WRONLY | os.O_CREAT | os.O_TRUNC, 0o644)
    try:
        for i, specs in enumerate(units_specs):
            t0 = time.time()
            xs = [synth.generate(sp, threads=threads or None) for sp in specs]
            plans = [afx.afx_encode_plan(x, threads) for x in xs]
            rel, tensors = 0, []
            for sp, plan in zip(specs, plans):
                tensors.append(StoreTensor(sp.name, tuple(sp.shape), rel, int(plan[2])))
                rel = _up(rel + int(plan[2]), BLOB_ALIGN)
            size = _up(max(rel, 1), PAGE)
            buf = np.zeros(size, np.uint8)
            for sp, x, plan, t in zip(specs, xs, plans, tensors):
                afx.afx_encode(x, sp.shape, threads=threads, out=(buf.ctypes.data + t.offset, t.bytes), plan=plan)
            del xs
            _pwrite_all(fd, memoryview(buf), off)
            units.append(StoreUnit(unit_name(specs), off, size, tensors))
            off += size
            if progress:
                progress(f"[store] unit {i + 1}/{len(units_specs)} {units[-1].name}: {size} B, {time.time() - t0:.1f}s")
        index = json.dumps({"format": "afx-store", "version": VERSION, "units": [
            {"name": u.name, "offset": u.offset, "bytes": u.bytes,
             "tensors": [{"name": t.name, "shape": list(t.shape), "offset": t.offset, "bytes": t.bytes}
                         for t in u.tensors]} for u in units]}).encode()
        _pwrite_all(fd, memoryview(index), off)
        file_bytes = off + len(index)
        header = HEADER.pack(MAGIC, VERSION, off, len(index), file_bytes).ljust(PAGE, b"\0")
        _pwrite_all(fd, memoryview(header), 0)
        os.fsync(fd)
        os.posix_fadvise(fd, 0, 0, os.POSIX_FADV_DONTNEED)
    finally:
        os.close(fd)
    return Store(path, units, file_bytes)


def _pwrite_all(fd: int, mv: memoryview, off: int) -> None:
    while len(mv):
        n = os.pwrite(fd, mv, off)
        mv, off = mv[n:], off + n


def open_store(path: str) -> Store:
    with open(path, "rb") as f:
        magic, version, ioff, ibytes, fbytes = HEADER.unpack(f.read(HEADER.size))
        if magic != MAGIC:
            raise ValueError(f"{path}: not an afx store")
        if version != VERSION:
            raise ValueError(f"{path}: store version {version}, expected {VERSION}")
        if os.fstat(f.fileno()).st_size < fbytes:
            raise ValueError(f"{path}: truncated store")
        f.seek(ioff)
        index = json.loads(f.read(ibytes))
    units = [StoreUnit(u["name"], int(u["offset"]), int(u["bytes"]),
                       [StoreTensor(t["name"], tuple(t["shape"]), int(t["offset"]), int(t["bytes"]))
                        for t in u["tensors"]]) for u in index["units"]]
    for u in units:
        if u.offset % PAGE or u.bytes % PAGE or u.offset + u.bytes > ioff:
            raise ValueError(f"{path}: unit {u.name} out of place")
        for t in u.tensors:
            if t.offset % BLOB_ALIGN or t.offset + t.bytes > u.bytes:
                raise ValueError(f"{path}: tensor {t.name} out of place")
    return Store(path, units, fbytes)


def _out_slot(n: int) -> int:
    return (n + 127) // 128 * 128  # keeps every output 256-byte aligned


class DiskStreamer:
    """Read, copy and restore the units of a store in order, three steps of
    consecutive units in flight at once: while unit i is restored on the
    compute stream, unit i+1 is copied on a side stream and units i+2 and
    i+3 are read from disk into pinned host memory by a reader thread."""

    N_HOST = 3  # pinned staging buffers
    N_DEV = 2  # device blob/output buffers

    def __init__(self, store: Store, device="cuda", threads: int = 16, direct: bool = True):
        import torch

        self.torch = torch
        self.store = store
        self.dev = torch.device(device)
        self.threads = threads
        self.direct = direct
        max_unit = max(u.bytes for u in store.units)
        max_vals = max(sum(_out_slot(int(np.prod(t.shape))) for t in u.tensors) for u in store.units)
        self.host = [torch.empty(max_unit, dtype=torch.uint8, pin_memory=True) for _ in range(self.N_HOST)]
        self.blob = [torch.empty(max_unit, dtype=torch.uint8, device=self.dev) for _ in range(self.N_DEV)]
        self.out = [torch.empty(max_vals, dtype=torch.int16, device=self.dev) for _ in range(self.N_DEV)]
        self.copy_stream = torch.cuda.Stream(self.dev)  # default priority

    def read_unit(self, i: int, h: int):
        """Read unit i into staging buffer h and validate its blobs (reader thread)."""
        u = self.store.units[i]
        t0 = time.perf_counter()
        afx.afx_file_read(self.store.path, u.offset, u.bytes, self.host[h].data_ptr(), self.threads, self.direct)
        t1 = time.perf_counter()
        infos = [afx.afx_query(self.host[h].data_ptr() + t.offset, t.bytes) for t in u.tensors]
        return infos, t1 - t0, time.perf_counter() - t1

    def run(self, on_unit=None) -> dict:
        """One pass over the store. ``on_unit(i, unit, out_tensor)`` runs after
        unit i is restored (it synchronizes; use only off the clock)."""
        torch = self.torch
        units = self.store.units
        n = len(units)
        main = torch.cuda.current_stream(self.dev)
        ev = lambda: torch.cuda.Event(enable_timing=True)
        copied = [ev() for _ in range(n)]
        decoded = [ev() for _ in range(n)]
        dec_start = [ev() for _ in range(n)]
        reader = ThreadPoolExecutor(max_workers=1)

        def read(i):
            if i >= self.N_HOST:
                copied[i - self.N_HOST].synchronize()  # its staging buffer has been copied out
            return self.read_unit(i, i % self.N_HOST)

        torch.cuda.synchronize(self.dev)
        t_start = time.perf_counter()
        futs = {i: reader.submit(read, i) for i in range(min(self.N_HOST, n))}
        read_s = check_s = wait_s = 0.0
        try:
            for i, u in enumerate(units):
                tw = time.perf_counter()
                infos, r_s, c_s = futs.pop(i).result()
                wait_s += time.perf_counter() - tw
                read_s += r_s
                check_s += c_s
                h, b = i % self.N_HOST, i % self.N_DEV
                with torch.cuda.stream(self.copy_stream):
                    if i >= self.N_DEV:
                        self.copy_stream.wait_event(decoded[i - self.N_DEV])  # device buffer b is free
                    self.blob[b][:u.bytes].copy_(self.host[h][:u.bytes], non_blocking=True)
                    copied[i].record(self.copy_stream)
                if i + self.N_HOST < n:
                    futs[i + self.N_HOST] = reader.submit(read, i + self.N_HOST)
                oo, jobs = 0, []
                for info, t in zip(infos, u.tensors):
                    m = int(info.n_elems)
                    jobs.append((info, self.blob[b].data_ptr() + t.offset, self.out[b].data_ptr() + 2 * oo, 2 * m))
                    oo += _out_slot(m)
                main.wait_event(copied[i])
                dec_start[i].record(main)
                afx.afx_decode_layer_async(afx.make_jobs(jobs), main.cuda_stream)
                decoded[i].record(main)
                if on_unit is not None:
                    decoded[i].synchronize()
                    on_unit(i, u, self.out[b])
            torch.cuda.synchronize(self.dev)
        finally:
            reader.shutdown(wait=True)
        e2e_s = time.perf_counter() - t_start
        # read_s: time in afx_file_read; validate_s: afx_query of every blob
        # (both on the reader thread); wait_s: time the launching thread waited
        # for a unit's bytes
        return {"e2e_s": e2e_s, "read_s": read_s, "validate_s": check_s, "wait_s": wait_s,
                "decode_ms": [s.elapsed_time(e) for s, e in zip(dec_start, decoded)],
                "restored_bytes": self.store.restored_bytes, "stored_bytes": sum(u.bytes for u in units)}

    def read_only_s(self) -> float:
        """Time reading every unit from disk into pinned memory, nothing else."""
        t0 = time.perf_counter()
        for i, u in enumerate(self.store.units):
            afx.afx_file_read(self.store.path, u.offset, u.bytes, self.host[i % self.N_HOST].data_ptr(),
                              self.threads, self.direct)
        return time.perf_counter() - t0

    def copy_only_s(self) -> float:
        """Time copying every unit's stored bytes from pinned memory to the GPU
        on the side stream, nothing else (the contents are whatever the
        staging buffers hold)."""
        torch = self.torch
        torch.cuda.synchronize(self.dev)
        t0 = time.perf_counter()
        with torch.cuda.stream(self.copy_stream):
            for i, u in enumerate(self.store.units):
                self.blob[i % self.N_DEV][:u.bytes].copy_(self.host[i % self.N_HOST][:u.bytes], non_blocking=True)
        torch.cuda.synchronize(self.dev)
        return time.perf_counter() - t0


class HostUnpackStreamer:
    """The pages' placement of the unpack, for comparison: read each unit
    from disk into pinned memory (reader thread, two units ahead), restore it
    on the host into a pinned BF16 buffer with afx_decode_host, and copy the
    restored bytes (S, not S_disk) to the GPU on a side stream while the next
    unit is being restored."""

    N_HOST = 3  # pinned staging buffers for stored bytes
    N_OUT = 2  # pinned BF16 buffers and device outputs

    def __init__(self, store: Store, device="cuda", read_threads: int = 16, unpack_threads: int = 16,
                 direct: bool = True):
        import torch

        self.torch = torch
        self.store = store
        self.dev = torch.device(device)
        self.read_threads = read_threads
        self.unpack_threads = unpack_threads
        self.direct = direct
        max_unit = max(u.bytes for u in store.units)
        max_vals = max(sum(_out_slot(int(np.prod(t.shape))) for t in u.tensors) for u in store.units)
        self.host = [torch.empty(max_unit, dtype=torch.uint8, pin_memory=True) for _ in range(self.N_HOST)]
        self.host_out = [torch.empty(max_vals, dtype=torch.int16, pin_memory=True) for _ in range(self.N_OUT)]
        self.out = [torch.empty(max_vals, dtype=torch.int16, device=self.dev) for _ in range(self.N_OUT)]
        self.copy_stream = torch.cuda.Stream(self.dev)  # default priority

    def run(self, on_unit=None) -> dict:
        """One pass; ``on_unit(i, unit, out_tensor)`` runs after unit i is on
        the GPU (it synchronizes; use only off the clock)."""
        torch = self.torch
        units = self.store.units
        n = len(units)
        copied = [torch.cuda.Event() for _ in range(n)]
        reader = ThreadPoolExecutor(max_workers=1)

        def read(i):
            u, h = units[i], i % self.N_HOST
            t0 = time.perf_counter()
            afx.afx_file_read(self.store.path, u.offset, u.bytes, self.host[h].data_ptr(), self.read_threads,
                              self.direct)
            return time.perf_counter() - t0

        torch.cuda.synchronize(self.dev)
        t_start = time.perf_counter()
        futs = {i: reader.submit(read, i) for i in range(min(self.N_HOST, n))}
        read_s = unpack_s = wait_s = 0.0
        try:
            for i, u in enumerate(units):
                tw = time.perf_counter()
                read_s += futs.pop(i).result()
                wait_s += time.perf_counter() - tw
                h, o = i % self.N_HOST, i % self.N_OUT
                if i >= self.N_OUT:
                    copied[i - self.N_OUT].synchronize()  # its pinned BF16 buffer has been copied out
                t0 = time.perf_counter()
                oo = 0
                for t in u.tensors:
                    m = int(np.prod(t.shape))
                    afx.afx_decode_host(self.host[h].data_ptr() + t.offset, t.bytes,
                                        (self.host_out[o].data_ptr() + 2 * oo, 2 * m), self.unpack_threads)
                    oo += _out_slot(m)
                unpack_s += time.perf_counter() - t0
                if i + self.N_HOST < n:  # staging buffer h is free again
                    futs[i + self.N_HOST] = reader.submit(read, i + self.N_HOST)
                with torch.cuda.stream(self.copy_stream):
                    self.out[o][:oo].copy_(self.host_out[o][:oo], non_blocking=True)
                    copied[i].record(self.copy_stream)
                if on_unit is not None:
                    copied[i].synchronize()
                    on_unit(i, u, self.out[o])
            torch.cuda.synchronize(self.dev)
        finally:
            reader.shutdown(wait=True)
        return {"e2e_s": time.perf_counter() - t_start, "read_s": read_s, "unpack_s": unpack_s, "wait_s": wait_s,
                "restored_bytes": self.store.restored_bytes}

    def unpack_only_s(self, i: int) -> float:
        """Time the host restore of unit i alone (its bytes read first)."""
        u = self.store.units[i]
        afx.afx_file_read(self.store.path, u.offset, u.bytes, self.host[0].data_ptr(), self.read_threads, self.direct)
        t0 = time.perf_counter()
        oo = 0
        for t in u.tensors:
            m = int(np.prod(t.shape))
            afx.afx_decode_host(self.host[0].data_ptr() + t.offset, t.bytes,
                                (self.host_out[0].data_ptr() + 2 * oo, 2 * m), self.unpack_threads)
            oo += _out_slot(m)
        return time.perf_counter() - t0


def check_unit(out, specs) -> bool:
    """Regenerate a unit's original bits and compare with its restore."""
    import torch

    off, ok = 0, True
    for sp in specs:
        x = synth.generate(sp)
        ref = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(out.device)
        ok &= bool(torch.equal(out[off:off + x.size], ref))
        off += _out_slot(x.size)
    return ok
