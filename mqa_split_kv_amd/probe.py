"""HBM read ceiling and copy-kernel reference (libpa_probe.so), for measurement only.

    python -m mqa_split_kv_amd.probe [--gib 2] [--copy-mib 512]

read : streams a fresh buffer once per launch (nontemporal 16-byte loads) and reports
       the best GB/s over a few grid sizes - the practical read ceiling of the HBM.
copy : a plain 16-byte copy of a known size, launched on its own so that rocprofv3
       FETCH_SIZE / WRITE_SIZE readings of it calibrate the decode kernel's.
gather: reads a buffer once as fixed-size chunks in a random order (a page gather; one
       chunk = one page of one KV head) - the read ceiling of that access pattern.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB = os.path.join(HERE, "lib", "libpa_probe.so")


def _lib():
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built; run `python -m mqa_split_kv_amd.build`")
    L = ctypes.CDLL(PROBE_LIB)
    L.pa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                ctypes.c_void_p]
    L.pa_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                ctypes.c_void_p]
    L.pa_probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return L


def read_ceiling(gib: float = 2.0, reps: int = 5, grids=(1024, 2048, 4096, 8192)) -> dict:
    import torch

    L = _lib()
    nbytes = int(gib * (1 << 30)) // 4096 * 4096
    # two buffers, alternated, so consecutive launches do not hit the 256 MB MALL
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    for b in bufs:
        b.fill_(1)
    sink = torch.empty(max(grids), dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = {}
    for g in grids:
        L.pa_probe_read(ctypes.c_void_p(bufs[0].data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), g, stream)
        torch.cuda.synchronize()
        times = []
        for r in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            L.pa_probe_read(ctypes.c_void_p(bufs[r % 2].data_ptr()), nbytes,
                            ctypes.c_void_p(sink.data_ptr()), g, stream)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        best[g] = nbytes / min(times) / 1e9
    g = max(best, key=best.get)
    return {"bytes": nbytes, "best_gbs": round(best[g], 1), "best_grid": g,
            "by_grid": {str(k): round(v, 1) for k, v in best.items()}}


def gather_ceiling(gib: float = 2.0, chunks=(2048, 16384), reps: int = 4, per_wg=(4, 16, 64)) -> dict:
    """Best GB/s reading `gib` GiB once as `chunk`-byte pieces in a seeded random order."""
    import torch

    L = _lib()
    nbytes = int(gib * (1 << 30)) // 65536 * 65536
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    for b in bufs:
        b.fill_(1)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    gen = torch.Generator(device="cpu").manual_seed(7)
    res = {}
    for chunk in chunks:
        n = nbytes // chunk
        order = torch.randperm(n, generator=gen).to(torch.int32).cuda()
        sink = torch.empty(n, dtype=torch.int32, device="cuda")
        best = 0.0
        for pw in per_wg:
            assert L.pa_probe_gather(ctypes.c_void_p(bufs[0].data_ptr()), ctypes.c_void_p(order.data_ptr()),
                                     n, chunk, pw, ctypes.c_void_p(sink.data_ptr()), stream) == 0
            torch.cuda.synchronize()
            for r in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                L.pa_probe_gather(ctypes.c_void_p(bufs[r % 2].data_ptr()), ctypes.c_void_p(order.data_ptr()),
                                  n, chunk, pw, ctypes.c_void_p(sink.data_ptr()), stream)
                e1.record()
                torch.cuda.synchronize()
                best = max(best, n * chunk / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        res[str(chunk)] = round(best, 1)
    return res


def copy_once(mib: int = 512, blocks: int = 2048) -> dict:
    import torch

    L = _lib()
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    rc = L.pa_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n, blocks, stream)
    e1.record()
    torch.cuda.synchronize()
    assert rc == 0
    assert bool((dst[:: 1 << 20] == 1).all())
    return {"bytes_read": n, "bytes_written": n, "us": round(e0.elapsed_time(e1) * 1e3, 2)}


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--gib", type=float, default=2.0)
    ap.add_argument("--copy-mib", type=int, default=512)
    ap.add_argument("--copy-only", action="store_true")
    a = ap.parse_args()
    res = {"copy": copy_once(a.copy_mib)}
    if not a.copy_only:
        res["read"] = read_ceiling(a.gib)
        res["gather_random"] = gather_ceiling(a.gib)
    print(json.dumps(res), flush=True)
