"""Per-workgroup timestamps of the single-partition attention kernel (diagnostics).

Loads ``libas_attn_stamps.so`` (built by ``sequence_dit_amd.build`` beside the product
library: the same sources, with the single-partition bf16 kernels compiled with
``-DAS_WG_STAMPS``), runs the image DiT and video DiT workloads warm, stamps one launch of
each and prints, per class of query tile (full, or the partial last one), the mean time from
a workgroup's start to its first barrier (its Q rows and first K tile arriving), through its
key tiles, and through its epilogue; the launch's span from the first start to the last end;
the shader clock (s_memtime ticks per s_memrealtime time) and when the workgroups started.

Usage: ``python -m sequence_dit_amd.wg_stamps`` (needs a GPU).
"""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np

from . import _native as N
from . import inputs

STAMPS_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libas_attn_stamps.so")
STAMP_WGS = 16384   # kStampWGs of the kernel
REALTIME_NS = 10.0  # s_memrealtime runs at 100 MHz


def _load():
    L = N.load(STAMPS_LIB)
    L.as_debug_wg_stamps.restype = ctypes.c_int
    L.as_debug_wg_stamps.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L.as_debug_wg_stamps_clear.restype = ctypes.c_int
    L.as_debug_wg_stamps_clear.argtypes = []
    return L


def stamp_launch(L, torch, w, dev="cuda:0"):
    """Stamps of one warm single-partition launch of workload w: array [workgroups, 8]."""
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    B, H, Sq, D = q.shape
    out = torch.empty((w.P, B, H, Sq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((w.P, B, H, Sq), dtype=torch.float32, device=dev)
    flat = [int(x) for r in w.ranges for x in r]
    ranges = (ctypes.c_int32 * len(flat))(*flat)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), N.AS_BF16, B, H, Sq, k.shape[2], D,
            N._i64(q.stride()[:3]), N._i64(k.stride()[:3]), ranges, w.P, float(w.scale),
            out.data_ptr(), lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
    for _ in range(5):
        N.check(L.as_partition_attn(*args))
    torch.cuda.synchronize()
    assert L.as_debug_wg_stamps_clear() == 0
    N.check(L.as_partition_attn(*args))
    torch.cuda.synchronize()
    units = (w.P * B * H + 7) // 8 * 8
    n_qtiles = (Sq + 255) // 256
    nwg = min(units * n_qtiles, STAMP_WGS)
    host = np.zeros((STAMP_WGS, 8), dtype=np.uint64)
    assert L.as_debug_wg_stamps(host.ctypes.data, host.nbytes) == 0
    st = host[:nwg].astype(np.int64)
    return st[st[:, 0] > 0], n_qtiles, Sq % 256 != 0


def summarize(name, st, n_qtiles, partial):
    t0 = st[:, 0].min()
    us = lambda x: (x - t0) * REALTIME_NS / 1e3  # noqa: E731
    start, first, tiles_end, end = us(st[:, 0]), us(st[:, 1]), us(st[:, 2]), us(st[:, 3])
    qtile = st[:, 6] & 0xFFFFFFFF
    clock = (st[:, 5] - st[:, 4]) / np.maximum((st[:, 3] - st[:, 0]) * REALTIME_NS, 1.0)   # GHz
    lines = [f"### {name}: {len(st)} workgroups, span {end.max():.1f} us, shader clock "
             f"{np.median(clock):.2f} GHz (median over workgroups)", "",
             "| query tiles | workgroups | start to first barrier (us) | key tiles (us) | epilogue (us) | whole (us) |",
             "|---|---|---|---|---|---|"]
    classes = [("full", qtile < n_qtiles - 1 if partial else qtile >= 0)]
    if partial:
        classes.append(("partial (last)", qtile == n_qtiles - 1))
    for label, m in classes:
        lines.append(f"| {label} | {int(m.sum())} | {(first - start)[m].mean():.2f} | {(tiles_end - first)[m].mean():.2f} | "
                     f"{(end - tiles_end)[m].mean():.2f} | {(end - start)[m].mean():.2f} |")
    hist, edges = np.histogram(start, bins=8)
    lines += ["", "Workgroup starts (us from the first): " +
              ", ".join(f"{edges[i]:.0f}-{edges[i + 1]:.0f}: {hist[i]}" for i in range(len(hist))), ""]
    return "\n".join(lines)


def main() -> int:
    import torch
    if not torch.cuda.is_available():
        print("wg_stamps needs a GPU", file=sys.stderr)
        return 2
    L = _load()
    print("## Workgroup phases of the single-partition attention kernel (bf16, fp32 states)\n")
    print("Command (repo root, MI355X): `python -m sequence_dit_amd.wg_stamps`; one warm launch per "
          "workload of the diagnostics build (libas_attn_stamps.so), whose workgroups stamp "
          "s_memrealtime and s_memtime from their first thread.\n")
    for cfg, name in ((2, "image DiT (B1 H24 D128, Sq 576, P 8 x 576 keys)"),
                      (3, "video DiT (B1 H48 D64, Sq 2222, P 8 x ~2222 keys)")):
        st, nq, partial = stamp_launch(L, torch, inputs.make(cfg))
        print(summarize(name, st, nq, partial), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
