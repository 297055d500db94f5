"""Runs the unmodified single-thread oracle on many independent pieces at
once: a thread pool whose tasks each make ordinary oracle calls (ctypes
releases the GIL for the duration of a foreign call, so the calls run in
parallel).  Used where a parity test compares whole full-size outputs."""
from __future__ import annotations

import concurrent.futures as cf
import os

_pool = None


def threads() -> int:
    """Worker threads: the host's cores, at most 16 (a GPU machine's CPU share)."""
    return max(1, min(16, os.cpu_count() or 1))


def pmap(fn, items):
    global _pool
    if _pool is None:
        _pool = cf.ThreadPoolExecutor(threads())
    return list(_pool.map(fn, items))
