"""Minimal ctypes access to HIP events (for timing kernels on a given stream)."""

from __future__ import annotations

import ctypes

_hip = None


def hip():
    global _hip
    if _hip is None:
        L = ctypes.CDLL("libamdhip64.so")
        L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _hip = L
    return _hip


def event_create() -> int:
    ev = ctypes.c_void_p()
    err = hip().hipEventCreate(ctypes.byref(ev))
    if err != 0:
        raise RuntimeError(f"hipEventCreate failed: {err}")
    return ev.value


def event_destroy(ev: int):
    hip().hipEventDestroy(ev)


def event_record(ev: int, stream: int):
    err = hip().hipEventRecord(ev, stream)
    if err != 0:
        raise RuntimeError(f"hipEventRecord failed: {err}")


def elapsed_ms(start: int, stop: int) -> float:
    hip().hipEventSynchronize(stop)
    ms = ctypes.c_float(0.0)
    err = hip().hipEventElapsedTime(ctypes.byref(ms), start, stop)
    if err != 0:
        raise RuntimeError(f"hipEventElapsedTime failed: {err}")
    return float(ms.value)
