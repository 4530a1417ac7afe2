"""Seeded synthetic 4D-STEM workloads (input generation only).

The five workloads mirror the acquisitions the method is benchmarked on:
Poisson counts, bright inside a disk that drifts per scan and dim outside it,
with optional sentinel pixels. This module draws inputs and builds query
masks; it holds none of the coding or reduction arithmetic, and it is the only
code that both the CPU oracle and the GPU library take inputs from.
"""
import ctypes
import os
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


class _Params(ctypes.Structure):
    _fields_ = [
        ("scan_rows", ctypes.c_uint32), ("scan_cols", ctypes.c_uint32),
        ("det_rows", ctypes.c_uint32), ("det_cols", ctypes.c_uint32),
        ("dtype", ctypes.c_uint32), ("shift_kind", ctypes.c_uint32),
        ("sentinel_pct", ctypes.c_uint32), ("pad_", ctypes.c_uint32),
        ("lam_in", ctypes.c_double), ("lam_out", ctypes.c_double),
        ("cr", ctypes.c_double), ("cc", ctypes.c_double), ("radius", ctypes.c_double),
        ("seed", ctypes.c_uint64),
    ]


def build(force=False):
    """Compile libsynth.so with gcc (plain C, no GPU code)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        cmd = f"gcc -O2 -fPIC -shared -pthread -o {_LIB_PATH}.tmp {src} -lm && mv {_LIB_PATH}.tmp {_LIB_PATH}"
        if os.system(cmd) != 0:
            raise RuntimeError("failed to build libsynth.so")


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER(_Params)
        lib.synth_counts.argtypes = [P, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int]
        lib.synth_scaled.argtypes = [P, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int]
        lib.synth_shift.argtypes = [P, ctypes.c_uint64, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
        lib.synth_is_sentinel.argtypes = [P, ctypes.c_uint32]
        lib.synth_is_sentinel.restype = ctypes.c_int
        _lib = lib
    return _lib


@dataclass(frozen=True)
class Workload:
    name: str
    scan_rows: int
    scan_cols: int
    det_rows: int
    det_cols: int
    dtype: int  # 1 = uint8, 2 = uint16
    lam_in: float
    lam_out: float
    cr: float
    cc: float
    radius: float
    shift_kind: int  # 0 none, 1 jitter +-1, 2 smooth field +-3
    sentinel_pct: int
    seed: int
    layout: int  # 0 byte-rANS, 1 paired tANS

    @property
    def S(self):
        return self.scan_rows * self.scan_cols

    @property
    def P(self):
        return self.det_rows * self.det_cols

    @property
    def np_dtype(self):
        return np.uint8 if self.dtype == 1 else np.uint16

    def params(self):
        return _Params(self.scan_rows, self.scan_cols, self.det_rows, self.det_cols, self.dtype,
                       self.shift_kind, self.sentinel_pct, 0, self.lam_in, self.lam_out,
                       self.cr, self.cc, self.radius, self.seed)

    def with_scans(self, scan_rows, scan_cols):
        return replace(self, scan_rows=scan_rows, scan_cols=scan_cols)


# The five benchmark workloads (seed = 1000 + index).
WORKLOADS = {
    "tiny_u8": Workload("tiny_u8", 16, 16, 64, 64, 1, 2.0, 0.05, 32, 32, 10, 1, 0, 1001, 0),
    "scan128_u16": Workload("scan128_u16", 128, 128, 192, 192, 2, 5.0, 0.1, 96, 96, 30, 2, 0, 1002, 0),
    "scan256_u16_sentinel": Workload("scan256_u16_sentinel", 256, 256, 192, 192, 2, 5.0, 0.1, 96, 96, 30, 2, 1, 1003, 0),
    "scan512_u8_lowdose": Workload("scan512_u8_lowdose", 512, 512, 192, 192, 1, 0.8, 0.02, 96, 96, 30, 2, 0, 1004, 0),
    "scan1024_u16_paired": Workload("scan1024_u16_paired", 1024, 1024, 192, 192, 2, 5.0, 0.1, 96, 96, 30, 2, 0, 1005, 1),
}


def counts(w: Workload, first=0, n=None, threads=None):
    """Counts of scans [first, first+n) as an (n, P) array of the native dtype."""
    n = w.S - first if n is None else n
    threads = threads or min(16, os.cpu_count() or 1)
    out = np.empty((n, w.P), dtype=w.np_dtype)
    p = w.params()
    if _load().synth_counts(ctypes.byref(p), first, n, out.ctypes.data, threads) != 0:
        raise ValueError("synth_counts failed")
    return out


def scaled(w: Workload, first=0, n=None, threads=None):
    """float32 intensities 0.731*count - 0.25 + noise, from sentinel-free counts."""
    n = w.S - first if n is None else n
    threads = threads or min(16, os.cpu_count() or 1)
    out = np.empty((n, w.P), dtype=np.float32)
    p = w.params()
    if _load().synth_scaled(ctypes.byref(p), first, n, out.ctypes.data, threads) != 0:
        raise ValueError("synth_scaled failed")
    return out


def shift(w: Workload, s):
    p = w.params()
    dr, dc = ctypes.c_int32(), ctypes.c_int32()
    _load().synth_shift(ctypes.byref(p), s, ctypes.byref(dr), ctypes.byref(dc))
    return dr.value, dc.value


def sentinels(w: Workload):
    """uint8[P]: 1 where the pixel is a sentinel (dtype maximum in every frame)."""
    p = w.params()
    lib = _load()
    return np.array([lib.synth_is_sentinel(ctypes.byref(p), i) for i in range(w.P)], dtype=np.uint8)


def valid_pixels(w: Workload):
    """uint8[P] validity mask that excludes the sentinels, or None when there are none."""
    if w.sentinel_pct == 0:
        return None
    return (1 - sentinels(w)).astype(np.uint8)


def disk_mask(det_rows, det_cols, cr, cc, r):
    """uint8[P]: 1 where (kr-cr)^2 + (kc-cc)^2 <= r^2."""
    kr, kc = np.meshgrid(np.arange(det_rows), np.arange(det_cols), indexing="ij")
    d2 = (kr - cr) ** 2 + (kc - cc) ** 2
    return (d2 <= r * r).astype(np.uint8).ravel()


def annulus_mask(det_rows, det_cols, cr, cc, r_in, r_out):
    """uint8[P]: 1 where r_in^2 <= (kr-cr)^2 + (kc-cc)^2 <= r_out^2."""
    kr, kc = np.meshgrid(np.arange(det_rows), np.arange(det_cols), indexing="ij")
    d2 = (kr - cr) ** 2 + (kc - cc) ** 2
    return ((d2 >= r_in * r_in) & (d2 <= r_out * r_out)).astype(np.uint8).ravel()


def query_masks(w: Workload):
    """The named masks each workload is queried with."""
    if w.name == "tiny_u8":
        return {"bf": disk_mask(64, 64, 32, 32, 8), "adf": annulus_mask(64, 64, 32, 32, 14, 30)}
    if w.name == "scan512_u8_lowdose":
        return {"bf": disk_mask(192, 192, 96, 96, 53), "adf": annulus_mask(192, 192, 96, 96, 60, 90)}
    bf = disk_mask(w.det_rows, w.det_cols, 96, 96, 30)
    return {"bf": bf, "df": (1 - bf).astype(np.uint8)}


def sweep_masks(w: Workload):
    """Moving BF r=53 mask at 64 positions (centre shifts of -7..7 in steps of 2)."""
    offs = [-7, -5, -3, -1, 1, 3, 5, 7]
    return [disk_mask(w.det_rows, w.det_cols, 96 + a, 96 + b, 53) for a in offs for b in offs]
