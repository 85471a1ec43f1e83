"""Seeded synthetic inputs for the merge / front-coding hot path.

Shared by the oracle tests, the GPU parity tests and ``bench.py``.  It draws
keys and values, sorts and de-duplicates each side, and packs records into the
per-side layout (key byte arena + n+1 u32 offsets, value byte arena + n+1 u32
offsets, one tombstone byte per record).  It contains none of the merge or
encoding arithmetic.

The five named workloads follow the shapes of the merge's evaluation setting:
two strictly sorted unique-key string record sets, older A and newer B, with a
stated fraction of B's keys also present in A and a tombstone rate on B.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.cpp")
_LIB = os.path.join(_HERE, "libgen.so")

KEY_UNIFORM, KEY_PATHS, KEY_U128, KEY_URL = 0, 1, 2, 3
VAL_UNIFORM, VAL_FIXED, VAL_LOGUNIFORM = 0, 1, 2

BASE64_SYMBOLS = b"ABCDEFGHIJKLMNOPQRSTUVWXYZabcdefghijklmnopqrstuvwxyz0123456789+/"
LOWER = b"abcdefghijklmnopqrstuvwxyz"


class _Params(ctypes.Structure):
    _fields_ = [
        ("key_kind", ctypes.c_int),
        ("kmin", ctypes.c_uint32), ("kmax", ctypes.c_uint32),
        ("alphabet", ctypes.c_char_p), ("nalpha", ctypes.c_uint32),
        ("seg_min", ctypes.c_uint32), ("seg_max", ctypes.c_uint32),
        ("vocab", ctypes.c_uint32),
        ("sl_min", ctypes.c_uint32), ("sl_max", ctypes.c_uint32),
        ("zipf_s", ctypes.c_double),
        ("hosts", ctypes.c_uint32), ("host_zipf", ctypes.c_double),
        ("hl_min", ctypes.c_uint32), ("hl_max", ctypes.c_uint32),
        ("digits", ctypes.c_uint32),
        ("val_kind", ctypes.c_int),
        ("vmin", ctypes.c_uint32), ("vmax", ctypes.c_uint32),
        ("nA", ctypes.c_uint64), ("nB", ctypes.c_uint64), ("nX", ctypes.c_uint64),
        ("tombA", ctypes.c_double), ("tombB", ctypes.c_double),
        ("seed", ctypes.c_uint64),
    ]


@dataclass
class Workload:
    """One synthetic workload: side sizes, overlap and the key/value recipe."""
    name: str
    nA: int
    nB: int
    overlap: float          # fraction of B's keys also present in A
    tombB: float            # Bernoulli tombstone probability on B
    key: dict = field(default_factory=dict)
    val: dict = field(default_factory=dict)
    seed: int = 0
    tombA: float = 0.0

    def scaled(self, scale: float) -> "Workload":
        w = Workload(**{**self.__dict__})
        w.nA = max(0, int(round(self.nA * scale)))
        w.nB = max(0, int(round(self.nB * scale)))
        w.name = f"{self.name}@{scale:g}"
        return w


# The five workloads.  "M" and "k" are decimal.
WORKLOADS = {
    1: Workload("uniform-az-10k+10k", 10_000, 10_000, 0.30, 0.05,
                key=dict(kind=KEY_UNIFORM, kmin=8, kmax=24, alphabet=LOWER),
                val=dict(kind=VAL_UNIFORM, vmin=0, vmax=32), seed=0x5EED0001),
    2: Workload("zipf-paths-1M+1M", 1_000_000, 1_000_000, 0.50, 0.02,
                key=dict(kind=KEY_PATHS, seg_min=2, seg_max=6, vocab=5000, sl_min=3, sl_max=10,
                         zipf_s=1.1),
                val=dict(kind=VAL_FIXED, vmin=16), seed=0x5EED0002),
    3: Workload("base64-8to64B-8M+8M", 8_000_000, 8_000_000, 0.50, 0.05,
                key=dict(kind=KEY_UNIFORM, kmin=8, kmax=64, alphabet=BASE64_SYMBOLS),
                val=dict(kind=VAL_UNIFORM, vmin=0, vmax=64), seed=0x5EED0003),
    4: Workload("u128-skewed-15M+100k", 15_000_000, 100_000, 0.80, 0.10,
                key=dict(kind=KEY_U128),
                val=dict(kind=VAL_FIXED, vmin=16), seed=0x5EED0004),
    5: Workload("url-64to256B-2M+2M", 2_000_000, 2_000_000, 0.40, 0.20,
                key=dict(kind=KEY_URL, kmin=64, kmax=256, hosts=20, host_zipf=1.2, hl_min=5,
                         hl_max=12, vocab=5000, sl_min=3, sl_max=10, zipf_s=1.1, digits=12),
                val=dict(kind=VAL_LOGUNIFORM, vmax=256), seed=0x5EED0005),
}


def build(force: bool = False) -> str:
    """Compile the generator's shared library in place (g++, host only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.gen_run.restype = ctypes.c_void_p
        lib.gen_run.argtypes = [ctypes.POINTER(_Params)]
        lib.gen_error.restype = ctypes.c_int
        lib.gen_error.argtypes = [ctypes.c_void_p]
        lib.gen_sizes.argtypes = [ctypes.c_void_p, ctypes.c_int] + [ctypes.POINTER(ctypes.c_uint64)] * 3
        lib.gen_copy.argtypes = [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 5
        lib.gen_free.argtypes = [ctypes.c_void_p]
        _lib = lib
    return _lib


@dataclass
class HostSide:
    """One input side in host memory (numpy)."""
    keys: np.ndarray      # uint8 [key_off[n]]
    key_off: np.ndarray   # uint32 [n+1]
    vals: np.ndarray      # uint8 [val_off[n]]
    val_off: np.ndarray   # uint32 [n+1]
    tomb: np.ndarray      # uint8 [n]

    @property
    def n(self) -> int:
        return int(self.tomb.shape[0])

    def key(self, i: int) -> bytes:
        return self.keys[self.key_off[i]:self.key_off[i + 1]].tobytes()

    def value(self, i: int):
        """The value bytes of record i, or None for a tombstone."""
        if self.tomb[i]:
            return None
        return self.vals[self.val_off[i]:self.val_off[i + 1]].tobytes()

    def records(self):
        return [(self.key(i), self.value(i)) for i in range(self.n)]

    def nbytes(self) -> int:
        return int(self.keys.nbytes + self.key_off.nbytes + self.vals.nbytes
                   + self.val_off.nbytes + self.tomb.nbytes)


def side_from_records(records) -> HostSide:
    """Pack [(key bytes, value bytes or None for a tombstone), ...] as given.

    The caller supplies records already in the order it wants; no sorting here.
    """
    keys = bytearray()
    vals = bytearray()
    key_off = [0]
    val_off = [0]
    tomb = []
    for k, v in records:
        keys += bytes(k)
        key_off.append(len(keys))
        if v is None:
            tomb.append(1)
        else:
            vals += bytes(v)
            tomb.append(0)
        val_off.append(len(vals))
    return HostSide(np.frombuffer(bytes(keys), dtype=np.uint8).copy(),
                    np.asarray(key_off, dtype=np.uint32),
                    np.frombuffer(bytes(vals), dtype=np.uint8).copy(),
                    np.asarray(val_off, dtype=np.uint32),
                    np.asarray(tomb, dtype=np.uint8))


def make(workload, seed: int | None = None):
    """Generate (A, B) host sides for a Workload or a workload number 1..5."""
    w = WORKLOADS[workload] if isinstance(workload, int) else workload
    lib = _load()
    k, v = w.key, w.val
    alpha = k.get("alphabet", b"")
    p = _Params()
    p.key_kind = k["kind"]
    p.kmin, p.kmax = k.get("kmin", 0), k.get("kmax", 0)
    p.alphabet, p.nalpha = alpha, len(alpha)
    p.seg_min, p.seg_max = k.get("seg_min", 0), k.get("seg_max", 0)
    p.vocab = k.get("vocab", 0)
    p.sl_min, p.sl_max = k.get("sl_min", 0), k.get("sl_max", 0)
    p.zipf_s = k.get("zipf_s", 0.0)
    p.hosts, p.host_zipf = k.get("hosts", 0), k.get("host_zipf", 0.0)
    p.hl_min, p.hl_max = k.get("hl_min", 0), k.get("hl_max", 0)
    p.digits = k.get("digits", 0)
    p.val_kind = v["kind"]
    p.vmin, p.vmax = v.get("vmin", 0), v.get("vmax", 0)
    p.nA, p.nB = w.nA, w.nB
    p.nX = int(round(w.overlap * w.nB))
    p.tombA, p.tombB = w.tombA, w.tombB
    p.seed = w.seed if seed is None else seed
    h = lib.gen_run(ctypes.byref(p))
    try:
        err = lib.gen_error(h)
        if err:
            raise ValueError(f"generator failed (code {err}) for {w.name}")
        sides = []
        for s in (0, 1):
            n, kb, vb = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
            lib.gen_sizes(h, s, ctypes.byref(n), ctypes.byref(kb), ctypes.byref(vb))
            hs = HostSide(np.empty(kb.value, np.uint8), np.empty(n.value + 1, np.uint32),
                          np.empty(vb.value, np.uint8), np.empty(n.value + 1, np.uint32),
                          np.empty(n.value, np.uint8))
            lib.gen_copy(h, s, hs.keys.ctypes.data, hs.key_off.ctypes.data, hs.vals.ctypes.data,
                         hs.val_off.ctypes.data, hs.tomb.ctypes.data)
            sides.append(hs)
    finally:
        lib.gen_free(h)
    return sides[0], sides[1]
