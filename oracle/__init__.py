"""CPU oracle for the replacement merge into a front-coded bit payload.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product path in
``merge_front_coded_amd`` never does.  It shares no code with the GPU library.

The arithmetic lives in ``oracle.c`` (plain single-threaded C, one bit at a
time); this module only compiles it and marshals numpy arrays.  Each wrapper
names the passage of the pages its C function follows.

Pinned by the ``-m "not gpu"`` tests against the pages' worked merge examples,
brute-force set semantics, the closed-form record length, an independent
decoder and hand-derived payloads; the navigation sections by hand-derived
sections, an independent section reader (every entry selected back), the
exact sparse threshold and value widths read back from decoded payloads; the
payload decoder by a hand-derived payload, malformed lengths, and round trips
checked against the merged input records and the independent Python
decoder; the byte-profile encoder by hand-derived records, LEB128 edge
values and an independent byte-profile reader.  No function here is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
NONE = 0xFFFFFFFF


class _Side(ctypes.Structure):
    _fields_ = [("keys", ctypes.c_void_p), ("key_off", ctypes.c_void_p),
                ("vals", ctypes.c_void_p), ("val_off", ctypes.c_void_p),
                ("tomb", ctypes.c_void_p), ("n", ctypes.c_uint32)]


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (host only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        S = ctypes.POINTER(_Side)
        u32 = ctypes.c_uint32
        lib.or_key_cmp.restype = ctypes.c_int
        lib.or_key_cmp.argtypes = [S, u32, S, u32]
        lib.or_key_lcp_bits.restype = ctypes.c_uint64
        lib.or_key_lcp_bits.argtypes = [S, u32, S, u32]
        lib.or_merge.argtypes = [S, S, P]
        lib.or_corank.restype = u32
        lib.or_corank.argtypes = [P, u32, u32]
        lib.or_keep.restype = u32
        lib.or_keep.argtypes = [S, S, P, u32, P, P, P]
        lib.or_encode.restype = ctypes.c_uint64
        lib.or_encode.argtypes = [S, S, P, u32, P, P, P, P, ctypes.c_uint64]
        lib.or_collision.restype = u32
        lib.or_collision.argtypes = [S, S, P, P, P, P, P, P]
        lib.or_rank.restype = u32
        lib.or_rank.argtypes = [P, u32]
        lib.or_common_width.restype = ctypes.c_uint64
        lib.or_common_width.argtypes = [S, S, P, u32]
        lib.or_ef_entries.argtypes = [P, u32, ctypes.c_uint64, ctypes.c_uint64, P]
        lib.or_ef_encode.argtypes = [P, ctypes.c_uint64, ctypes.c_uint64, P, P, P, P, P]
        lib.or_bp_width.restype = ctypes.c_uint64
        lib.or_bp_width.argtypes = [S, S, P, u32]
        lib.or_bp_encode.restype = ctypes.c_uint64
        lib.or_bp_encode.argtypes = [S, S, P, u32, ctypes.c_uint64, P, P, P, P, ctypes.c_uint64]
        lib.or_fc_decode.restype = ctypes.c_int
        lib.or_fc_decode.argtypes = [P, ctypes.c_uint64, u32, P, ctypes.c_uint64, P, P, ctypes.c_uint64, P, P]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data if a.size else 0


def _side(h):
    """Marshal a host side (gen.HostSide or anything with the same fields)."""
    s = _Side()
    s.keys, s.key_off = _ptr(h.keys), _ptr(h.key_off)
    s.vals, s.val_off = _ptr(h.vals), _ptr(h.val_off)
    s.tomb, s.n = _ptr(h.tomb), int(h.tomb.shape[0])
    return s


def key_cmp(X, i: int, Y, j: int) -> int:
    """Unsigned bytewise order, proper prefix first (<0, 0, >0)."""
    return _load().or_key_cmp(ctypes.byref(_side(X)), i, ctypes.byref(_side(Y)), j)


def key_lcp_bits(X, i: int, Y, j: int) -> int:
    """Leading equal bits of key i of X and key j of Y, clamped to the shorter key."""
    return int(_load().or_key_lcp_bits(ctypes.byref(_side(X)), i, ctypes.byref(_side(Y)), j))


def merge(A, B) -> np.ndarray:
    """Stable two-pointer merge, ties to the older side A.  Refs: A_i -> i, B_j -> |A|+j."""
    refs = np.empty(A.n + B.n, np.uint32)
    _load().or_merge(ctypes.byref(_side(A)), ctypes.byref(_side(B)), _ptr(refs))
    return refs


def corank(refs: np.ndarray, nA: int, d: int) -> int:
    """Number of A records among the first d merged outputs."""
    return int(_load().or_corank(_ptr(refs), nA, d))


def diagonals(N: int, items_per_part: int):
    """Diagonals d_p = min(p * items, N) for p = 0..ceil(N/items)."""
    P = (N + items_per_part - 1) // items_per_part
    return [min(p * items_per_part, N) for p in range(P + 1)]


def splits(refs: np.ndarray, nA: int, items_per_part: int) -> np.ndarray:
    """Co-rank at every partition diagonal.

    Same definition as ``corank`` (A records among the first d outputs), with
    the counts of all prefixes taken at once by a cumulative sum so that large
    inputs finish quickly.
    """
    counts = np.zeros(refs.shape[0] + 1, np.int64)
    np.cumsum(refs < nA, out=counts[1:])
    d = np.asarray(diagonals(refs.shape[0], items_per_part), np.int64)
    return counts[d].astype(np.uint32)


def keep(A, B, refs: np.ndarray):
    """Keep-newer over the merged refs -> (final_refs, ord_A, ord_B, S)."""
    N = int(refs.shape[0])
    final = np.empty(N, np.uint32)
    ord_A = np.empty(A.n, np.uint32)
    ord_B = np.empty(B.n, np.uint32)
    S = _load().or_keep(ctypes.byref(_side(A)), ctypes.byref(_side(B)), _ptr(refs), N,
                        _ptr(final), _ptr(ord_A), _ptr(ord_B))
    return final[:S].copy(), ord_A, ord_B, int(S)


def payload_capacity_bytes(A, B) -> int:
    """A safe byte capacity for the encoder: every record at its largest."""
    n = A.n + B.n
    raw = int(A.keys.size + B.keys.size + A.vals.size + B.vals.size)
    return raw + (n * (3 * 65 + 1) + 7) // 8 + 16


def encode(A, B, final: np.ndarray):
    """Front-code the survivors -> (len_bits, lcp_bits, off, T, payload bytes).

    ``payload`` is the MSB-first bit stream, zero padded to 4 * ceil(T/32) bytes.
    """
    S = int(final.shape[0])
    len_bits = np.empty(S, np.uint32)
    lcp_bits = np.empty(S, np.uint32)
    off = np.empty(S + 1, np.uint64)
    cap = payload_capacity_bytes(A, B)
    buf = np.zeros(cap, np.uint8)
    T = _load().or_encode(ctypes.byref(_side(A)), ctypes.byref(_side(B)), _ptr(final), S,
                          _ptr(len_bits), _ptr(lcp_bits), _ptr(off), _ptr(buf), cap)
    if T == 0xFFFFFFFFFFFFFFFF:
        raise RuntimeError("oracle payload capacity exceeded")
    nbytes = 4 * ((int(T) + 31) // 32)
    return len_bits, lcp_bits, off, int(T), buf[:nbytes].copy()


def collision(A, B):
    """Collision-bit ordinals -> dict(C, R, lb, ord_A, ord_B, final, S)."""
    C = np.empty(A.n, np.uint8)
    R = np.empty(A.n + 1, np.uint32)
    lb = np.empty(B.n, np.uint32)
    ord_A = np.empty(A.n, np.uint32)
    ord_B = np.empty(B.n, np.uint32)
    final = np.empty(A.n + B.n, np.uint32)
    S = _load().or_collision(ctypes.byref(_side(A)), ctypes.byref(_side(B)), _ptr(C), _ptr(R),
                             _ptr(lb), _ptr(ord_A), _ptr(ord_B), _ptr(final))
    return dict(C=C, R=R, lb=lb, ord_A=ord_A, ord_B=ord_B, final=final[:S].copy(), S=int(S))


def rank(words: np.ndarray, positions) -> np.ndarray:
    """Exclusive rank (set bits strictly below p) at each position."""
    w = np.ascontiguousarray(words, dtype=np.uint32)
    lib = _load()
    return np.asarray([lib.or_rank(_ptr(w), int(p)) for p in positions], dtype=np.uint32)


class _EfInfo(ctypes.Structure):
    _fields_ = [(f, ctypes.c_uint64) for f in ("n", "L", "width", "low_words", "high_bits", "high_words",
                                               "groups", "exceptions")]


def common_width(A, B, final: np.ndarray) -> int:
    """The encoded value width all survivors share, else 0 (0 when S = 0)."""
    f = np.ascontiguousarray(final, dtype=np.uint32)
    return int(_load().or_common_width(ctypes.byref(_side(A)), ctypes.byref(_side(B)), _ptr(f), f.size))


def ef_entries(off: np.ndarray, S: int, T: int, width: int) -> np.ndarray:
    """The offsets of records 0, 15, 30, ... and T, each less width x its ordinal."""
    o = np.ascontiguousarray(off, dtype=np.uint64)
    e = np.empty((S + 14) // 15 + 1, np.uint64)
    _load().or_ef_entries(_ptr(o), S, T, width, _ptr(e))
    return e


def ef_encode(entries: np.ndarray, width: int = 0) -> dict:
    """Elias-Fano sections of non-decreasing entries -> dict(lows, highs,
    samples, exceptions, and the header fields n, L, width, low_words,
    high_bits, high_words, groups, n_exceptions)."""
    e = np.ascontiguousarray(entries, dtype=np.uint64)
    n = int(e.size)
    if n == 0:
        raise ValueError("at least one entry (the EOF entry) is needed")
    lows = np.zeros(n + 1, np.uint64)
    highs = np.zeros((3 * n + 1 + 63) // 64 + 1, np.uint64)
    groups = (n + 255) // 256
    samples = np.zeros(2 * groups, np.uint64)
    exc = np.zeros(n, np.uint64)
    info = _EfInfo()
    _load().or_ef_encode(_ptr(e), n, width, _ptr(lows), _ptr(highs), _ptr(samples), _ptr(exc),
                         ctypes.byref(info))
    out = {f: int(getattr(info, f)) for f, _ in _EfInfo._fields_}
    out["n_exceptions"] = out.pop("exceptions")
    out.update(lows=lows[:info.low_words].copy(), highs=highs[:info.high_words].copy(), samples=samples,
               exceptions=exc[:info.exceptions].copy())
    return out


def ef_navigation(A, B, final: np.ndarray, off: np.ndarray, T: int) -> dict:
    """The output navigation of a merged payload: common width, entries, EF sections."""
    S = int(final.shape[0])
    w = common_width(A, B, final)
    return ef_encode(ef_entries(off, S, T, w), w)


def fc_decode(payload: np.ndarray, T: int, S: int, key_cap: int, val_cap: int):
    """Decode a front-coded payload of S records -> a side (gen.HostSide).

    key_cap / val_cap bound the arenas; raises ValueError on a malformed
    payload or too small a capacity."""
    import gen
    p = np.ascontiguousarray(payload, dtype=np.uint8)
    keys = np.zeros(max(key_cap, 1), np.uint8)
    vals = np.zeros(max(val_cap, 1), np.uint8)
    key_off = np.zeros(S + 1, np.uint32)
    val_off = np.zeros(S + 1, np.uint32)
    tomb = np.zeros(S, np.uint8)
    rc = _load().or_fc_decode(_ptr(p), T, S, _ptr(keys), key_cap, _ptr(key_off), _ptr(vals), val_cap,
                              _ptr(val_off), _ptr(tomb))
    if rc:
        raise ValueError("malformed payload or capacity too small")
    return gen.HostSide(keys=keys[:key_off[S]].copy(), key_off=key_off, vals=vals[:val_off[S]].copy(),
                        val_off=val_off, tomb=tomb)


def bp_width(A, B, final: np.ndarray) -> int:
    """Byte-profile framing width: 1 + L when every present survivor's value
    is L bytes (or none is present), else 0 (variable framing)."""
    f = np.ascontiguousarray(final, dtype=np.uint32)
    return int(_load().or_bp_width(ctypes.byref(_side(A)), ctypes.byref(_side(B)), _ptr(f), f.size))


def bp_encode(A, B, final: np.ndarray):
    """Byte-profile encoding -> dict(width, len_bytes, lcp_bytes, off, T (bytes), payload)."""
    f = np.ascontiguousarray(final, dtype=np.uint32)
    S = int(f.size)
    w = bp_width(A, B, f)
    len_bytes = np.empty(S, np.uint32)
    lcp_bytes = np.empty(S, np.uint32)
    off = np.empty(S + 1, np.uint64)
    cap = payload_capacity_bytes(A, B) + S * (24 + w)  # (+ w: a tombstone's filler bytes)
    buf = np.zeros(cap, np.uint8)
    T = _load().or_bp_encode(ctypes.byref(_side(A)), ctypes.byref(_side(B)), _ptr(f), S, w, _ptr(len_bytes),
                             _ptr(lcp_bytes), _ptr(off), _ptr(buf), cap)
    if T == 0xFFFFFFFFFFFFFFFF:
        raise RuntimeError("oracle payload capacity exceeded")
    return dict(width=w, len_bytes=len_bytes, lcp_bytes=lcp_bytes, off=off, T=int(T), payload=buf[:T].copy())


def run(A, B, items_per_part: int = 2048):
    """The whole path on the CPU: merge, co-ranks, keep-newer, front coding."""
    refs = merge(A, B)
    final, ord_A, ord_B, S = keep(A, B, refs)
    len_bits, lcp_bits, off, T, payload = encode(A, B, final)
    return dict(refs=refs, splits=splits(refs, A.n, items_per_part),
                final=final, ord_A=ord_A, ord_B=ord_B, S=S, len_bits=len_bits, lcp_bits=lcp_bits,
                off=off, T=T, payload=payload)
