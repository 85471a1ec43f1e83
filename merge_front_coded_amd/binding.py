"""ctypes binding of the C ABI in include/em.h: same names, marshalling only.

Device buffers are torch tensors (PyTorch-ROCm supplies device memory and
streams); every step of the path runs in the HIP library.  If ``libem.so``
has not been built the import fails loudly: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libem.so")

EM_OK = 0
EM_EINVAL = -1
EM_ERANGE = -2
EM_ENOSPC = -3
EM_EDEVICE = -4
EM_NONE = 0xFFFFFFFF
EM_MAX_RECORDS = 1 << 24
EM_ARENA_PAD = 32
EM_MAX_ITEMS_PER_PART = 4096


class EmError(RuntimeError):
    def __init__(self, code: int, call: str, lib):
        msg = lib.em_strerror(code).decode()
        if code == EM_EDEVICE:
            msg += f" (hipError {lib.em_last_hip_error()})"
        super().__init__(f"{call}: {msg} [{code}]")
        self.code = code


class em_side_t(ctypes.Structure):
    _fields_ = [("keys", ctypes.c_void_p), ("key_off", ctypes.c_void_p),
                ("vals", ctypes.c_void_p), ("val_off", ctypes.c_void_p),
                ("tomb", ctypes.c_void_p), ("n", ctypes.c_uint32),
                ("key_bytes", ctypes.c_uint64), ("val_bytes", ctypes.c_uint64)]


def load_library(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m merge_front_coded_amd.build` "
                          "(the merge path runs only in the HIP library)")
    lib = ctypes.CDLL(path)
    P, S = ctypes.c_void_p, ctypes.POINTER(em_side_t)
    u32, u64, sz, i32 = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_int
    sig = {
        "em_workspace_bytes": (sz, [u32, u32, u32]),
        "em_payload_bound_bits": (i32, [S, S, ctypes.POINTER(u64)]),
        "em_partition": (i32, [S, S, u32, P, P, sz, P]),
        "em_merge_keep": (i32, [S, S, P, u32, P, P, P, P, P, sz, P]),
        "em_collision_rank": (i32, [S, S, P, P, P, P, P, sz, P]),
        "em_collision_rank_mode": (i32, [S, S, u32, P, P, P, P, P, sz, P]),
        "em_collision_workspace_bytes": (sz, [u32, u32, u32]),
        "em_rank2048_probe": (i32, [P, u32, P, u32, P, P, sz, P]),
        "em_rank2048_workspace_bytes": (sz, [u32]),
        "em_fc_lengths": (i32, [S, S, P, u32, P, P, P, sz, P]),
        "em_scan": (i32, [P, u32, P, P, sz, P]),
        "em_scan_noalloc": (i32, [P, u32, P, P]),
        "em_emit": (i32, [S, S, P, P, u32, P, u64, P, u64, P, sz, P]),
        "em_rank512_probe": (i32, [P, u32, P, u32, P, P, sz, P]),
        "em_merge_fc_workspace_bytes": (sz, [u32, u32, u32]),
        "em_merge_fc": (i32, [S, S, P, u32, u32, P, u64, P, P, P, P, P, P, P, P, P, sz, P]),
        "em_merge_fc_onepass": (i32, [S, S, P, u32, u32, P, u64, P, P, P, P, P, P, P, P, P, sz, P]),
        "em_onepass_workspace_bytes": (sz, [u32, u32, u32]),
        "em_merge_lengths": (i32, [S, S, P, u32, u32, P, P, P, P, P, P, P, P, sz, P]),
        "em_emit_merged": (i32, [S, S, u32, P, u64, P, P, P, P, P, P, sz, P]),
        "em_rank512_workspace_bytes": (sz, [u32]),
        "em_ef_entry_count": (u32, [u32]),
        "em_ef_capacity": (i32, [u32, ctypes.POINTER(u64), ctypes.POINTER(u64), ctypes.POINTER(u64),
                                 ctypes.POINTER(u64)]),
        "em_ef_workspace_bytes": (sz, [u32]),
        "em_ef_navigation": (i32, [S, S, P, u32, P, u64, P, u64, P, u64, P, u64, P, u64, P, P, sz, P]),
        "em_ef_encode": (i32, [P, u32, u64, P, u64, P, u64, P, u64, P, u64, P, P, sz, P]),
        "em_fcin_workspace_bytes": (sz, [u32]),
        "em_fcin_parse": (i32, [P, u64, u64, u32, P, P, P, P, P, P, P, P, sz, P]),
        "em_fcin_materialize": (i32, [P, u64, u32, P, u64, P, P, u64, P, P, P, P, sz, P]),
        "em_fcin_prefix8": (i32, [P, u64, u32, P, P, sz, P]),
        "em_fcin_compare": (i32, [P, u64, u32, P, sz, P, u64, u32, P, sz, u32, P, P, u32, P, P, P]),
        "em_bp_workspace_bytes": (sz, [u32]),
        "em_bp_lengths": (i32, [S, S, P, P, u32, P, P, P, sz, P]),
        "em_bp_emit": (i32, [S, S, P, P, u32, P, u64, P, P, u64, P, P]),
        "em_bp_navigation": (i32, [P, u32, u64, P, P, u64, P, u64, P, u64, P, u64, P, P, sz, P]),
        "em_strerror": (ctypes.c_char_p, [i32]),
        "em_last_hip_error": (i32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


def _p(t) -> int | None:
    """Device address of a tensor (None for None)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("buffers passed to the HIP library must be device tensors")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(rc: int, call: str):
    if rc != EM_OK:
        raise EmError(rc, call, lib())


class DeviceSide:
    """One input side in device memory, laid out as em_side_t requires."""

    def __init__(self, keys, key_off, vals, val_off, tomb, n: int, key_bytes: int, val_bytes: int):
        self.keys, self.key_off, self.vals, self.val_off, self.tomb = keys, key_off, vals, val_off, tomb
        self.n, self.key_bytes, self.val_bytes = int(n), int(key_bytes), int(val_bytes)
        self._struct = em_side_t(_p(keys), _p(key_off), _p(vals), _p(val_off), _p(tomb), self.n,
                                 self.key_bytes, self.val_bytes)

    @property
    def struct(self) -> em_side_t:
        return self._struct

    @staticmethod
    def _arena(data, device) -> torch.Tensor:
        n = int(data.shape[0])
        t = torch.zeros(((n + 15) // 16) * 16 + EM_ARENA_PAD, dtype=torch.uint8, device=device)
        if n:
            t[:n].copy_(torch.from_numpy(data))
        return t

    @classmethod
    def from_host(cls, hs, device="cuda"):
        """Upload a host side (key/value arenas, u32 offsets, tombstone bytes)."""
        keys = cls._arena(hs.keys, device)
        vals = cls._arena(hs.vals, device)
        key_off = torch.from_numpy(hs.key_off.view("int32")).to(device)
        val_off = torch.from_numpy(hs.val_off.view("int32")).to(device)
        tomb = torch.from_numpy(hs.tomb).to(device) if hs.tomb.size else \
            torch.zeros(16, dtype=torch.uint8, device=device)
        return cls(keys, key_off, vals, val_off, tomb, hs.tomb.shape[0], int(hs.key_off[-1]),
                   int(hs.val_off[-1]))

    def nbytes(self) -> int:
        """Input bytes of this side: arenas, offsets and tombstone flags."""
        return self.key_bytes + self.val_bytes + 8 * (self.n + 1) + self.n


# ---- the C ABI, one wrapper per entry point ----

def em_workspace_bytes(nA: int, nB: int, items_per_part: int) -> int:
    return int(lib().em_workspace_bytes(nA, nB, items_per_part))


def em_rank512_workspace_bytes(nbits: int) -> int:
    return int(lib().em_rank512_workspace_bytes(nbits))


def em_rank2048_workspace_bytes(nbits: int) -> int:
    return int(lib().em_rank2048_workspace_bytes(nbits))


# collision modes (include/em.h)
EM_COLLISION_512, EM_COLLISION_2048, EM_COLLISION_512_TILED, EM_COLLISION_512_COMPACT = 0, 1, 2, 3
COLLISION_MODES = {"512": EM_COLLISION_512, "2048": EM_COLLISION_2048, "512-tiled": EM_COLLISION_512_TILED,
                   "512-compact": EM_COLLISION_512_COMPACT}


def em_collision_workspace_bytes(nA: int, nB: int, mode: int) -> int:
    return int(lib().em_collision_workspace_bytes(nA, nB, mode))


def em_payload_bound_bits(A: DeviceSide, B: DeviceSide) -> int:
    out = ctypes.c_uint64()
    _check(lib().em_payload_bound_bits(ctypes.byref(A.struct), ctypes.byref(B.struct),
                                       ctypes.byref(out)), "em_payload_bound_bits")
    return int(out.value)


def em_partition(A, B, items_per_part, splits, ws, stream=None):
    _check(lib().em_partition(ctypes.byref(A.struct), ctypes.byref(B.struct), items_per_part,
                              _p(splits), _p(ws), ws.numel(), _stream(stream)), "em_partition")


def em_merge_keep(A, B, splits, items_per_part, final_refs, ord_A, ord_B, d_S, ws, stream=None):
    _check(lib().em_merge_keep(ctypes.byref(A.struct), ctypes.byref(B.struct), _p(splits),
                               items_per_part, _p(final_refs), _p(ord_A), _p(ord_B), _p(d_S), _p(ws),
                               ws.numel(), _stream(stream)), "em_merge_keep")


def em_collision_rank(A, B, final_refs, ord_A, ord_B, d_S, ws, stream=None):
    _check(lib().em_collision_rank(ctypes.byref(A.struct), ctypes.byref(B.struct), _p(final_refs),
                                   _p(ord_A), _p(ord_B), _p(d_S), _p(ws), ws.numel(),
                                   _stream(stream)), "em_collision_rank")


def em_fc_lengths(A, B, final_refs, S, len_bits, lcp_bits, ws, stream=None):
    _check(lib().em_fc_lengths(ctypes.byref(A.struct), ctypes.byref(B.struct), _p(final_refs), S,
                               _p(len_bits), _p(lcp_bits), _p(ws), ws.numel(), _stream(stream)),
           "em_fc_lengths")


def em_scan(len_bits, S, off, ws, stream=None):
    _check(lib().em_scan(_p(len_bits), S, _p(off), _p(ws), ws.numel(), _stream(stream)), "em_scan")


def em_scan_noalloc(len_bits, S, off, stream=None):
    _check(lib().em_scan_noalloc(_p(len_bits), S, _p(off), _stream(stream)), "em_scan_noalloc")


def em_emit(A, B, final_refs, lcp_bits, S, off, T, payload, ws, stream=None):
    _check(lib().em_emit(ctypes.byref(A.struct), ctypes.byref(B.struct), _p(final_refs), _p(lcp_bits),
                         S, _p(off), T, _p(payload), payload.numel(), _p(ws), ws.numel(),
                         _stream(stream)), "em_emit")


def em_collision_rank_mode(A, B, mode, final_refs, ord_A, ord_B, d_S, ws, stream=None):
    _check(lib().em_collision_rank_mode(ctypes.byref(A.struct), ctypes.byref(B.struct), mode, _p(final_refs),
                                        _p(ord_A), _p(ord_B), _p(d_S), _p(ws), ws.numel(), _stream(stream)),
           "em_collision_rank_mode")


def em_rank2048_probe(bitmap, nbits, positions, out, ws, stream=None):
    _check(lib().em_rank2048_probe(_p(bitmap), nbits, _p(positions), positions.numel(), _p(out), _p(ws),
                                   ws.numel(), _stream(stream)), "em_rank2048_probe")


def em_rank512_probe(bitmap, nbits, positions, out, ws, stream=None):
    _check(lib().em_rank512_probe(_p(bitmap), nbits, _p(positions), positions.numel(), _p(out), _p(ws),
                                  ws.numel(), _stream(stream)), "em_rank512_probe")


def em_merge_fc_workspace_bytes(nA: int, nB: int, items_per_part: int) -> int:
    return int(lib().em_merge_fc_workspace_bytes(nA, nB, items_per_part))


def em_merge_fc(A, B, coarse_splits, coarse_items, items_per_part, payload, d_S, d_T, ws,
                final_refs=None, ord_A=None, ord_B=None, len_bits=None, lcp_bits=None, off=None,
                stream=None):
    _check(lib().em_merge_fc(ctypes.byref(A.struct), ctypes.byref(B.struct), _p(coarse_splits),
                             coarse_items, items_per_part, _p(payload), payload.numel(), _p(d_S),
                             _p(d_T), _p(final_refs), _p(ord_A), _p(ord_B), _p(len_bits),
                             _p(lcp_bits), _p(off), _p(ws), ws.numel(), _stream(stream)),
           "em_merge_fc")


def em_onepass_workspace_bytes(nA: int, nB: int, items_per_part: int) -> int:
    return int(lib().em_onepass_workspace_bytes(nA, nB, items_per_part))


def em_merge_fc_onepass(A, B, coarse_splits, coarse_items, items_per_part, payload, d_S, d_T, ws,
                        final_refs=None, ord_A=None, ord_B=None, len_bits=None, lcp_bits=None, off=None,
                        stream=None):
    _check(lib().em_merge_fc_onepass(ctypes.byref(A.struct), ctypes.byref(B.struct), _p(coarse_splits),
                                     coarse_items, items_per_part, _p(payload), payload.numel(), _p(d_S),
                                     _p(d_T), _p(final_refs), _p(ord_A), _p(ord_B), _p(len_bits),
                                     _p(lcp_bits), _p(off), _p(ws), ws.numel(), _stream(stream)),
           "em_merge_fc_onepass")


def em_merge_lengths(A, B, coarse_splits, coarse_items, items_per_part, d_S, d_T, ws, final_refs=None,
                     ord_A=None, ord_B=None, len_bits=None, lcp_bits=None, stream=None):
    _check(lib().em_merge_lengths(ctypes.byref(A.struct), ctypes.byref(B.struct), _p(coarse_splits),
                                  coarse_items, items_per_part, _p(d_S), _p(d_T), _p(final_refs), _p(ord_A),
                                  _p(ord_B), _p(len_bits), _p(lcp_bits), _p(ws), ws.numel(), _stream(stream)),
           "em_merge_lengths")


def em_emit_merged(A, B, items_per_part, payload, d_S, d_T, ws, final_refs=None, lcp_bits=None, off=None,
                   stream=None):
    _check(lib().em_emit_merged(ctypes.byref(A.struct), ctypes.byref(B.struct), items_per_part, _p(payload),
                                payload.numel(), _p(d_S), _p(d_T), _p(final_refs), _p(lcp_bits), _p(off),
                                _p(ws), ws.numel(), _stream(stream)), "em_emit_merged")


# ---- output navigation (include/em.h: em_ef_*) ----

EF_INFO_FIELDS = ("n", "L", "width", "low_words", "high_bits", "high_words", "groups", "exceptions")


def em_ef_entry_count(S: int) -> int:
    return int(lib().em_ef_entry_count(S))


def em_ef_capacity(n_entries: int):
    """u64 word capacities (lows, highs, samples, exceptions) for n entries."""
    out = [ctypes.c_uint64() for _ in range(4)]
    _check(lib().em_ef_capacity(n_entries, *[ctypes.byref(o) for o in out]), "em_ef_capacity")
    return tuple(int(o.value) for o in out)


def em_ef_workspace_bytes(n_entries: int) -> int:
    return int(lib().em_ef_workspace_bytes(n_entries))


class EfSections:
    """Device buffers for the navigation sections of n entries (allocated once)."""

    def __init__(self, n_entries: int, device="cuda"):
        import torch
        self.n_entries = n_entries
        caps = em_ef_capacity(n_entries)
        i64 = dict(dtype=torch.int64, device=device)
        self.lows, self.highs, self.samples, self.exceptions = (torch.zeros(max(c, 1), **i64) for c in caps)
        self.info = torch.zeros(len(EF_INFO_FIELDS), **i64)
        self.ws = torch.empty(max(em_ef_workspace_bytes(n_entries), 256), dtype=torch.uint8, device=device)

    def _args(self):
        return (_p(self.lows), self.lows.numel(), _p(self.highs), self.highs.numel(), _p(self.samples),
                self.samples.numel(), _p(self.exceptions), self.exceptions.numel(), _p(self.info), _p(self.ws),
                self.ws.numel())

    def host(self) -> dict:
        """The sections and header as host arrays (synchronizes)."""
        import numpy as np
        info = dict(zip(EF_INFO_FIELDS, (int(x) for x in self.info.cpu().numpy().view(np.uint64))))
        out = dict(info)
        out["n_exceptions"] = out.pop("exceptions")
        cut = {"lows": info["low_words"], "highs": info["high_words"], "samples": 2 * info["groups"],
               "exceptions": info["exceptions"]}
        for k, n in cut.items():
            out[k] = getattr(self, k)[:n].cpu().numpy().view(np.uint64).copy()
        return out


def em_ef_navigation(A, B, final_refs, S, off, T, sec: EfSections, stream=None):
    _check(lib().em_ef_navigation(ctypes.byref(A.struct), ctypes.byref(B.struct), _p(final_refs), S, _p(off), T,
                                  *sec._args(), _stream(stream)), "em_ef_navigation")


def em_ef_encode(entries, width, sec: EfSections, stream=None):
    _check(lib().em_ef_encode(_p(entries), entries.numel(), width, *sec._args(), _stream(stream)), "em_ef_encode")


# ---- front-coded input (include/em.h: em_fcin_*) ----

FCIN_ERRORS = {1: "field past T or bad EG0 code", 2: "inherited prefix longer than the predecessor's key",
               4: "key not whole bytes", 8: "block does not end where the next starts",
               16: "arena of 2^32 bytes or more", 32: "output arena too small"}


def em_fcin_workspace_bytes(S: int) -> int:
    return int(lib().em_fcin_workspace_bytes(S))


def em_fcin_parse(payload, T, S, d_totals, ws, off=None, nav: "EfSections | None" = None, stream=None):
    n = (None,) * 5 if nav is None else (nav.info, nav.lows, nav.highs, nav.samples, nav.exceptions)
    _check(lib().em_fcin_parse(_p(payload), payload.numel(), T, S, _p(off), *[_p(t) for t in n], _p(d_totals),
                               _p(ws), ws.numel(), _stream(stream)), "em_fcin_parse")


def em_fcin_materialize(payload, S, keys, key_off, vals, val_off, tomb, d_totals, ws, stream=None):
    _check(lib().em_fcin_materialize(_p(payload), payload.numel(), S, _p(keys), keys.numel(), _p(key_off),
                                     _p(vals), vals.numel(), _p(val_off), _p(tomb), _p(d_totals), _p(ws),
                                     ws.numel(), _stream(stream)), "em_fcin_materialize")


def em_fcin_prefix8(payload, S, pfx, ws, stream=None):
    _check(lib().em_fcin_prefix8(_p(payload), payload.numel(), S, _p(pfx), _p(ws), ws.numel(), _stream(stream)),
           "em_fcin_prefix8")


def em_fcin_compare(payload_a, S_a, ws_a, payload_b, S_b, ws_b, n, ia, jb, from_byte, lcp_bits=None, cmp=None,
                    stream=None):
    _check(lib().em_fcin_compare(_p(payload_a), payload_a.numel(), S_a, _p(ws_a), ws_a.numel(), _p(payload_b),
                                 payload_b.numel(), S_b, _p(ws_b), ws_b.numel(), n, _p(ia), _p(jb), from_byte,
                                 _p(lcp_bits), _p(cmp), _stream(stream)), "em_fcin_compare")


def fcin_decode(payload, T: int, S: int, off=None, nav: "EfSections | None" = None, device="cuda") -> DeviceSide:
    """Decode a front-coded payload of S records into a DeviceSide (parse,
    read the arena sizes, materialize).  Block starts come from off (u64 record
    offsets) or from the navigation sections."""
    ws = torch.empty(max(em_fcin_workspace_bytes(S), 256), dtype=torch.uint8, device=device)
    d_totals = torch.zeros(3, dtype=torch.int64, device=device)
    em_fcin_parse(payload, T, S, d_totals, ws, off=off, nav=nav)
    kb, vb, err = (int(x) & 0xFFFFFFFFFFFFFFFF for x in d_totals.cpu())
    if err:
        raise EmError(EM_EINVAL, "em_fcin_parse: " + ", ".join(m for b, m in FCIN_ERRORS.items() if err & b), lib())
    keys = torch.zeros(((kb + 15) // 16) * 16 + EM_ARENA_PAD, dtype=torch.uint8, device=device)
    vals = torch.zeros(((vb + 15) // 16) * 16 + EM_ARENA_PAD, dtype=torch.uint8, device=device)
    key_off = torch.empty(S + 1, dtype=torch.int32, device=device)
    val_off = torch.empty(S + 1, dtype=torch.int32, device=device)
    tomb = torch.zeros(max(S, 16), dtype=torch.uint8, device=device)
    em_fcin_materialize(payload, S, keys, key_off, vals, val_off, tomb, d_totals, ws)
    err = int(d_totals[2].item())
    if err:
        raise EmError(EM_EINVAL, "em_fcin_materialize: " + ", ".join(m for b, m in FCIN_ERRORS.items() if err & b),
                      lib())
    return DeviceSide(keys, key_off, vals, val_off, tomb, S, kb, vb)


# ---- byte profile (include/em.h: em_bp_*) ----

def em_bp_workspace_bytes(S: int) -> int:
    return int(lib().em_bp_workspace_bytes(S))


def em_bp_lengths(A, B, final_refs, lcp_bits, S, len_bytes, d_width, ws, stream=None):
    _check(lib().em_bp_lengths(ctypes.byref(A.struct), ctypes.byref(B.struct), _p(final_refs), _p(lcp_bits), S,
                               _p(len_bytes), _p(d_width), _p(ws), ws.numel(), _stream(stream)), "em_bp_lengths")


def em_bp_emit(A, B, final_refs, lcp_bits, S, off, T, d_width, payload, d_overflow, stream=None):
    _check(lib().em_bp_emit(ctypes.byref(A.struct), ctypes.byref(B.struct), _p(final_refs), _p(lcp_bits), S,
                            _p(off), T, _p(d_width), _p(payload), payload.numel(), _p(d_overflow), _stream(stream)),
           "em_bp_emit")


def em_bp_navigation(off, S, T, d_width, sec: "EfSections", stream=None):
    _check(lib().em_bp_navigation(_p(off), S, T, _p(d_width), *sec._args(), _stream(stream)), "em_bp_navigation")
