"""Host orchestration of the hot path.

Paths:
  merge      partition -> merge_keep -> [host reads S] -> fc_lengths -> scan
             -> [host reads T] -> emit  (the six-call C ABI)
  collision  collision_rank instead of partition + merge_keep
  fused      coarse partition -> merge_fc (the whole path in one kernel; S and
             T stay on the device)
All buffers are allocated once up front (sized from em_workspace_bytes and
em_payload_bound_bits) and reused by every run.
"""
from __future__ import annotations

import torch

from . import binding as em


# staged key bytes of one merge partition, by partition size (em_merge_keep.hip)
_KEY_CAP = {256: 26 * 1024, 512: 26 * 1024, 1024: 48 * 1024, 2048: 60 * 1024, 4096: 32 * 1024}


def choose_items_per_part(A: em.DeviceSide, B: em.DeviceSide) -> int:
    """Largest partition (256..4096 outputs) whose keys are expected to fit the
    merge kernel's LDS key buffer, so the partition's comparisons read LDS."""
    n = A.n + B.n
    mean = (A.key_bytes + B.key_bytes) / n if n else 0.0
    best = 256
    for items in (256, 512, 1024, 2048, 4096):
        if items * (mean * 1.1 + 4) <= _KEY_CAP[items]:
            best = items
    return best


# staged key and value bytes of one partition in the fused kernel
_FUSE_KEY_CAP, _FUSE_VAL_CAP, _FUSE_MAX_ITEMS, _FUSE_COARSE_PARTS = 14 * 1024, 12 * 1024, 256, 16


def choose_fused_items(A: em.DeviceSide, B: em.DeviceSide) -> int:
    """Largest partition (32..256 outputs) whose key and value bytes are expected
    to fit the fused kernel's LDS staging buffers."""
    n = A.n + B.n
    mk = (A.key_bytes + B.key_bytes) / n if n else 0.0
    mv = (A.val_bytes + B.val_bytes) / n if n else 0.0
    best = 32
    for items in (32, 64, 128, 256):
        if (items + 3) * (mk * 1.1) + 64 <= _FUSE_KEY_CAP and items * (mv * 1.1) + 64 <= _FUSE_VAL_CAP:
            best = items
    return best


class Pipeline:
    def __init__(self, A: em.DeviceSide, B: em.DeviceSide, items_per_part: int | None = None,
                 path: str = "merge", keep_ordinals: bool = True, keep_lcp: bool = True,
                 keep_all: bool = True, coarse_parts: int = _FUSE_COARSE_PARTS, device="cuda"):
        if path not in ("merge", "collision", "fused"):
            raise ValueError("path is 'merge', 'collision' or 'fused'")
        self.A, self.B = A, B
        if path == "fused":
            self.items = int(items_per_part) if items_per_part else choose_fused_items(A, B)
            self.coarse = self.items * coarse_parts
        else:
            self.items = int(items_per_part) if items_per_part else choose_items_per_part(A, B)
            self.coarse = 0
        self.path = path
        self.keep_all = keep_all
        N = A.n + B.n
        self.N = N
        P = (N + (self.coarse or self.items) - 1) // (self.coarse or self.items)
        i32 = dict(dtype=torch.int32, device=device)
        self.splits = torch.empty(P + 1, **i32)
        self.final = torch.empty(max(N, 1), **i32)
        self.ord_A = torch.empty(max(A.n, 1), **i32) if keep_ordinals else None
        self.ord_B = torch.empty(max(B.n, 1), **i32) if keep_ordinals else None
        self.d_S = torch.zeros(1, **i32)
        self.len_bits = torch.empty(max(N, 1) + 4, **i32)
        self.lcp = torch.empty(max(N, 1), **i32) if keep_lcp else None
        self.off = torch.empty(N + 1, dtype=torch.int64, device=device)
        self.d_T = torch.zeros(1, dtype=torch.int64, device=device)
        self.bound_bits = em.em_payload_bound_bits(A, B)
        self.payload = torch.empty((self.bound_bits + 31) // 32 + 1, **i32)
        ws_bytes = em.em_workspace_bytes(A.n, B.n, min(self.items, 4096))
        if path == "fused":
            ws_bytes = max(ws_bytes, em.em_merge_fc_workspace_bytes(A.n, B.n, self.items))
        self.ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=device)
        self.S = 0
        self.T = 0

    def run(self, stream=None, read_counts: bool = True):
        """One pass of the whole path.  Returns (S, T).

        The fused path needs no host read between its calls; with
        read_counts=False it leaves S and T on the device (read_counts()).
        """
        A, B = self.A, self.B
        if self.path == "fused":
            em.em_partition(A, B, self.coarse, self.splits, self.ws, stream)
            k = self.keep_all
            em.em_merge_fc(A, B, self.splits, self.coarse, self.items, self.payload, self.d_S, self.d_T,
                           self.ws, final_refs=self.final if k else None,
                           ord_A=self.ord_A if k else None, ord_B=self.ord_B if k else None,
                           len_bits=self.len_bits if k else None, lcp_bits=self.lcp if k else None,
                           off=self.off if k else None, stream=stream)
            if read_counts:
                self.read_counts()
            return self.S, self.T
        if self.path == "merge":
            em.em_partition(A, B, self.items, self.splits, self.ws, stream)
            em.em_merge_keep(A, B, self.splits, self.items, self.final, self.ord_A, self.ord_B,
                             self.d_S, self.ws, stream)
        else:
            em.em_collision_rank(A, B, self.final, self.ord_A, self.ord_B, self.d_S, self.ws, stream)
        S = int(self.d_S.item()) & 0xFFFFFFFF
        em.em_fc_lengths(A, B, self.final, S, self.len_bits, self.lcp, self.ws, stream)
        em.em_scan(self.len_bits, S, self.off, self.ws, stream)
        T = int(self.off[S].item())
        em.em_emit(A, B, self.final, self.lcp, S, self.off, T, self.payload, self.ws, stream)
        self.S, self.T = S, T
        return S, T

    def read_counts(self):
        self.S = int(self.d_S.item()) & 0xFFFFFFFF
        self.T = int(self.d_T.item())
        return self.S, self.T

    # ---- host copies of the results (for checks; not part of a run) ----

    def payload_bytes(self) -> bytes:
        nw = (self.T + 31) // 32
        return self.payload[:nw].cpu().numpy().tobytes()

    def host(self, name: str, count: int | None = None):
        t = getattr(self, name)
        if count is not None:
            t = t[:count]
        a = t.cpu().numpy()
        return a.view("uint32") if a.dtype.itemsize == 4 else a.view("uint64")
