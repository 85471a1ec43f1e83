"""Host orchestration of the hot path.

Paths:
  merge      partition -> merge_keep -> [host reads S] -> fc_lengths -> scan
             -> [host reads T] -> emit  (the six-call C ABI)
  collision  collision_rank_mode (collision_mode: "512", "2048", "512-tiled",
             "512-compact") instead of partition + merge_keep
  fused      partition -> merge_lengths (merge, keep, LCPs, lengths, bit
             offsets) -> emit_merged (the emitter); S and T stay on the
             device.  one_call=True runs the same work as em_merge_fc;
             one_pass=True runs partition -> em_merge_fc_onepass (each
             partition emits its own words; 512 outputs per partition,
             whose co-ranks em_partition finds).
All buffers are allocated once up front (sized from em_workspace_bytes and
em_payload_bound_bits) and reused by every run.
"""
from __future__ import annotations

import torch

from . import binding as em


def choose_items_per_part(A: em.DeviceSide, B: em.DeviceSide) -> int:
    """Partition size of the merge: 2048 outputs (LDS holds offsets and 8-byte
    prefixes only, so two or three partitions share a compute unit), smaller
    for small inputs so that every compute unit still gets partitions."""
    n = A.n + B.n
    for items in (2048, 1024, 512):
        if n >= items * 512:
            return items
    return 256


_FUSE_COARSE_PARTS = 1


def choose_onepass_items(A: em.DeviceSide, B: em.DeviceSide) -> int:
    """Partition size of the single pass: 512 outputs (four 256-thread
    workgroups, 40 KB of LDS each, share a compute unit), 256 for inputs too
    small to give every compute unit partitions."""
    return 512 if A.n + B.n >= 512 * 512 else 256


def choose_fused_items(A: em.DeviceSide, B: em.DeviceSide) -> int:
    """Partition size of em_merge_fc's first kernel (at most 2048 outputs; the
    same choice as the merge path)."""
    return choose_items_per_part(A, B)


class Pipeline:
    def __init__(self, A: em.DeviceSide, B: em.DeviceSide, items_per_part: int | None = None,
                 path: str = "merge", keep_ordinals: bool = True, keep_lcp: bool = True,
                 keep_all: bool = True, coarse_parts: int = _FUSE_COARSE_PARTS, one_call: bool = False,
                 collision_mode: str = "512-tiled", one_pass: bool = False, device="cuda"):
        if path not in ("merge", "collision", "fused"):
            raise ValueError("path is 'merge', 'collision' or 'fused'")
        self.A, self.B = A, B
        if path == "fused" and one_pass:
            self.items = int(items_per_part) if items_per_part else choose_onepass_items(A, B)
            self.coarse = self.items * coarse_parts
        elif path == "fused":
            self.items = int(items_per_part) if items_per_part else choose_fused_items(A, B)
            self.coarse = self.items * coarse_parts
        else:
            self.items = int(items_per_part) if items_per_part else choose_items_per_part(A, B)
            self.coarse = 0
        self.path = path
        if collision_mode not in em.COLLISION_MODES:
            raise ValueError(f"collision_mode is one of {sorted(em.COLLISION_MODES)}")
        self.collision_mode = em.COLLISION_MODES[collision_mode]
        self.keep_all = keep_all
        self.one_call = one_call
        self.one_pass = one_pass
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
            if one_pass:
                ws_bytes = max(ws_bytes, em.em_onepass_workspace_bytes(A.n, B.n, self.items))
        if path == "collision":
            ws_bytes = max(ws_bytes, em.em_collision_workspace_bytes(A.n, B.n, self.collision_mode))
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
            outs = dict(final_refs=self.final if k else None, ord_A=self.ord_A if k else None,
                        ord_B=self.ord_B if k else None, len_bits=self.len_bits if k else None,
                        lcp_bits=self.lcp if k else None)
            if self.one_pass:
                em.em_merge_fc_onepass(A, B, self.splits, self.coarse, self.items, self.payload, self.d_S,
                                       self.d_T, self.ws, off=self.off if k else None, stream=stream, **outs)
            elif self.one_call:
                em.em_merge_fc(A, B, self.splits, self.coarse, self.items, self.payload, self.d_S, self.d_T,
                               self.ws, off=self.off if k else None, stream=stream, **outs)
            else:
                em.em_merge_lengths(A, B, self.splits, self.coarse, self.items, self.d_S, self.d_T, self.ws,
                                    stream=stream, **outs)
                em.em_emit_merged(A, B, self.items, self.payload, self.d_S, self.d_T, self.ws,
                                  final_refs=outs["final_refs"], lcp_bits=outs["lcp_bits"],
                                  off=self.off if k else None, stream=stream)
            if read_counts:
                self.read_counts()
            return self.S, self.T
        if self.path == "merge":
            em.em_partition(A, B, self.items, self.splits, self.ws, stream)
            em.em_merge_keep(A, B, self.splits, self.items, self.final, self.ord_A, self.ord_B,
                             self.d_S, self.ws, stream)
        else:
            em.em_collision_rank_mode(A, B, self.collision_mode, self.final, self.ord_A, self.ord_B, self.d_S,
                                      self.ws, stream)
        S = int(self.d_S.item()) & 0xFFFFFFFF
        em.em_fc_lengths(A, B, self.final, S, self.len_bits, self.lcp, self.ws, stream)
        em.em_scan(self.len_bits, S, self.off, self.ws, stream)
        T = int(self.off[S].item())
        em.em_emit(A, B, self.final, self.lcp, S, self.off, T, self.payload, self.ws, stream)
        self.S, self.T = S, T
        return S, T

    def ef_navigation(self, stream=None):
        """The output navigation sections of the last run (em_ef_navigation),
        into buffers allocated on first use for the largest possible S.  Needs
        the survivors' references and offsets: any path but the fused one with
        keep_all=False."""
        if self.path == "fused" and not self.keep_all:
            raise ValueError("the fused path keeps final refs and offsets only with keep_all=True")
        if getattr(self, "nav", None) is None:
            self.nav = em.EfSections(em.em_ef_entry_count(self.N))
        if self.path == "fused":
            self.read_counts()
        em.em_ef_navigation(self.A, self.B, self.final, self.S, self.off, self.T, self.nav, stream)
        return self.nav

    def byte_profile(self, stream=None):
        """The byte-profile encoding of the last run's survivors (em_bp_lengths,
        em_scan, em_bp_emit): returns (width, T in bytes); the payload is in
        self.bp_payload, the byte offsets in self.bp_off.  Needs the
        survivors' references and LCPs: any path but the fused one with
        keep_all=False."""
        if self.path == "fused" and not self.keep_all:
            raise ValueError("the fused path keeps final refs and LCPs only with keep_all=True")
        if self.lcp is None:
            raise ValueError("the byte profile needs the bit LCPs (keep_lcp=True)")
        if self.path == "fused":
            self.read_counts()
        S = self.S
        if getattr(self, "bp_len", None) is None:
            i32 = dict(dtype=torch.int32, device=self.final.device)
            self.bp_len = torch.empty(max(self.N, 1) + 4, **i32)
            self.bp_off = torch.empty(self.N + 1, dtype=torch.int64, device=self.final.device)
            self.bp_width = torch.zeros(1, **i32)
            self.bp_over = torch.zeros(1, **i32)
            self.bp_ws = torch.empty(max(em.em_bp_workspace_bytes(self.N), 256), dtype=torch.uint8,
                                     device=self.final.device)
            self.bp_payload = None  # sized from T at the first call
        em.em_bp_lengths(self.A, self.B, self.final, self.lcp, S, self.bp_len, self.bp_width, self.bp_ws, stream)
        em.em_scan(self.bp_len, S, self.bp_off, self.ws, stream)
        T = int(self.bp_off[S].item())
        W = int(self.bp_width.item())
        if self.bp_payload is None or self.bp_payload.numel() < T:
            self.bp_payload = torch.zeros(max(T, 1) + 16, dtype=torch.uint8, device=self.final.device)
        em.em_bp_emit(self.A, self.B, self.final, self.lcp, S, self.bp_off, T, self.bp_width, self.bp_payload,
                      self.bp_over, stream)
        return W, T

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
