"""Shared helpers of the GPU tests: run the HIP path through the C ABI and
compare every output with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import functools

import numpy as np

import gen
import oracle


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (run the CPU suite with -m 'not gpu')")


@functools.lru_cache(maxsize=8)
def workload(wid: int, scale: float = 1.0):
    """Seeded inputs, generated once per process."""
    w = gen.WORKLOADS[wid] if scale == 1.0 else gen.WORKLOADS[wid].scaled(scale)
    return gen.make(w)


def run_gpu(Ah, Bh, items=2048, path="merge", keep_lcp=True, **kw):
    import merge_front_coded_amd as em
    A = em.DeviceSide.from_host(Ah)
    B = em.DeviceSide.from_host(Bh)
    pl = em.Pipeline(A, B, items_per_part=items, path=path, keep_lcp=keep_lcp, **kw)
    pl.run()
    return pl


def compare(pl, ref, Ah, Bh, check_splits=True, label=""):
    """Element-by-element parity of every output of the path."""
    import torch
    torch.cuda.synchronize()
    S = pl.S
    assert S == ref["S"], f"{label}: S {S} != {ref['S']}"
    N = Ah.n + Bh.n
    if check_splits and pl.path == "merge":
        got = pl.host("splits")
        want = ref["splits"]
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"{label}: splits differ at {bad[:5]} got {got[bad[:5]]} want {want[bad[:5]]}"
    if N:
        got = pl.host("final", S)
        bad = np.nonzero(got != ref["final"])[0]
        assert bad.size == 0, f"{label}: final refs differ at {bad[:5]}: {got[bad[:5]]} vs {ref['final'][bad[:5]]}"
    if Ah.n:
        got = pl.host("ord_A", Ah.n)
        bad = np.nonzero(got != ref["ord_A"])[0]
        assert bad.size == 0, f"{label}: ord_A differs at {bad[:5]}"
    if Bh.n:
        got = pl.host("ord_B", Bh.n)
        bad = np.nonzero(got != ref["ord_B"])[0]
        assert bad.size == 0, f"{label}: ord_B differs at {bad[:5]}"
    if S:
        got = pl.host("len_bits", S)
        bad = np.nonzero(got != ref["len_bits"])[0]
        assert bad.size == 0, f"{label}: len_bits differ at {bad[:5]}: {got[bad[:5]]} vs {ref['len_bits'][bad[:5]]}"
        if pl.lcp is not None:
            got = pl.host("lcp", S)
            bad = np.nonzero(got != ref["lcp_bits"])[0]
            assert bad.size == 0, f"{label}: lcp differs at {bad[:5]}"
    got = pl.host("off", S + 1)
    bad = np.nonzero(got != ref["off"])[0]
    assert bad.size == 0, f"{label}: off differs at {bad[:5]}"
    assert pl.T == ref["T"], f"{label}: T {pl.T} != {ref['T']}"
    got = np.frombuffer(pl.payload_bytes(), np.uint8)
    want = ref["payload"]
    assert got.size == want.size, f"{label}: payload size {got.size} != {want.size}"
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{label}: payload differs first at byte {bad[0]} (bit {8 * bad[0]}) of {got.size}"


def check_path(Ah, Bh, items=2048, path="merge", keep_lcp=True, label="", **kw):
    if path == "fused" and items and items > 2048:
        items = 2048
    ref = oracle.run(Ah, Bh, items_per_part=items or 256)
    pl = run_gpu(Ah, Bh, items=items, path=path, keep_lcp=keep_lcp, **kw)
    compare(pl, ref, Ah, Bh, label=label or f"{path}/items={items}")
    return pl, ref
