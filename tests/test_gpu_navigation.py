"""GPU parity of the output navigation (em_ef_navigation, em_ef_encode)
against the CPU oracle, bit for bit: the header, packed lows, high bits,
sample pairs and exception positions, on merged payloads of every generated
workload (through the six-call and the fused paths), a fixed value width, an
empty merge, and crafted entry sequences (repeats, one entry, group edges,
the exact 4095/4096-bit sparse threshold, wide gaps)."""
import numpy as np
import pytest

import gen
import oracle
import torch  # imported at collection so that its first-load time is not charged to a test
from gpu_util import require_gpu, run_gpu, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _same(got, want, label):
    for k in ("n", "L", "width", "low_words", "high_bits", "high_words", "groups", "n_exceptions"):
        assert got[k] == want[k], f"{label}: {k} {got[k]} != {want[k]}"
    for k in ("lows", "highs", "samples", "exceptions"):
        g, w = got[k], np.asarray(want[k], np.uint64)
        assert g.size == w.size, f"{label}: {k} has {g.size} words, oracle {w.size}"
        bad = np.nonzero(g != w)[0]
        assert bad.size == 0, f"{label}: {k} differs at word {bad[:5]}"


def _check_pipeline(Ah, Bh, label, path="merge"):
    pl = run_gpu(Ah, Bh, items=None if path == "fused" else 256, path=path)
    sec = pl.ef_navigation()
    torch.cuda.synchronize()
    S, T = pl.S, pl.T
    ref = oracle.run(Ah, Bh, items_per_part=256)
    assert (S, T) == (ref["S"], ref["T"])
    want = oracle.ef_navigation(Ah, Bh, ref["final"], ref["off"], ref["T"])
    _same(sec.host(), want, label)
    return want


@pytest.mark.parametrize("wid,scale", [(1, 1.0), (2, 0.01), (3, 0.002), (4, 0.002), (5, 0.005)])
def test_navigation_of_generated_workloads(wid, scale):
    A, B = workload(wid, scale)
    print(f"navigation workload {wid} at {scale}: {A.n}+{B.n}", flush=True)
    _check_pipeline(A, B, f"w{wid}/merge")
    _check_pipeline(A, B, f"w{wid}/fused", path="fused")


def test_navigation_fixed_width_and_empty():
    keys = [b"key%06d" % i for i in range(5000)]
    rng = np.random.default_rng(3)
    A = gen.side_from_records([(k, rng.bytes(16)) for k in keys[::2]])
    B = gen.side_from_records([(k, rng.bytes(16)) for k in keys[1::3]])
    print("navigation, every value 16 bytes", flush=True)
    want = _check_pipeline(A, B, "fixed width")
    assert want["width"] == 1 + 9 + 128
    empty = gen.side_from_records([])
    print("navigation, empty merge", flush=True)
    want = _check_pipeline(empty, empty, "empty")
    assert want["n"] == 1


def _encode(e, width=0):
    import merge_front_coded_amd as em
    e = np.asarray(e, np.uint64)
    dev = torch.from_numpy(e.view(np.int64)).cuda()
    sec = em.EfSections(int(e.size))
    em.em_ef_encode(dev, width, sec)
    torch.cuda.synchronize()
    return sec.host()


def test_encode_crafted_entries():
    rng = np.random.default_rng(9)
    cases = {
        "one entry": [0],
        "one large entry": [123456789],
        "repeats": [0, 0, 0, 1, 1, 5, 5, 5],
        "hand example": [0, 5, 9, 20],
    }
    for n in (255, 256, 257, 513, 4097):
        cases[f"uniform n={n}"] = np.cumsum(rng.integers(0, 1000, n))
        cases[f"clustered n={n}"] = np.cumsum(np.where(rng.random(n) < 0.02, rng.integers(10 ** 5, 10 ** 7, n),
                                                       rng.integers(0, 3, n)))
    cases["wide gaps"] = np.cumsum(rng.integers(0, 2 ** 40, 3000, dtype=np.int64))
    for top in (3839, 3840):  # the 4095/4096-bit span of group 0 (L = 0)
        cases[f"threshold top={top}"] = np.concatenate([np.linspace(0, top, 256).round(),
                                                        np.full(2048 - 256, 3840)])
    for name, e in cases.items():
        e = np.asarray(e, np.uint64)
        print(f"encode: {name} ({e.size} entries)", flush=True)
        _same(_encode(e, 7), oracle.ef_encode(e, 7), name)
