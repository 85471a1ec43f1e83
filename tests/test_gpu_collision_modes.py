"""GPU parity of the four collision-path modes (rank512 with independent
searches, rank2048, rank512 with 32-record A tiles, rank512 with a compact A
list merged by Merge Path) against the CPU oracle, bit for bit, on the edge
cases of the keep step: empty sides, all and no collisions, proper-prefix and
binary keys, dense collisions, a skewed pair of sides and more outputs than
one compact-merge workgroup takes."""
import random

import pytest

import gen
import torch  # imported at collection so that its first-load time is not charged to a test
from gpu_util import check_path, require_gpu, workload

pytestmark = pytest.mark.gpu

MODES = ["512", "2048", "512-tiled", "512-compact"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _rand_bytes(rng, lo, hi):
    return bytes(rng.randrange(256) for _ in range(rng.randrange(lo, hi + 1)))


def _check(A, B, mode, label):
    print(f"collision {mode}: {label} ({A.n}+{B.n})", flush=True)
    return check_path(A, B, items=64, path="collision", collision_mode=mode, label=f"{mode}/{label}")


@pytest.mark.parametrize("mode", MODES)
def test_modes_on_generated_workloads(mode):
    A, B = workload(1)
    _check(A, B, mode, "uniform 10k+10k")
    for wid, scale in ((2, 0.01), (3, 0.001), (4, 0.002), (5, 0.004)):
        A, B = workload(wid, scale)
        _check(A, B, mode, f"workload {wid} at {scale}")


@pytest.mark.parametrize("mode", MODES)
def test_modes_on_edge_cases(mode):
    rng = random.Random(11)
    keys = sorted({_rand_bytes(rng, 1, 12) for _ in range(3000)})
    full = gen.side_from_records([(k, _rand_bytes(rng, 0, 9)) for k in keys])
    empty = gen.side_from_records([])
    for A, B, name in ((empty, full, "A empty"), (full, empty, "B empty"), (empty, empty, "both empty")):
        pl, _ = _check(A, B, mode, name)
        if name == "both empty":
            assert pl.S == 0 and pl.T == 0
    # every key collides (B has tombstones), and no key collides
    B_all = gen.side_from_records([(k, None if rng.random() < 0.3 else _rand_bytes(rng, 0, 9)) for k in keys])
    _check(full, B_all, mode, "all collide")
    _check(gen.side_from_records([(k, b"a") for k in keys[::2]]),
           gen.side_from_records([(k, b"b") for k in keys[1::2]]), mode, "none collide")
    # proper prefixes and binary bytes (all strings of length <= 3 over 6 symbols)
    import itertools
    alpha = [0x00, 0x01, 0x7F, 0x80, 0xFE, 0xFF]
    bkeys = sorted([b""] + [bytes(t) for L in (1, 2, 3) for t in itertools.product(alpha, repeat=L)])
    a, b = [], []
    for k in bkeys:
        u = rng.random()
        if u < 0.4:
            a.append((k, _rand_bytes(rng, 0, 5)))
            b.append((k, None if rng.random() < 0.2 else _rand_bytes(rng, 0, 5)))
        elif u < 0.7:
            a.append((k, None if rng.random() < 0.2 else _rand_bytes(rng, 0, 5)))
        else:
            b.append((k, _rand_bytes(rng, 0, 5)))
    _check(gen.side_from_records(a), gen.side_from_records(b), mode, "byte keys with proper prefixes")
    # a large older side and a small newer side, collisions at bitmap word and
    # rank block edges
    big = [b"k%07d" % i for i in range(9000)]
    hits = sorted({i for i in (0, 31, 32, 33, 511, 512, 513, 2047, 2048, 2049, 8999)} |
                  {rng.randrange(9000) for _ in range(40)})
    A = gen.side_from_records([(k, b"old") for k in big])
    B = gen.side_from_records(sorted([(big[i], b"new") for i in hits] + [(b"k%07d+" % i, None) for i in (5, 600)]))
    _check(A, B, mode, "skewed, collisions at block edges")
