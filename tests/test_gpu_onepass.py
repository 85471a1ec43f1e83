"""GPU parity of the single-pass call (em_merge_fc_onepass): every output --
payload, S, T, survivors, ordinals, lengths, LCPs, offsets -- element by
element against the CPU oracle, for every partition size and coarse split,
on the generated workloads (including the long shared prefixes of the path
and URL keys, where the prefix cache moves to the common prefix), on records
longer than the LDS window (one record over several slices, and over
partition boundaries), on chunks whose values do not fit the stage, on empty
sides, on partitions without survivors and on tiny last partitions."""
import random

import numpy as np
import pytest

import gen
import oracle
import torch  # imported at collection so that its first-load time is not charged to a test
from gpu_util import check_path, require_gpu, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("items,coarse_parts", [(1, 1), (1, 16), (3, 5), (17, 16), (64, 2), (255, 16), (256, 1),
                                                (257, 1), (511, 3), (512, 4), (513, 2), (1000, 1), (1024, 4),
                                                (1024, 1)])
def test_onepass_every_partition_size(items, coarse_parts):
    A, B = workload(1, 0.3)
    print(f"one pass uniform-az 3000+3000 items={items} coarse={coarse_parts}", flush=True)
    check_path(A, B, items=items, path="fused", coarse_parts=coarse_parts, one_pass=True)


@pytest.mark.parametrize("wid,scale", [(1, 1.0), (2, 0.01), (3, 0.002), (4, 0.002), (5, 0.005)])
def test_onepass_generated_workloads(wid, scale):
    A, B = workload(wid, scale)
    print(f"one pass workload {wid} at {scale}", flush=True)
    check_path(A, B, items=None, path="fused", one_pass=True)


def test_onepass_long_records_and_edges():
    rng = np.random.default_rng(21)
    # values up to 40 KB: one record spans several window slices (and, with
    # small partitions, partition boundaries fall inside long runs of bits)
    keys = [b"long%05d" % i for i in range(300)]
    vals = [rng.bytes(40000) if i % 13 == 0 else (None if i % 5 == 0 else rng.bytes(int(rng.integers(0, 50))))
            for i in range(300)]
    A = gen.side_from_records(list(zip(keys[::2], vals[::2])))
    B = gen.side_from_records(list(zip(keys[1::2], vals[1::2])))
    for items in (1, 7, 64, 512, 1024):
        print(f"one pass long records items={items}", flush=True)
        check_path(A, B, items=items, path="fused", one_pass=True)
    # every key in both sides (half the outputs dropped), one side empty,
    # both empty, a last partition of one record
    r = random.Random(3)
    ks = sorted({bytes(r.randrange(256) for _ in range(r.randrange(0, 9))) for _ in range(700)})
    both = gen.side_from_records([(k, b"a") for k in ks])
    newer = gen.side_from_records([(k, None if i % 4 == 0 else b"bb") for i, k in enumerate(ks)])
    empty = gen.side_from_records([])
    for label, (X, Y) in {"all collide": (both, newer), "A empty": (empty, newer), "B empty": (both, empty),
                          "both empty": (empty, empty)}.items():
        for items in (1, 64, 1024):
            print(f"one pass {label} items={items}", flush=True)
            check_path(X, Y, items=items, path="fused", one_pass=True)
    n = 2 * 64 + 1
    one_more = gen.side_from_records([(b"k%04d" % i, b"v" * (i % 3)) for i in range(n)])
    check_path(one_more, empty, items=64, path="fused", one_pass=True)


@pytest.mark.parametrize("items", [1, 64, 256, 512, 1024])
def test_onepass_long_common_prefixes(items):
    """Keys sharing long prefixes, so that the prefix cache moves to the
    partition's common prefix: a 37-byte prefix with short tails (some keys
    equal to the prefix itself), B keys that leave the prefix after 9 bytes,
    and tails that differ only past the cached eight bytes."""
    rng = random.Random(40 + items)
    base = b"https://host-%02d.example/" % 7 + b"a" * 13  # 37 bytes
    keys = set()
    for _ in range(2500):
        tail = bytes(rng.choice(b"ab\x00\xff") for _ in range(rng.randrange(0, 13)))
        keys.add(base + tail)
        keys.add(base[:9] + bytes([rng.randrange(256)]) + tail)
        keys.add(base + b"Z" * 8 + tail)  # ties on the cached bytes
    keys = sorted(keys)
    a_keys = [k for i, k in enumerate(keys) if i % 3 != 1]
    b_keys = [k for i, k in enumerate(keys) if i % 3 != 0]
    A = gen.side_from_records([(k, bytes(rng.randrange(256) for _ in range(rng.randrange(0, 9)))) for k in a_keys])
    B = gen.side_from_records([(k, None if rng.random() < 0.1 else b"v" * rng.randrange(0, 5)) for k in b_keys])
    print(f"one pass long common prefixes items={items}: {A.n}+{B.n}", flush=True)
    check_path(A, B, items=items, path="fused", one_pass=True)
