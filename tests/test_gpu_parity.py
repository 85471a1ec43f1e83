"""GPU parity: the HIP path through the C ABI against the CPU oracle, bit for
bit, on seeded inputs that span many tiles and end in ragged tails, plus the
edge cases of the method (empty sides, all/no collisions, proper-prefix and
binary keys, long records, equal pairs split by partition boundaries, the W15
phase)."""
import random

import numpy as np
import pytest

import gen
import oracle
import torch  # imported at collection so that its first-load time is not charged to a test
from gpu_util import check_path, compare, require_gpu, run_gpu, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _records_side(recs):
    return gen.side_from_records(recs)


def _rand_bytes(rng, lo, hi):
    return bytes(rng.randrange(256) for _ in range(rng.randrange(lo, hi + 1)))


def _split(keys, rng, p_both=0.3, p_tomb=0.1, vmax=40, tomb_a=False):
    a, b = [], []
    for k in keys:
        u = rng.random()
        val = lambda: None if rng.random() < p_tomb else _rand_bytes(rng, 0, vmax)
        if u < p_both:
            a.append((k, None if (tomb_a and rng.random() < p_tomb) else _rand_bytes(rng, 0, vmax)))
            b.append((k, val()))
        elif u < (1 + p_both) / 2:
            a.append((k, None if (tomb_a and rng.random() < p_tomb) else _rand_bytes(rng, 0, vmax)))
        else:
            b.append((k, val()))
    return _records_side(a), _records_side(b)


@pytest.mark.parametrize("items", [1, 3, 7, 64, 255, 256, 1000, 2048, 4096])
def test_uniform_workload_every_partition_size(items):
    A, B = workload(1, 0.3)
    print(f"uniform-az 3000+3000 items={items}", flush=True)
    check_path(A, B, items=items)


def test_uniform_workload_full_10k():
    A, B = workload(1)
    print("uniform-az 10k+10k", flush=True)
    check_path(A, B, items=2048)
    check_path(A, B, items=2048, path="collision")
    check_path(A, B, items=256, path="fused")


@pytest.mark.parametrize("items,coarse_parts", [(1, 1), (1, 16), (3, 5), (17, 16), (64, 2), (100, 3),
                                                (255, 16), (256, 1), (256, 16), (513, 2), (1000, 1),
                                                (1024, 1), (1024, 4)])
def test_fused_every_partition_size(items, coarse_parts):
    A, B = workload(1, 0.3)
    print(f"fused uniform-az 3000+3000 items={items} coarse={coarse_parts}", flush=True)
    check_path(A, B, items=items, path="fused", coarse_parts=coarse_parts)


@pytest.mark.parametrize("wid,scale", [(5, 0.02), (2, 0.08), (3, 0.005)])
def test_fused_after_the_sampled_partitions(wid, scale):
    """Several hundred 256-output partitions, past the 128 that always try the
    merge on cached prefixes: on the URL and path inputs most partitions then
    go straight to the exact merge, on the base64 inputs they keep trying the
    cached one; the outputs are exact either way."""
    A, B = workload(wid, scale)
    P = -(-(A.n + B.n) // 256)
    print(f"workload {wid} at {scale}: {A.n}+{B.n}, {P} partitions", flush=True)
    assert P > 300
    check_path(A, B, items=256, path="fused")


@pytest.mark.parametrize("scale,items", [(0.4096, 1), (0.4097, 1), (1.0, 2), (1.0, 1)])
def test_fused_many_partitions(scale, items):
    """8192, 8194, 10000 and 20000 partitions: the scan of partition bit
    totals keeps up to eight values per thread in registers and loops above
    that (8192 is the last count that fits)."""
    A, B = workload(1, scale)
    P = -(-(A.n + B.n) // items)
    print(f"fused uniform-az {A.n}+{B.n} items={items}: {P} partitions", flush=True)
    check_path(A, B, items=items, path="fused")


@pytest.mark.parametrize("items", [64, 1024, 2048])
def test_fused_one_call_matches_oracle(items):
    """em_merge_fc (both halves in one call) gives the same outputs."""
    A, B = workload(2, 0.01)
    print(f"fused one call zipf-paths 10k+10k items={items}", flush=True)
    check_path(A, B, items=items, path="fused", one_call=True)


def test_empty_sides():
    rng = random.Random(1)
    keys = sorted({_rand_bytes(rng, 1, 12) for _ in range(300)})
    full = _records_side([(k, _rand_bytes(rng, 0, 9)) for k in keys])
    empty = _records_side([])
    for A, B, name in ((empty, full, "A empty"), (full, empty, "B empty"), (empty, empty, "both empty")):
        print(name, flush=True)
        for path in ("merge", "collision", "fused"):
            pl, ref = check_path(A, B, items=64, path=path, label=f"{name}/{path}")
            if name == "both empty":
                assert pl.S == 0 and pl.T == 0


def test_all_and_no_collisions():
    rng = random.Random(2)
    keys = sorted({_rand_bytes(rng, 1, 20) for _ in range(5000)})
    A = _records_side([(k, _rand_bytes(rng, 0, 16)) for k in keys])
    B = _records_side([(k, None if rng.random() < 0.3 else _rand_bytes(rng, 0, 16)) for k in keys])
    for path in ("merge", "collision", "fused"):
        check_path(A, B, items=256, path=path, label=f"all collide/{path}")
    A2 = _records_side([(k, b"a") for k in keys[::2]])
    B2 = _records_side([(k, b"b") for k in keys[1::2]])
    for path in ("merge", "collision", "fused"):
        check_path(A2, B2, items=256, path=path, label=f"none collide/{path}")


def test_proper_prefix_and_binary_keys():
    # all strings of length <= 3 over {00, 01, 61, 7F, 80, FE, FF}
    alpha = [0x00, 0x01, 0x61, 0x7F, 0x80, 0xFE, 0xFF]
    keys = [b""]
    for L in (1, 2, 3):
        import itertools
        keys += [bytes(t) for t in itertools.product(alpha, repeat=L)]
    keys.sort()
    rng = random.Random(3)
    for trial in range(4):
        A, B = _split(keys, rng, p_both=0.4, p_tomb=0.2, vmax=12, tomb_a=True)
        for items in (5, 256, 2048):
            for path in ("merge", "collision", "fused"):
                check_path(A, B, items=items, path=path, label=f"binary trial {trial}/{items}/{path}")


def test_long_records_span_many_words():
    rng = random.Random(4)
    keys = sorted({b"common/prefix/" * rng.randrange(0, 20) + _rand_bytes(rng, 1, 200) for _ in range(600)})
    recs = [(k, _rand_bytes(rng, 0, 3000)) for k in keys]
    A = _records_side(recs[::2])
    B = _records_side([(k, None if i % 4 == 0 else v) for i, (k, v) in enumerate(recs[1::2])])
    for path in ("merge", "collision", "fused"):
        check_path(A, B, items=64, path=path)
    # records much longer than a staging buffer or the output window
    check_path(A, B, items=256, path="fused", label="fused, long records")
    # emitter recomputing l when no lcp array is kept
    check_path(A, B, items=64, keep_lcp=False, label="emit without lcp array")


def test_staged_chunks_over_several_slices():
    """Records of about 500 bytes (keys of 50-150 bytes, values of 0-800):
    the emitter sizes its chunks to fill about 90% of its output window
    (about 18 records here), so with this spread about one chunk in eight
    overflows the window and is emitted in two slices while its source bytes
    still fit the stage: the staged path across slices, after the first
    slice's window was cleared at the chunk's start."""
    rng = random.Random(11)
    keys = sorted({_rand_bytes(rng, 50, 150) for _ in range(4000)})
    recs = [(k, _rand_bytes(rng, 0, 800)) for k in keys]
    A = _records_side(recs[::2])
    B = _records_side([(k, None if i % 5 == 0 else v) for i, (k, v) in enumerate(recs[1::2])])
    check_path(A, B, items=2048, path="fused", label="staged chunks over several slices")


def test_records_longer_than_the_window():
    """One record in ten carries a value of 20-60 KB (up to half a megabit,
    several of the emitter's 80-kilobit windows) between short records: such
    a record is emitted over several slices, and its workgroup's sources do
    not fit the stage and are read in place."""
    rng = random.Random(21)
    keys = sorted({_rand_bytes(rng, 1, 40) for _ in range(300)})
    recs = [(k, _rand_bytes(rng, 20000, 60000) if i % 10 == 0 else _rand_bytes(rng, 0, 50))
            for i, k in enumerate(keys)]
    A = _records_side(recs[::2])
    B = _records_side([(k, None if i % 7 == 0 else v) for i, (k, v) in enumerate(recs[1::2])])
    for path in ("fused", "merge"):
        check_path(A, B, items=64, path=path, label=f"{path}, records longer than the window")


def test_equal_pairs_split_by_partition_boundaries():
    rng = random.Random(5)
    keys = sorted({_rand_bytes(rng, 2, 6) for _ in range(3000)})
    A, B = _split(keys, rng, p_both=0.8, p_tomb=0.1, vmax=6)
    for items in (2, 3, 4, 5, 17, 256, 511):
        check_path(A, B, items=items, label=f"dense collisions items={items}")
    for items in (2, 5, 17, 256):
        check_path(A, B, items=items, path="fused", coarse_parts=3, label=f"fused dense items={items}")


@pytest.mark.parametrize("n", [1, 2, 14, 15, 16, 29, 30, 31, 46])
def test_w15_phase_counts(n):
    keys = [b"key/%05d/" % i + b"x" * (i % 7) for i in range(n)]
    rng = random.Random(n)
    A = _records_side([(k, _rand_bytes(rng, 0, 5)) for k in keys[::2]])
    B = _records_side([(k, None if i % 3 == 0 else b"v") for i, k in enumerate(keys[1::2])])
    check_path(A, B, items=4)
    check_path(A, B, items=4, path="fused", coarse_parts=2)


@pytest.mark.parametrize("wid,scale", [(2, 0.02), (3, 0.002), (4, 0.001), (5, 0.005)])
def test_scaled_workloads(wid, scale):
    A, B = workload(wid, scale)
    print(f"workload {wid} at {scale}: {A.n}+{B.n}", flush=True)
    for path in ("merge", "collision", "fused"):
        check_path(A, B, items=None if path == "fused" else 2048, path=path,
                   label=f"w{wid}@{scale}/{path}")


def test_scan_random_lengths_many_tiles():
    import torch
    import merge_front_coded_amd as em
    rng = np.random.default_rng(6)
    for n in (0, 1, 4095, 4096, 4097, 100_000, 1_234_567):
        lens = rng.integers(0, 1 << 31, size=n, dtype=np.uint64).astype(np.uint32)
        dev = torch.from_numpy(np.concatenate([lens, np.zeros(4, np.uint32)]).view(np.int32)).cuda()
        off = torch.empty(n + 1, dtype=torch.int64, device="cuda")
        ws = torch.empty(em.em_workspace_bytes(n, 0, 4096), dtype=torch.uint8, device="cuda")
        em.em_scan(dev, n, off, ws)
        want = np.zeros(n + 1, np.uint64)
        np.cumsum(lens.astype(np.uint64), out=want[1:])
        got = off.cpu().numpy().view(np.uint64)
        assert np.array_equal(got, want), f"scan n={n}"


@pytest.mark.parametrize("layout", ["512", "2048"])
def test_rank_probe_boundaries(layout):
    """GPU rank queries of both temporary layouts against the oracle's prefix
    counts, at every position of small maps and at block and run edges of
    large ones, on all-zero, all-one, sparse and random maps."""
    import torch
    import merge_front_coded_amd as em
    probe = em.em_rank512_probe if layout == "512" else em.em_rank2048_probe
    ws_bytes = em.em_rank512_workspace_bytes if layout == "512" else em.em_rank2048_workspace_bytes
    rng = np.random.default_rng(7)
    for nbits in (0, 1, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1023, 1024, 1025, 1535, 1536, 1537, 2047, 2048,
                  2049, 4095, 4096, 4097, 100_003):
        for fill in ("zero", "one", "sparse", "random"):
            bits = {"zero": np.zeros(nbits, np.uint8), "one": np.ones(nbits, np.uint8),
                    "sparse": (rng.random(nbits) < 0.01).astype(np.uint8),
                    "random": (rng.random(nbits) < 0.5).astype(np.uint8)}[fill]
            words = np.zeros((nbits + 31) // 32 + 1, np.uint32)
            idx = np.nonzero(bits)[0]
            np.bitwise_or.at(words, idx >> 5, (np.uint32(1) << (idx & 31).astype(np.uint32)))
            # garbage past nbits must be ignored
            if nbits % 32:
                words[nbits >> 5] |= np.uint32(0xFFFFFFFF) << np.uint32(nbits % 32)
            if nbits <= 4096:
                pos = np.arange(nbits + 1, dtype=np.uint32)
            else:
                edges = np.arange(0, nbits + 1, 512, dtype=np.int64)
                pos = np.concatenate([rng.integers(0, nbits + 1, 5000), [0, 31, 32, 33, 63, 64, 65, nbits],
                                      edges, edges - 1, edges + 1])
                pos = np.unique(pos[(pos >= 0) & (pos <= nbits)]).astype(np.uint32)
            want = oracle.rank(_masked(words, nbits), pos)
            dev_words = torch.from_numpy(words.view(np.int32)).cuda()
            dev_pos = torch.from_numpy(pos.view(np.int32)).cuda()
            out = torch.empty(max(pos.size, 1), dtype=torch.int32, device="cuda")
            ws = torch.empty(ws_bytes(nbits), dtype=torch.uint8, device="cuda")
            probe(dev_words, nbits, dev_pos, out, ws)
            got = out.cpu().numpy().view(np.uint32)[:pos.size]
            assert np.array_equal(got, want), f"rank{layout} nbits={nbits} fill={fill}"


def _masked(words, nbits):
    w = words.copy()
    if nbits % 32:
        w[nbits >> 5] &= np.uint32((1 << (nbits % 32)) - 1)
    w[(nbits + 31) >> 5:] = 0
    return w


def test_argument_errors_are_reported():
    import torch
    import merge_front_coded_amd as em
    A, B = workload(1, 0.05)
    dA, dB = em.DeviceSide.from_host(A), em.DeviceSide.from_host(B)
    pl = em.Pipeline(dA, dB, items_per_part=256)
    with pytest.raises(em.EmError) as e:
        em.em_partition(dA, dB, 0, pl.splits, pl.ws)
    assert e.value.code == -1
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(em.EmError) as e:
        em.em_merge_keep(dA, dB, pl.splits, 1, pl.final, pl.ord_A, pl.ord_B, pl.d_S, small)
    assert e.value.code == -3
    pl.run()
    tiny = torch.empty(1, dtype=torch.int32, device="cuda")
    with pytest.raises(em.EmError) as e:
        em.em_emit(dA, dB, pl.final, pl.lcp, pl.S, pl.off, pl.T, tiny, pl.ws)
    assert e.value.code == -3


def test_repeated_runs_are_identical():
    A, B = workload(1, 0.3)
    ref = oracle.run(A, B, items_per_part=512)
    pl = run_gpu(A, B, items=512)
    for _ in range(3):
        pl.payload.fill_(-1)
        pl.final.fill_(-1)
        pl.run()
        compare(pl, ref, A, B, label="rerun")


def test_fused_emitter_reruns_with_chunk_tickets():
    """More chunks than resident emitter workgroups, so that most chunks are
    handed out by the ticket counters; emitting again from the same workspace
    (the counters were left at zero) gives the same payload."""
    import merge_front_coded_amd as em

    A, B = workload(3, 0.03)
    print(f"fused emitter reruns base64 {A.n}+{B.n}", flush=True)
    pl, ref = check_path(A, B, items=2048, path="fused")
    for i in range(2):
        pl.payload.fill_(-1)
        em.em_emit_merged(pl.A, pl.B, pl.items, pl.payload, pl.d_S, pl.d_T, pl.ws,
                          final_refs=pl.final, lcp_bits=pl.lcp)
        torch.cuda.synchronize()
        assert pl.payload_bytes() == ref["payload"].tobytes(), f"emit rerun {i}"
