"""GPU parity of the byte-profile encoding (em_bp_lengths, em_scan,
em_bp_emit, em_bp_navigation) against the CPU oracle, byte for byte: the
framing width, record lengths, offsets, payload and navigation sections, on
every generated workload (two of which have fixed 17-byte framing), through
the six-call and fused paths, and on edge cases: LEB128 counts of two and
three bytes, all tombstones (width 1), stored empty values, block edges and
the empty merge."""
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


def _check(Ah, Bh, label, path="merge", want_width=None):
    import merge_front_coded_amd as em
    pl = run_gpu(Ah, Bh, items=None if path == "fused" else 256, path=path)
    W, T = pl.byte_profile()
    torch.cuda.synchronize()
    S = pl.S
    ref = oracle.run(Ah, Bh, items_per_part=256)
    bp = oracle.bp_encode(Ah, Bh, ref["final"])
    print(f"{label}: S={S} width={W} T={T} bytes", flush=True)
    assert (S, W, T) == (ref["S"], bp["width"], bp["T"]), label
    if want_width is not None:
        assert W == want_width, label
    assert int(pl.bp_over.item()) == 0, label
    assert np.array_equal(pl.bp_len[:S].cpu().numpy().view(np.uint32), bp["len_bytes"]), label
    assert np.array_equal(pl.bp_off[:S + 1].cpu().numpy().view(np.uint64), bp["off"]), label
    got = pl.bp_payload[:T].cpu().numpy()
    bad = np.nonzero(got != bp["payload"])[0]
    assert bad.size == 0, f"{label}: payload differs first at byte {bad[:3]}"
    # navigation over the byte offsets
    sec = em.EfSections(em.em_ef_entry_count(S))
    em.em_bp_navigation(pl.bp_off, S, T, pl.bp_width, sec)
    nav = sec.host()
    want = oracle.ef_encode(oracle.ef_entries(bp["off"], S, T, W), W)
    for k in ("n", "L", "width", "high_bits", "groups", "n_exceptions"):
        assert nav[k] == want[k], f"{label}: navigation {k}"
    for k in ("lows", "highs", "samples", "exceptions"):
        assert np.array_equal(nav[k], np.asarray(want[k], np.uint64)), f"{label}: navigation {k}"


@pytest.mark.parametrize("wid,scale", [(1, 0.5), (2, 0.005), (3, 0.001), (4, 0.001), (5, 0.002)])
def test_byte_profile_generated(wid, scale):
    A, B = workload(wid, scale)
    _check(A, B, f"workload {wid} at {scale}", want_width=17 if wid in (2, 4) else None)
    _check(A, B, f"workload {wid} at {scale}, fused", path="fused")


def test_byte_profile_edges():
    rng = np.random.default_rng(8)
    # two- and three-byte LEB128: keys of 100..20000 bytes sharing long prefixes,
    # values of 0..300 bytes
    keys = sorted({b"P" * int(rng.integers(100, 20000)) + bytes([int(rng.integers(0, 256))]) for _ in range(60)})
    A = gen.side_from_records([(k, rng.bytes(int(rng.integers(0, 300)))) for k in keys[::2]])
    B = gen.side_from_records([(k, None if i % 3 == 0 else rng.bytes(int(rng.integers(0, 300))))
                               for i, k in enumerate(keys[1::2])])
    _check(A, B, "long keys and values")
    # all tombstones: width 1 (the tag alone)
    keys = [b"t%05d" % i for i in range(400)]
    A = gen.side_from_records([(k, None) for k in keys[::2]])
    B = gen.side_from_records([(k, None) for k in keys[1::2]])
    _check(A, B, "all tombstones", want_width=1)
    # stored empty values everywhere: width 1 too (L = 0)
    A = gen.side_from_records([(k, b"") for k in keys[::2]])
    B = gen.side_from_records([(k, b"") for k in keys[1::2]])
    _check(A, B, "empty values", want_width=1)
    # block edges
    for n in (1, 15, 16, 31):
        ks = [b"edge/%03d" % i for i in range(n)]
        _check(gen.side_from_records([(k, b"v" * (i % 4)) for i, k in enumerate(ks)]), gen.side_from_records([]),
               f"{n} records")
    empty = gen.side_from_records([])
    _check(empty, empty, "empty")


def test_byte_profile_window_fallback():
    """Workgroups whose bytes overflow the LDS window write to the payload
    directly, beside workgroups that use it."""
    rng = np.random.default_rng(12)
    keys = [b"w%05d/" % i + b"k" * int(rng.integers(0, 30)) for i in range(2000)]
    vals = [rng.bytes(30000) if i % 97 == 0 else (None if i % 7 == 0 else rng.bytes(int(rng.integers(0, 40))))
            for i in range(2000)]
    A = gen.side_from_records(list(zip(keys[::2], vals[::2])))
    B = gen.side_from_records(list(zip(keys[1::2], vals[1::2])))
    _check(A, B, "window fallback")
