"""GPU parity of the front-coded input path (em_fcin_parse +
em_fcin_materialize): payloads written by the GPU path are decoded back into
arenas and compared byte for byte with the CPU oracle's decoder, with block
starts taken from the record offsets and from the navigation sections; a
decoded side is merged again and compared with the oracle; block edges,
sub-byte prefixes, long inherited chains, fixed-width values, the empty
payload and malformed lengths are covered.  The prefix cache filled from the
literal owners (em_fcin_prefix8) is compared with the first eight bytes of
the oracle's decoded keys."""
import numpy as np
import pytest

import gen
import oracle
import torch  # imported at collection so that its first-load time is not charged to a test
from gpu_util import check_path, require_gpu, run_gpu, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _host_side(d):
    """A DeviceSide read back (arenas cut to their lengths)."""
    n = d.n
    key_off = d.key_off[:n + 1].cpu().numpy().view(np.uint32).copy()
    val_off = d.val_off[:n + 1].cpu().numpy().view(np.uint32).copy()
    return gen.HostSide(keys=d.keys[:d.key_bytes].cpu().numpy().copy(), key_off=key_off,
                        vals=d.vals[:d.val_bytes].cpu().numpy().copy(), val_off=val_off,
                        tomb=d.tomb[:n].cpu().numpy().copy())


def _same_side(got, want, label):
    for f in ("keys", "key_off", "vals", "val_off", "tomb"):
        g, w = getattr(got, f), getattr(want, f)
        assert g.size == w.size, f"{label}: {f} size {g.size} != {w.size}"
        bad = np.nonzero(g != w)[0]
        assert bad.size == 0, f"{label}: {f} differs at {bad[:5]}"


def _round_trip(Ah, Bh, label, nav=False):
    import merge_front_coded_amd as em
    pl = run_gpu(Ah, Bh, items=256)
    torch.cuda.synchronize()
    S, T = pl.S, pl.T
    payload_h = np.frombuffer(pl.payload_bytes(), np.uint8)
    want = oracle.fc_decode(payload_h, T, S, int(Ah.keys.size + Bh.keys.size) + 16,
                            int(Ah.vals.size + Bh.vals.size) + 16)
    print(f"{label}: S={S} T={T}", flush=True)
    d = em.fcin_decode(pl.payload, T, S, off=pl.off)
    _same_side(_host_side(d), want, f"{label}/off")
    if nav:
        sec = pl.ef_navigation()
        d2 = em.fcin_decode(pl.payload, T, S, nav=sec)
        _same_side(_host_side(d2), want, f"{label}/navigation")
    return d, want


@pytest.mark.parametrize("wid,scale", [(1, 0.3), (2, 0.005), (3, 0.001), (4, 0.001), (5, 0.002)])
def test_decode_generated_payloads(wid, scale):
    A, B = workload(wid, scale)
    _round_trip(A, B, f"workload {wid} at {scale}", nav=True)


def test_decode_edges():
    rng = np.random.default_rng(5)
    empty = gen.side_from_records([])
    for n in (1, 14, 15, 16, 29, 30, 31, 46):
        keys = [b"blk/%04d/" % i + b"z" * (i % 5) for i in range(n)]
        A = gen.side_from_records([(k, rng.bytes(int(rng.integers(0, 5)))) for k in keys[::2]])
        B = gen.side_from_records([(k, None if i % 3 == 0 else b"v") for i, k in enumerate(keys[1::2])])
        _round_trip(A, B, f"{n} records", nav=True)
    # sub-byte prefixes: keys over bytes that differ in single bits
    import itertools
    alpha = [0x00, 0x01, 0x02, 0x40, 0x80, 0x81, 0xFE, 0xFF]
    keys = sorted({bytes(t) for L in (1, 2, 3) for t in itertools.product(alpha, repeat=L)} | {b""})
    A = gen.side_from_records([(k, b"a") for k in keys[::3]])
    B = gen.side_from_records([(k, None if i % 4 == 0 else b"") for i, k in enumerate(keys[1::2])])
    _round_trip(A, B, "sub-byte prefixes", nav=True)
    # long inherited chains: each key extends a long shared prefix by one byte
    keys = sorted({b"p" * int(rng.integers(1, 300)) + bytes([int(rng.integers(0, 256))]) for _ in range(700)})
    A = gen.side_from_records([(k, rng.bytes(3)) for k in keys[::2]])
    B = gen.side_from_records([(k, rng.bytes(1)) for k in keys[1::2]])
    _round_trip(A, B, "long chains", nav=True)
    # every value 16 bytes: the navigation subtracts a common width
    keys = [b"fixed%06d" % i for i in range(3000)]
    A = gen.side_from_records([(k, rng.bytes(16)) for k in keys[::2]])
    B = gen.side_from_records([(k, rng.bytes(16)) for k in keys[1::2]])
    _round_trip(A, B, "fixed width", nav=True)
    # empty payload
    _round_trip(empty, empty, "empty")


def test_decode_window_fallback():
    """Workgroups whose key and value bytes overflow the LDS window write to
    the arenas directly, beside workgroups that use it; oversized arena
    capacities change the records per workgroup, not the arenas."""
    import merge_front_coded_amd as em
    rng = np.random.default_rng(11)
    keys = [b"w%05d/" % i + b"k" * int(rng.integers(0, 30)) for i in range(2000)]
    vals = [rng.bytes(30000) if i % 97 == 0 else (None if i % 7 == 0 else rng.bytes(int(rng.integers(0, 40))))
            for i in range(2000)]
    A = gen.side_from_records(list(zip(keys[::2], vals[::2])))
    B = gen.side_from_records(list(zip(keys[1::2], vals[1::2])))
    d, want = _round_trip(A, B, "window fallback", nav=True)
    pl = run_gpu(A, B, items=256)
    S, T = pl.S, pl.T
    for scale in (1, 40):
        ws = torch.empty(max(em.em_fcin_workspace_bytes(S), 256), dtype=torch.uint8, device="cuda")
        tot = torch.zeros(3, dtype=torch.int64, device="cuda")
        em.em_fcin_parse(pl.payload, T, S, tot, ws, off=pl.off)
        kb, vb, err = (int(x) for x in tot.cpu())
        assert err == 0 and (kb, vb) == (want.keys.size, want.vals.size)
        keys_d = torch.zeros(kb * scale + 64, dtype=torch.uint8, device="cuda")
        vals_d = torch.zeros(vb * scale + 64, dtype=torch.uint8, device="cuda")
        ko = torch.empty(S + 1, dtype=torch.int32, device="cuda")
        vo = torch.empty(S + 1, dtype=torch.int32, device="cuda")
        tb = torch.empty(S, dtype=torch.uint8, device="cuda")
        em.em_fcin_materialize(pl.payload, S, keys_d, ko, vals_d, vo, tb, tot, ws)
        torch.cuda.synchronize()
        assert int(tot[2].item()) == 0
        got = gen.HostSide(keys=keys_d[:kb].cpu().numpy(), key_off=ko.cpu().numpy().view(np.uint32),
                           vals=vals_d[:vb].cpu().numpy(), val_off=vo.cpu().numpy().view(np.uint32),
                           tomb=tb.cpu().numpy())
        _same_side(got, want, f"arena capacity x{scale}")


def test_decoded_side_merges_again():
    """A side decoded from a payload enters the merge like any other."""
    import merge_front_coded_amd as em
    A, B = workload(1, 0.2)
    d, want = _round_trip(A, B, "merge again")
    C, _ = workload(1, 0.1)
    ref = oracle.run(want, C, items_per_part=256)
    pl = em.Pipeline(d, em.DeviceSide.from_host(C), items_per_part=256)
    pl.run()
    torch.cuda.synchronize()
    assert (pl.S, pl.T) == (ref["S"], ref["T"])
    assert np.array_equal(pl.host("final", pl.S), ref["final"])
    assert pl.payload_bytes() == ref["payload"].tobytes()


def test_malformed_lengths_are_reported():
    import merge_front_coded_amd as em
    A, B = workload(1, 0.05)
    pl = run_gpu(A, B, items=256)
    torch.cuda.synchronize()
    S, T = pl.S, pl.T
    for bad_T in (T - 1, T + 1):
        with pytest.raises(em.EmError):
            em.fcin_decode(pl.payload, bad_T, S, off=pl.off)
    with pytest.raises(em.EmError):  # one record fewer: the last block ends early
        em.fcin_decode(pl.payload, T, S - 1, off=pl.off)


def _first8(side):
    """The first 8 bytes of every key as big-endian u64s, zero past the key's end."""
    off = side.key_off.astype(np.int64)
    lens = off[1:] - off[:-1]
    keys = np.concatenate([side.keys, np.zeros(8, np.uint8)])
    out = np.zeros(lens.size, np.uint64)
    for b in range(8):
        byte = np.where(lens > b, keys[np.minimum(off[:-1] + b, keys.size - 1)], 0).astype(np.uint64)
        out |= byte << np.uint64(56 - 8 * b)
    return out


def _prefix_cache_case(Ah, Bh, label):
    import merge_front_coded_amd as em
    pl = run_gpu(Ah, Bh, items=256)
    torch.cuda.synchronize()
    S, T = pl.S, pl.T
    payload_h = np.frombuffer(pl.payload_bytes(), np.uint8)
    want = oracle.fc_decode(payload_h, T, S, int(Ah.keys.size + Bh.keys.size) + 16,
                            int(Ah.vals.size + Bh.vals.size) + 16)
    print(f"{label}: S={S} T={T}", flush=True)
    ws = torch.empty(max(em.em_fcin_workspace_bytes(S), 256), dtype=torch.uint8, device="cuda")
    tot = torch.zeros(3, dtype=torch.int64, device="cuda")
    em.em_fcin_parse(pl.payload, T, S, tot, ws, off=pl.off)
    assert int(tot[2].item()) == 0
    pfx = torch.full((max(S, 1),), -1, dtype=torch.int64, device="cuda")
    em.em_fcin_prefix8(pl.payload, S, pfx, ws)
    torch.cuda.synchronize()
    got = pfx[:S].cpu().numpy().view(np.uint64)
    exp = _first8(want)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, f"{label}: prefix differs at {bad[:5]}: {[hex(int(got[i])) for i in bad[:3]]} " \
                          f"vs {[hex(int(exp[i])) for i in bad[:3]]}"


@pytest.mark.parametrize("wid,scale", [(1, 0.3), (2, 0.005), (3, 0.0025), (4, 0.001), (5, 0.002)])
def test_prefix_cache_from_owners(wid, scale):
    """Several 4096-record tiles and a ragged last one (workload 3 at this
    scale: about 30k survivors); URL keys inherit far more than 8 bytes."""
    A, B = workload(wid, scale)
    _prefix_cache_case(A, B, f"workload {wid} at {scale}")


def test_prefix_cache_edges():
    """Keys shorter than 8 bytes and empty, prefixes that end inside a byte,
    inherited runs longer than 8 bytes that end at and around byte 8, and one
    record."""
    rng = np.random.default_rng(23)
    recs = [(b"", b"e")]
    for i in range(3000):
        k = bytes(rng.integers(0, 4, int(rng.integers(0, 7)), dtype=np.uint8))
        recs.append((bytes([1 + i // 300]) + k, None if i % 5 == 0 else b"v"))
    for i in range(1500):
        recs.append((b"\x7f" * int(7 + i % 4) + bytes([i % 3, (i // 3) % 251]) + b"tail" * (i % 2), b"w"))
    recs = sorted(set(recs), key=lambda kv: kv[0])
    uniq = {}
    for k, v in recs:
        uniq[k] = v
    items = sorted(uniq.items())
    A = gen.side_from_records(items[::2])
    B = gen.side_from_records(items[1::2])
    _prefix_cache_case(A, B, "edges")
    _prefix_cache_case(gen.side_from_records([(b"only", b"x")]), gen.side_from_records([]), "one record")


@pytest.mark.parametrize("n", [4095, 4096, 4097, 8192, 12289])
def test_prefix_cache_tile_boundaries(n):
    """Record counts at and around whole tiles of the prefix scan (4096
    records), one side empty: every record survives, so S = n."""
    rng = np.random.default_rng(n)
    keys = sorted({bytes(rng.integers(65, 70, int(rng.integers(1, 14)), dtype=np.uint8)) for _ in range(3 * n)})[:n]
    assert len(keys) == n
    A = gen.side_from_records([(k, b"v" * (i % 3)) for i, k in enumerate(keys)])
    _prefix_cache_case(A, gen.side_from_records([]), f"{n} records")


def test_prefix_cache_after_navigation_parse():
    """Block starts from the navigation sections instead of the record
    offsets: the same prefixes."""
    import merge_front_coded_amd as em
    A, B = workload(2, 0.004)
    pl = run_gpu(A, B, items=256)
    torch.cuda.synchronize()
    S, T = pl.S, pl.T
    sec = pl.ef_navigation()
    out = []
    for kw in ({"off": pl.off}, {"nav": sec}):
        ws = torch.empty(max(em.em_fcin_workspace_bytes(S), 256), dtype=torch.uint8, device="cuda")
        tot = torch.zeros(3, dtype=torch.int64, device="cuda")
        em.em_fcin_parse(pl.payload, T, S, tot, ws, **kw)
        assert int(tot[2].item()) == 0
        pfx = torch.empty(S, dtype=torch.int64, device="cuda")
        em.em_fcin_prefix8(pl.payload, S, pfx, ws)
        torch.cuda.synchronize()
        out.append(pfx.cpu().numpy().view(np.uint64))
    assert np.array_equal(out[0], out[1])
    payload_h = np.frombuffer(pl.payload_bytes(), np.uint8)
    want = oracle.fc_decode(payload_h, T, S, int(A.keys.size + B.keys.size) + 16, int(A.vals.size + B.vals.size) + 16)
    assert np.array_equal(out[0], _first8(want))
