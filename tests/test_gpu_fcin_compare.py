"""GPU parity of the owner-search key comparison of two front-coded inputs
(em_fcin_compare): each input is front-coded alone by the CPU oracle and
parsed on the GPU; the bit LCP and the order of every pair are compared with
the oracle's on the original keys.  Pairs: equal keys (the comparisons a
merge must finish past its cache), merge neighbours, random pairs; a start
byte past bytes the pair shares; sub-byte differences, long inherited
chains, keys longer than one 256-bit window, empty keys, and indices past
an input; a start byte past differing bytes (checked against the oracle
on keys whose first bytes are zeroed)."""
import numpy as np
import pytest

import gen
import oracle
import torch  # imported at collection so that its first-load time is not charged to a test
from gpu_util import require_gpu, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _compressed(X):
    """X front-coded alone by the oracle (every record survives), parsed on the GPU."""
    import merge_front_coded_amd as em
    o = oracle.run(X, gen.side_from_records([]))
    S, T = o["S"], o["T"]
    assert S == X.n
    payload = torch.from_numpy(o["payload"].view(np.int32).copy()).cuda()
    off = torch.from_numpy(o["off"].view(np.int64).copy()).cuda()
    ws = torch.empty(max(em.em_fcin_workspace_bytes(S), 256), dtype=torch.uint8, device="cuda")
    tot = torch.zeros(3, dtype=torch.int64, device="cuda")
    em.em_fcin_parse(payload, T, S, tot, ws, off=off)
    assert int(tot[2].item()) == 0
    return payload, S, ws


def _keys(X):
    off = X.key_off.astype(np.int64)
    return [X.keys[off[i]:off[i + 1]].tobytes() for i in range(X.n)]


def _pairs(X, Y, rng, n_random=3000):
    """Equal keys, each Y key against its merge neighbours in X, random pairs."""
    kx, ky = _keys(X), _keys(Y)
    where = {k: i for i, k in enumerate(kx)}
    ia, jb = [], []
    for j, k in enumerate(ky):
        if k in where:
            ia.append(where[k])
            jb.append(j)
    pos = np.searchsorted(np.array(kx, dtype=object), np.array(ky, dtype=object)) if kx and ky else []
    for j, p in enumerate(pos):
        for i in (p - 1, p, p + 1):
            if 0 <= i < len(kx):
                ia.append(int(i))
                jb.append(j)
    if kx and ky:
        ia += rng.integers(0, len(kx), n_random).tolist()
        jb += rng.integers(0, len(ky), n_random).tolist()
    return np.array(ia, np.uint32), np.array(jb, np.uint32)


def _run(cx, cy, ia, jb, from_byte=0, with_cmp=True):
    import merge_front_coded_amd as em
    n = int(ia.size)
    ia_t = torch.from_numpy(ia.view(np.int32).copy()).cuda()
    jb_t = torch.from_numpy(jb.view(np.int32).copy()).cuda()
    lcp = torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    cmp = torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda") if with_cmp else None
    em.em_fcin_compare(cx[0], cx[1], cx[2], cy[0], cy[1], cy[2], n, ia_t, jb_t, from_byte, lcp_bits=lcp, cmp=cmp)
    torch.cuda.synchronize()
    got_l = lcp[:n].cpu().numpy().view(np.uint32)
    got_c = cmp[:n].cpu().numpy() if with_cmp else None
    return got_l, got_c


def _check(X, Y, ia, jb, label, from_byte=0):
    cx, cy = _compressed(X), _compressed(Y)
    got_l, got_c = _run(cx, cy, ia, jb, from_byte)
    want_l = np.array([oracle.key_lcp_bits(X, int(i), Y, int(j)) for i, j in zip(ia, jb)], np.uint32)
    want_c = np.array([np.sign(oracle.key_cmp(X, int(i), Y, int(j))) for i, j in zip(ia, jb)], np.int32)
    bad = np.nonzero((got_l != want_l) | (got_c != want_c))[0]
    assert bad.size == 0, f"{label}: pair {bad[:3]} (A {ia[bad[:3]]}, B {jb[bad[:3]]}): lcp {got_l[bad[:3]]} vs " \
                          f"{want_l[bad[:3]]}, cmp {got_c[bad[:3]]} vs {want_c[bad[:3]]}"
    return cx, cy


@pytest.mark.parametrize("wid,scale", [(2, 0.004), (3, 0.0005), (5, 0.001)])
def test_compare_generated(wid, scale):
    """Generated inputs: path keys with long shared prefixes (deep owner
    chains), random base64 keys, URLs of up to 256 bytes (several windows)."""
    A, B = workload(wid, scale)
    rng = np.random.default_rng(wid)
    ia, jb = _pairs(A, B, rng)
    print(f"workload {wid} at {scale}: |A|={A.n} |B|={B.n} pairs={ia.size}", flush=True)
    _check(A, B, ia, jb, f"workload {wid}")


def test_compare_from_byte():
    """A start byte inside the bytes a pair shares gives the full result; one
    at or past the shorter key's end gives its length and the length order."""
    A, B = workload(5, 0.001)
    rng = np.random.default_rng(9)
    ia, jb = _pairs(A, B, rng, n_random=500)
    ka, kb = _keys(A), _keys(B)
    cx, cy = _compressed(A), _compressed(B)
    for f in (1, 8, 9, 33):
        keep = np.array([ka[i][:f] == kb[j][:f] and min(len(ka[i]), len(kb[j])) >= f for i, j in zip(ia, jb)])
        si, sj = ia[keep], jb[keep]
        assert si.size > 100
        got_l, got_c = _run(cx, cy, si, sj, from_byte=f)
        want_l = np.array([oracle.key_lcp_bits(A, int(i), B, int(j)) for i, j in zip(si, sj)], np.uint32)
        want_c = np.array([np.sign(oracle.key_cmp(A, int(i), B, int(j))) for i, j in zip(si, sj)], np.int32)
        assert np.array_equal(got_l, want_l) and np.array_equal(got_c, want_c), f"from byte {f}"
    # a start past the shorter key: bit LCP = its length, order by length
    si, sj = ia[:200], jb[:200]
    got_l, got_c = _run(cx, cy, si, sj, from_byte=1 << 20)
    la = np.array([8 * len(ka[i]) for i in si]), np.array([8 * len(kb[j]) for j in sj])
    assert np.array_equal(got_l, np.minimum(*la).astype(np.uint32))
    assert np.array_equal(got_c, np.sign(la[0] - la[1]).astype(np.int32))
    # lcp only
    got_l2, _ = _run(cx, cy, si, sj, from_byte=1 << 20, with_cmp=False)
    assert np.array_equal(got_l2, got_l)


def _zero_head(X, f):
    """X with the first f bytes of every key set to zero (lengths kept)."""
    keys = X.keys.copy()
    off = X.key_off.astype(np.int64)
    for i in range(X.n):
        keys[off[i]:min(off[i] + f, off[i + 1])] = 0
    return gen.HostSide(keys=keys, key_off=X.key_off, vals=X.vals, val_off=X.val_off, tomb=X.tomb)


def test_compare_from_byte_skips_differences():
    """Bytes before the start byte count as shared even where they differ:
    the result is the oracle's on keys whose first bytes are zeroed."""
    A, B = workload(3, 0.0005)
    rng = np.random.default_rng(17)
    ia, jb = _pairs(A, B, rng, n_random=4000)
    cx, cy = _compressed(A), _compressed(B)
    for f in (2, 5):
        Az, Bz = _zero_head(A, f), _zero_head(B, f)
        got_l, got_c = _run(cx, cy, ia, jb, from_byte=f)
        want_l = np.array([oracle.key_lcp_bits(Az, int(i), Bz, int(j)) for i, j in zip(ia, jb)], np.uint32)
        want_c = np.array([np.sign(oracle.key_cmp(Az, int(i), Bz, int(j))) for i, j in zip(ia, jb)], np.int32)
        assert np.array_equal(got_l, want_l) and np.array_equal(got_c, want_c), f"from byte {f}"


def test_compare_edges():
    """Single-bit differences inside a byte, proper prefixes and empty keys;
    chains of inherited bytes up to 300 bytes long (keys spanning ten
    windows); one-record inputs; indices past an input."""
    import itertools
    rng = np.random.default_rng(3)
    alpha = [0x00, 0x01, 0x02, 0x40, 0x80, 0x81, 0xFE, 0xFF]
    keys = sorted({bytes(t) for L in (1, 2, 3) for t in itertools.product(alpha, repeat=L)} | {b""})
    A = gen.side_from_records([(k, b"a") for k in keys[::3]])
    B = gen.side_from_records([(k, None if i % 4 == 0 else b"") for i, k in enumerate(keys[1::2])])
    ia = np.repeat(np.arange(A.n, dtype=np.uint32), B.n)
    jb = np.tile(np.arange(B.n, dtype=np.uint32), A.n)
    sel = rng.choice(ia.size, 20000, replace=False)
    _check(A, B, ia[sel], jb[sel], "sub-byte")
    keys = sorted({b"p" * int(rng.integers(1, 300)) + bytes([int(rng.integers(0, 256))]) for _ in range(700)})
    A = gen.side_from_records([(k, rng.bytes(3)) for k in keys[::2]])
    B = gen.side_from_records([(k, rng.bytes(1)) for k in keys])  # B holds every key: A's keys are equal pairs
    ia, jb = _pairs(A, B, rng, n_random=2000)
    _check(A, B, ia, jb, "long chains")
    one_a = gen.side_from_records([(b"only", b"x")])
    one_b = gen.side_from_records([(b"onlz", None)])
    _check(one_a, one_b, np.array([0], np.uint32), np.array([0], np.uint32), "one record")
    cx, cy = _compressed(A), _compressed(B)
    got_l, got_c = _run(cx, cy, np.array([A.n, 0, 0], np.uint32), np.array([0, B.n, B.n + 5], np.uint32))
    assert np.array_equal(got_l, np.full(3, 0xFFFFFFFF, np.uint32)) and np.array_equal(got_c, np.zeros(3, np.int32))


def _compressed_on_gpu(X):
    """X front-coded alone by the GPU path at full size (its payload's parity
    is covered by the full-size digests), parsed on the GPU."""
    import merge_front_coded_amd as em
    empty = em.DeviceSide.from_host(gen.side_from_records([]))
    pl = em.Pipeline(em.DeviceSide.from_host(X), empty, path="fused", keep_all=True)
    pl.run()
    torch.cuda.synchronize()
    assert pl.S == X.n
    ws = torch.empty(max(em.em_fcin_workspace_bytes(pl.S), 256), dtype=torch.uint8, device="cuda")
    tot = torch.zeros(3, dtype=torch.int64, device="cuda")
    em.em_fcin_parse(pl.payload, pl.T, pl.S, tot, ws, off=pl.off)
    assert int(tot[2].item()) == 0
    return pl.payload, pl.S, ws


def test_compare_full_size_sampled():
    """8M+8M inputs (the benchmark's workload), each front-coded alone:
    20,000 B keys against the A key at or after them (equal keys where B
    replaces A) and 20,000 random pairs, from byte 0 and, for the pairs that
    share their first eight bytes, from byte 8."""
    A, B = workload(3)
    print(f"full size: |A|={A.n} |B|={B.n}", flush=True)
    cx, cy = _compressed_on_gpu(A), _compressed_on_gpu(B)
    rng = np.random.default_rng(33)
    jb = np.sort(rng.choice(B.n, 20000, replace=False)).astype(np.uint32)
    ia = np.empty_like(jb)
    for t, j in enumerate(jb):  # the first A key not below B's (binary search)
        k, lo, hi = B.key(int(j)), 0, A.n
        while lo < hi:
            mid = (lo + hi) // 2
            if A.key(mid) < k:
                lo = mid + 1
            else:
                hi = mid
        ia[t] = min(lo, A.n - 1)
    ia = np.concatenate([ia, rng.integers(0, A.n, 20000).astype(np.uint32)])
    jb = np.concatenate([jb, rng.integers(0, B.n, 20000).astype(np.uint32)])
    want_l = np.array([oracle.key_lcp_bits(A, int(i), B, int(j)) for i, j in zip(ia, jb)], np.uint32)
    want_c = np.array([np.sign(oracle.key_cmp(A, int(i), B, int(j))) for i, j in zip(ia, jb)], np.int32)
    assert (want_c == 0).sum() > 5000  # equal keys are among the pairs
    got_l, got_c = _run(cx, cy, ia, jb)
    assert np.array_equal(got_l, want_l) and np.array_equal(got_c, want_c), "from byte 0"
    keep = want_l >= 64
    got_l, got_c = _run(cx, cy, ia[keep], jb[keep], from_byte=8)
    assert np.array_equal(got_l, want_l[keep]) and np.array_equal(got_c, want_c[keep]), "from byte 8"
