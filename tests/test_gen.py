"""The seeded generator: each side strictly increasing (hence unique), the
stated overlap, tombstones only where asked, deterministic per seed."""
import numpy as np
import pytest

import gen


def _keys(side):
    return [side.key(i) for i in range(side.n)]


@pytest.mark.parametrize("wid,scale", [(1, 1.0), (2, 0.01), (3, 0.002), (4, 0.002), (5, 0.005)])
def test_workload_shape(wid, scale):
    w = gen.WORKLOADS[wid].scaled(scale)
    A, B = gen.make(w)
    assert A.n == w.nA and B.n == w.nB
    for s in (A, B):
        ks = _keys(s)
        assert all(ks[i] < ks[i + 1] for i in range(len(ks) - 1))  # strictly increasing
        assert s.key_off[0] == 0 and s.key_off[-1] == s.keys.size
        assert s.val_off[0] == 0 and s.val_off[-1] == s.vals.size
        assert np.all(np.diff(s.key_off.astype(np.int64)) >= 0)
        # tombstones carry no value bytes
        vl = np.diff(s.val_off.astype(np.int64))
        assert np.all(vl[s.tomb != 0] == 0)
    assert int(A.tomb.sum()) == 0
    both = len(set(_keys(A)) & set(_keys(B)))
    assert both == int(round(w.overlap * w.nB))
    if B.n >= 1000:
        assert abs(B.tomb.mean() - w.tombB) < 0.05


def test_deterministic_per_seed():
    w = gen.WORKLOADS[1].scaled(0.1)
    A1, B1 = gen.make(w)
    A2, B2 = gen.make(w)
    A3, _ = gen.make(w, seed=w.seed + 1)
    assert np.array_equal(A1.keys, A2.keys) and np.array_equal(B1.vals, B2.vals)
    assert not np.array_equal(A1.keys[:64], A3.keys[:64])


def test_key_shapes():
    A, _ = gen.make(gen.WORKLOADS[5].scaled(0.001))
    for k in _keys(A):
        assert 64 <= len(k) <= 256 and k.startswith(b"https://") and k[-12:].isdigit()
    A, _ = gen.make(gen.WORKLOADS[4].scaled(0.0005))
    assert all(len(k) == 16 for k in _keys(A))
    A, _ = gen.make(gen.WORKLOADS[2].scaled(0.002))
    assert all(2 <= k.count(b"/") + 1 <= 6 for k in _keys(A))
