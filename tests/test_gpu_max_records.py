"""The record cap: |A| + |B| = 2^24 - 1 input records, the most the C ABI
accepts.  Three-byte big-endian keys (A: the even numbers below 2^24; B: the
numbers that are 0 or 1 mod 4, less the last, so that a quarter of all keys is
in both sides), values of 0..4 bytes, tombstones on B.  Every output of the
fused path (with its per-record arrays kept), of its single-pass variant, of
the six-call path and of the collision path is compared element by element
with the CPU oracle."""
import numpy as np
import pytest

import gen
import oracle
import torch  # imported at collection so that its first-load time is not charged to a test
from gpu_util import compare, require_gpu, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _side(xs, vlen_mod, tomb):
    n = xs.size
    keys = np.stack([(xs >> 16) & 255, (xs >> 8) & 255, xs & 255], axis=1).astype(np.uint8).reshape(-1)
    key_off = (3 * np.arange(n + 1, dtype=np.int64)).astype(np.uint32)
    vlen = np.where(tomb, 0, xs % vlen_mod).astype(np.int64)
    val_off = np.zeros(n + 1, np.int64)
    np.cumsum(vlen, out=val_off[1:])
    vals = np.repeat((xs & 255).astype(np.uint8), vlen)
    return gen.HostSide(keys, key_off, vals, val_off.astype(np.uint32), tomb.astype(np.uint8))


def test_record_cap():
    x = np.arange(1 << 24, dtype=np.int64)
    a = x[x % 2 == 0]
    b = x[(x % 4 == 0) | (x % 4 == 1)][:-1]
    assert a.size + b.size == (1 << 24) - 1
    Ah = _side(a, 3, np.zeros(a.size, bool))
    Bh = _side(b, 5, b % 7 == 0)
    print("oracle on 2^24 - 1 records", flush=True)
    ref = oracle.run(Ah, Bh, items_per_part=2048)
    assert ref["S"] == a.size + b.size - (1 << 22)
    for path, kw in (("fused", {"items": None}), ("fused", {"items": None, "one_pass": True}),
                     ("merge", {"items": 2048}), ("collision", {"items": 2048})):
        print(f"  path {path} {kw}", flush=True)
        pl = run_gpu(Ah, Bh, path=path, **kw)
        compare(pl, ref, Ah, Bh, label=f"record cap, {path}")
        del pl
        torch.cuda.empty_cache()
