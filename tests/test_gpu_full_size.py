"""Full-size parity: every output of the HIP path (and the output navigation
sections built from it) on the five full-size
workloads, in the benchmark's launch configuration (the partition size the
pipeline chooses from the mean key length), against SHA-256 digests of the CPU oracle's outputs written by
tests/golden/make_full_size_digests.py (which calls only gen/ and oracle/).

A digest covers every element, so this is an element-by-element comparison
without rerunning the bit-at-a-time oracle on the GPU host.  The input digest
guards against the generator drifting from the inputs the digests were made
from."""
import hashlib
import json
import os

import numpy as np
import pytest

import gen
import torch  # imported at collection so that its first-load time is not charged to a test
from gpu_util import require_gpu, run_gpu

pytestmark = pytest.mark.gpu

DIGESTS = os.path.join(os.path.dirname(__file__), "golden", "full_size_digests.json")


def _sha(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_full_size_workload_matches_oracle(wid):
    with open(DIGESTS) as f:
        ref = json.load(f)[str(wid)]
    print(f"full-size workload {wid} ({ref['workload']})", flush=True)
    A, B = gen.make(wid)
    assert _sha(A.keys, A.key_off, A.vals, A.val_off, A.tomb, B.keys, B.key_off, B.vals, B.val_off,
                B.tomb) == ref["input"], "generator output drifted from the digested inputs"
    runs = [("fused", {}), ("merge", {})] + [("collision", {"collision_mode": m})
                                             for m in ("512-tiled", "512", "2048", "512-compact")]
    for path, kw in runs:
        print(f"  path {path} {kw}", flush=True)
        pl = run_gpu(A, B, items=None, path=path, **kw)
        torch.cuda.synchronize()
        S = pl.S
        assert S == ref["S"], f"{path}: S {S} != {ref['S']}"
        assert pl.T == ref["T"], f"{path}: T {pl.T} != {ref['T']}"
        got = {
            "final": _sha(pl.host("final", S)),
            "ord_A": _sha(pl.host("ord_A", A.n)),
            "ord_B": _sha(pl.host("ord_B", B.n)),
            "len_bits": _sha(pl.host("len_bits", S)),
            "lcp_bits": _sha(pl.host("lcp", S)),
            "off": _sha(pl.host("off", S + 1)),
            "payload": _sha(np.frombuffer(pl.payload_bytes(), np.uint8)),
        }
        nav = pl.ef_navigation().host()
        head = np.array([nav[k] for k in ("n", "L", "width", "low_words", "high_bits", "high_words", "groups",
                                          "n_exceptions")], np.uint64)
        got["ef"] = _sha(head, nav["lows"], nav["highs"], nav["samples"], nav["exceptions"])
        want = dict(ref)
        if path == "merge":
            got["splits"] = _sha(pl.host("splits"))
            want["splits"] = ref["splits"][str(pl.items)]
        bad = [k for k, v in got.items() if v != want[k]]
        assert not bad, f"{path}: outputs differing from the oracle: {bad}"
        del pl
        torch.cuda.empty_cache()
