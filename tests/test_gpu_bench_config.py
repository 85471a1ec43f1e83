"""Parity of exactly what bench.py times: the fused paths built by
bench.make_pipeline, which keep no per-record arrays (final references,
ordinals, lengths, LCPs and offsets are not written; the emitter reads its
inputs from the workspace).  S, T and every payload byte are compared with
the CPU oracle on scaled workloads, and S, T and the payload's SHA-256 with
the oracle's digests on the full-size headline workload (8M+8M base64 keys),
in the partition size the benchmark uses."""
import hashlib
import json
import os

import numpy as np
import pytest

import bench
import gen
import oracle
import torch  # imported at collection so that its first-load time is not charged to a test
from gpu_util import require_gpu, workload

pytestmark = pytest.mark.gpu

DIGESTS = os.path.join(os.path.dirname(__file__), "golden", "full_size_digests.json")
PATHS = ("fused", "onecall", "onepass")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bench_run(Ah, Bh, path, items=None):
    import merge_front_coded_amd as em
    A = em.DeviceSide.from_host(Ah)
    B = em.DeviceSide.from_host(Bh)
    pl = bench.make_pipeline(A, B, path, items)
    assert not pl.keep_all, "the benchmark's fused configuration keeps no per-record arrays"
    pl.run()
    pl.run()  # a second pass over the same buffers, as the timed steps do
    torch.cuda.synchronize()
    return pl


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("wid,scale", [(1, 1.0), (2, 1 / 32), (3, 1 / 128), (4, 1 / 128), (5, 1 / 64)])
def test_bench_configuration_matches_oracle(path, wid, scale):
    Ah, Bh = workload(wid, scale)
    print(f"workload {wid} @{scale:g} ({Ah.n}+{Bh.n}), path {path}", flush=True)
    ref = oracle.run(Ah, Bh, items_per_part=256)
    pl = _bench_run(Ah, Bh, path)
    assert (pl.S, pl.T) == (ref["S"], ref["T"])
    got = np.frombuffer(pl.payload_bytes(), np.uint8)
    bad = np.nonzero(got != ref["payload"])[0]
    assert got.size == ref["payload"].size and bad.size == 0, f"payload differs first at byte {bad[:1]}"


@pytest.mark.parametrize("path", PATHS)
def test_bench_configuration_full_size_headline(path):
    with open(DIGESTS) as f:
        ref = json.load(f)["3"]
    print(f"full-size headline workload, path {path}", flush=True)
    Ah, Bh = workload(3)
    pl = _bench_run(Ah, Bh, path)
    assert (pl.S, pl.T) == (ref["S"], ref["T"])
    assert hashlib.sha256(pl.payload_bytes()).hexdigest() == ref["payload"]
    # the benchmark's own check names the same digest
    assert bench.reference_digest(3) == (ref["S"], ref["T"], ref["payload"])
    del pl
    torch.cuda.empty_cache()
