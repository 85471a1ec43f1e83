"""Randomised parity sweep: many small seeded input pairs (sizes from empty to
a few thousand records, keys from empty to long with shared prefixes and
arbitrary bytes, values from empty to a few hundred bytes, tombstones on both
sides, collision rates from none to all) through every path -- six-call,
fused, single pass and the tiled collision mode -- compared element by element
with the CPU oracle, plus the byte-profile encoding and the decode of each
payload back into arenas."""
import numpy as np
import pytest

import gen
import oracle
import torch  # imported at collection so that its first-load time is not charged to a test
from gpu_util import check_path, require_gpu, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _random_pair(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.choice([0, 1, 2, 15, 16, 100, 700, 3000]))
    alphabet = [b"ab", bytes(range(256)), b"\x00\x01\xff"][seed % 3]
    prefix = rng.bytes(int(rng.integers(0, 40))) if seed % 2 else b""
    keys = set()
    while len(keys) < n:
        ln = int(rng.integers(0, 24))
        keys.add(prefix + bytes(alphabet[int(x)] for x in rng.integers(0, len(alphabet), ln)))
    keys = sorted(keys)
    overlap = float(rng.choice([0.0, 0.3, 1.0]))
    tomb_p = float(rng.choice([0.0, 0.2]))
    vmax = int(rng.choice([1, 17, 300]))

    def val():
        return None if rng.random() < tomb_p else rng.bytes(int(rng.integers(0, vmax)))

    a_keys, b_keys = [], []
    for k in keys:
        r = rng.random()
        if r < overlap / 2:
            a_keys.append(k)
            b_keys.append(k)
        elif r < 0.5 + overlap / 4:
            a_keys.append(k)
        else:
            b_keys.append(k)
    A = gen.side_from_records([(k, val()) for k in a_keys])
    B = gen.side_from_records([(k, val()) for k in b_keys])
    return A, B


@pytest.mark.parametrize("seed", range(96))
def test_random_pairs_every_path(seed):
    import merge_front_coded_amd as em
    A, B = _random_pair(seed)
    print(f"seed {seed}: {A.n}+{B.n} records", flush=True)
    items = [1, 7, 64, 256, 2048][seed % 5]
    check_path(A, B, items=items, path="merge")
    check_path(A, B, items=items, path="fused")
    check_path(A, B, items=min(items, 1024), path="fused", one_pass=True)
    check_path(A, B, items=items, path="collision", collision_mode="512-tiled")
    # the byte profile and the decode of the payload
    pl = run_gpu(A, B, items=items, path="merge")
    W, T = pl.byte_profile()
    torch.cuda.synchronize()
    ref = oracle.run(A, B, items_per_part=256)
    bp = oracle.bp_encode(A, B, ref["final"])
    assert (W, T) == (bp["width"], bp["T"])
    assert np.array_equal(pl.bp_payload[:T].cpu().numpy(), bp["payload"])
    S = pl.S
    want = oracle.fc_decode(np.frombuffer(pl.payload_bytes(), np.uint8), pl.T, S,
                            int(A.keys.size + B.keys.size) + 16, int(A.vals.size + B.vals.size) + 16)
    d = em.fcin_decode(pl.payload, pl.T, S, off=pl.off)
    assert (d.key_bytes, d.val_bytes) == (want.keys.size, want.vals.size)
    assert np.array_equal(d.keys[:d.key_bytes].cpu().numpy(), want.keys)
    assert np.array_equal(d.vals[:d.val_bytes].cpu().numpy(), want.vals)
    assert np.array_equal(d.key_off[:S + 1].cpu().numpy().view(np.uint32), want.key_off)
    assert np.array_equal(d.tomb[:S].cpu().numpy(), want.tomb)
