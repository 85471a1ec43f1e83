"""Full-size parity: every output of the HIP path (and the output navigation
sections built from it) on the five full-size workloads, with the partition
size the pipeline chooses from the mean key length and every per-record array
kept (final references, ordinals, lengths, LCPs, offsets), against SHA-256
digests of the CPU oracle's outputs written by
tests/golden/make_full_size_digests.py (which calls only gen/ and oracle/).
The benchmark's own configuration, which keeps none of the per-record arrays,
is checked in test_gpu_bench_config.py.

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


def _copy_runs(dst, dst_start, src, src_start, lens):
    """dst[dst_start[t] + u] = src[src_start[t] + u] for u < lens[t], all t at once."""
    lens = lens.astype(np.int64)
    total = int(lens.sum())
    if total == 0:
        return
    before = np.zeros(lens.size, np.int64)
    np.cumsum(lens[:-1], out=before[1:])
    step = np.arange(total, dtype=np.int64)
    dst[np.repeat(dst_start.astype(np.int64) - before, lens) + step] = \
        src[np.repeat(src_start.astype(np.int64) - before, lens) + step]


def _merged_side(A, B, final):
    """The survivors' records as one side: keys, values and tombstone flags
    taken from the inputs through the final references."""
    final = final.astype(np.int64)
    isA = final < A.n
    n = final.size
    klen = np.zeros(n, np.int64)
    vlen = np.zeros(n, np.int64)
    tomb = np.zeros(n, np.uint8)
    srcs = []
    for side, mask, idx in ((A, isA, final), (B, ~isA, final - A.n)):
        sel = np.nonzero(mask)[0]
        r = idx[sel]
        ko, vo = side.key_off.astype(np.int64), side.val_off.astype(np.int64)
        klen[sel] = ko[r + 1] - ko[r]
        tomb[sel] = side.tomb[r]
        vlen[sel] = np.where(side.tomb[r] != 0, 0, vo[r + 1] - vo[r])
        srcs.append((side, sel, r))
    key_off = np.zeros(n + 1, np.int64)
    np.cumsum(klen, out=key_off[1:])
    val_off = np.zeros(n + 1, np.int64)
    np.cumsum(vlen, out=val_off[1:])
    keys = np.empty(int(key_off[-1]), np.uint8)
    vals = np.empty(int(val_off[-1]), np.uint8)
    for side, sel, r in srcs:
        _copy_runs(keys, key_off[sel], side.keys, side.key_off[r], klen[sel])
        _copy_runs(vals, val_off[sel], side.vals, side.val_off[r], vlen[sel])
    return keys, key_off.astype(np.uint32), vals, val_off.astype(np.uint32), tomb


def _byte_profile_digest(pl):
    """The byte-profile encoding of a run, digested as the oracle's is."""
    import merge_front_coded_amd as em
    W, T = pl.byte_profile()
    torch.cuda.synchronize()
    S = pl.S
    assert int(pl.bp_over.item()) == 0
    sec = em.EfSections(em.em_ef_entry_count(S))
    em.em_bp_navigation(pl.bp_off, S, T, pl.bp_width, sec)
    nav = sec.host()
    head = np.array([nav[k] for k in ("n", "L", "width", "low_words", "high_bits", "high_words", "groups",
                                      "n_exceptions")], np.uint64)
    out = {"width": W, "T": T, "len_bytes": _sha(pl.bp_len[:S].cpu().numpy()),
           "off": _sha(pl.bp_off[:S + 1].cpu().numpy()), "payload": _sha(pl.bp_payload[:T].cpu().numpy()),
           "ef": _sha(head, nav["lows"], nav["highs"], nav["samples"], nav["exceptions"])}
    del sec
    pl.bp_payload = None
    return out


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_full_size_workload_matches_oracle(wid):
    with open(DIGESTS) as f:
        ref = json.load(f)[str(wid)]
    print(f"full-size workload {wid} ({ref['workload']})", flush=True)
    A, B = gen.make(wid)
    assert _sha(A.keys, A.key_off, A.vals, A.val_off, A.tomb, B.keys, B.key_off, B.vals, B.val_off,
                B.tomb) == ref["input"], "generator output drifted from the digested inputs"
    runs = [("fused", {}), ("fused", {"one_pass": True}), ("merge", {})] + [("collision", {"collision_mode": m})
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
        got["bp"] = _byte_profile_digest(pl)
        want = dict(ref)
        if path == "merge":
            got["splits"] = _sha(pl.host("splits"))
            want["splits"] = ref["splits"][str(pl.items)]
        bad = [k for k, v in got.items() if v != want[k]]
        assert not bad, f"{path}: outputs differing from the oracle: {bad}"
        if path == "merge":
            # the payload decoded back (front-coded input path), block starts
            # from the offsets and from the navigation: the survivors' records
            import merge_front_coded_amd as em
            keys, key_off, vals, val_off, tomb = _merged_side(A, B, pl.host("final", S).astype(np.int64))
            for how in ("off", "navigation"):
                print(f"  decode the payload, block starts from {how}", flush=True)
                d = em.fcin_decode(pl.payload, pl.T, S, **({"off": pl.off} if how == "off" else {"nav": pl.nav}))
                torch.cuda.synchronize()
                assert (d.key_bytes, d.val_bytes) == (keys.size, vals.size), how
                assert np.array_equal(d.key_off[:S + 1].cpu().numpy().view(np.uint32), key_off), how
                assert np.array_equal(d.val_off[:S + 1].cpu().numpy().view(np.uint32), val_off), how
                assert np.array_equal(d.tomb[:S].cpu().numpy(), tomb), how
                assert np.array_equal(d.keys[:keys.size].cpu().numpy(), keys), how
                assert np.array_equal(d.vals[:vals.size].cpu().numpy(), vals), how
                del d
                torch.cuda.empty_cache()
        del pl
        torch.cuda.empty_cache()
