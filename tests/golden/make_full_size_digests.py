#!/usr/bin/env python3
"""Write full_size_digests.json: SHA-256 digests of the CPU oracle's outputs on
the five full-size seeded workloads, so that the GPU parity tests can compare
every output element (through its digest) without rerunning the bit-at-a-time
oracle on the GPU host.

Calls only gen/ (inputs) and oracle/ (expected values).  Run from the
repository root:  python tests/golden/make_full_size_digests.py [ids...]
"""
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import gen  # noqa: E402
import oracle  # noqa: E402

OUT = os.path.join(HERE, "full_size_digests.json")
ITEM_SIZES = (256, 512, 1024, 2048, 4096)  # every partition size the library accepts in tiles


def sha(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(a.tobytes())
    return h.hexdigest()


def input_digest(A, B) -> str:
    return sha(A.keys, A.key_off, A.vals, A.val_off, A.tomb, B.keys, B.key_off, B.vals, B.val_off,
               B.tomb)


def ef_digest(nav) -> str:
    """The navigation header fields and sections, in a fixed order."""
    import numpy as np
    head = np.array([nav[k] for k in ("n", "L", "width", "low_words", "high_bits", "high_words", "groups",
                                      "n_exceptions")], np.uint64)
    return sha(head, nav["lows"], nav["highs"], nav["samples"], nav["exceptions"])


def bp_digest(A, B, final) -> dict:
    """The byte-profile encoding: width, T, and digests of the record lengths,
    byte offsets, payload and the navigation over the byte offsets."""
    bp = oracle.bp_encode(A, B, final)
    S = int(final.size)
    nav = oracle.ef_encode(oracle.ef_entries(bp["off"], S, bp["T"], bp["width"]), bp["width"])
    return {"width": bp["width"], "T": bp["T"], "len_bytes": sha(bp["len_bytes"]), "off": sha(bp["off"]),
            "payload": sha(bp["payload"]), "ef": ef_digest(nav)}


def main(ids):
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    for wid in ids:
        t0 = time.time()
        A, B = gen.make(wid)
        refs = oracle.merge(A, B)
        final, ord_A, ord_B, S = oracle.keep(A, B, refs)
        len_bits, lcp_bits, off, T, payload = oracle.encode(A, B, final)
        data[str(wid)] = {
            "workload": gen.WORKLOADS[wid].name, "nA": A.n, "nB": B.n,
            "input": input_digest(A, B), "S": S, "T": T,
            "splits": {str(i): sha(oracle.splits(refs, A.n, i)) for i in ITEM_SIZES},
            "final": sha(final), "ord_A": sha(ord_A), "ord_B": sha(ord_B),
            "len_bits": sha(len_bits), "lcp_bits": sha(lcp_bits), "off": sha(off),
            "payload": sha(payload), "payload_bytes": int(payload.size),
            "ef": ef_digest(oracle.ef_navigation(A, B, final, off, T)),
            "bp": bp_digest(A, B, final),
        }
        print(f"workload {wid}: S={S} T={T} ({time.time() - t0:.1f}s)", flush=True)
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main([int(x) for x in sys.argv[1:]] or [1, 2, 3, 4, 5])
