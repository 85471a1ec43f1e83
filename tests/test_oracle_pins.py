"""Pins for the CPU oracle: the pages' worked examples, closed forms, an
independent decoder, brute-force set semantics and hand-derived payloads.

Each check is chosen so that a plausible slip in the oracle (ties to the wrong
side, a dropped field, an off-by-one in the W15 rule, a wrong bit order, a
wrong ordinal formula term) fails at least one of them.
"""
import itertools
import json
import os
import random

import numpy as np
import pytest

import gen
import oracle
from fcdecode import decode, eg0_length, replace_merge, trailing_zero

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _int_side(vals):
    """Integers as 4-byte big-endian keys: bytewise order is numeric order."""
    return gen.side_from_records([(int(v).to_bytes(4, "big"), b"") for v in vals])


def _merged_values(A, B, refs):
    nA = A.n
    return [int.from_bytes(A.key(r) if r < nA else B.key(r - nA), "big") for r in refs]


# ---- merge and co-rank: the pages' worked examples ----

def test_merge_path_worked_example():
    g = _load("merge_path_worked_example.json")
    A, B = _int_side(g["a"]), _int_side(g["b"])
    refs = oracle.merge(A, B)
    assert _merged_values(A, B, refs) == g["merged"]
    path = " ".join("down" if r < A.n else "right" for r in refs)
    assert path == g["path"]
    assert oracle.corank(refs, A.n, 3) == g["diagonal_3_crosses_at_i"]
    sp = oracle.splits(refs, A.n, 2)
    assert oracle.diagonals(len(refs), 2) == g["slice_boundaries_k"]
    # each slice between consecutive crossings holds exactly its A and B spans
    for p in range(len(sp) - 1):
        d0, d1 = g["slice_boundaries_k"][p], g["slice_boundaries_k"][p + 1]
        got = sorted(_merged_values(A, B, refs[d0:d1]))
        want = sorted(g["a"][sp[p]:sp[p + 1]] + g["b"][d0 - sp[p]:d1 - sp[p + 1]])
        assert got == want


def test_dsa_corank_table():
    g = _load("dsa_corank_table.json")
    A, B = _int_side(g["A"]), _int_side(g["B"])
    refs = oracle.merge(A, B)
    assert _merged_values(A, B, refs) == g["merged"]
    for k, (i, j) in enumerate(g["corank_ij"]):
        assert oracle.corank(refs, A.n, k) == i and k - i == j


def test_corank_ties_go_to_older_side():
    g = _load("merge_path_ties_and_termination.json")["tie_case"]
    A, B = _int_side(g["a"]), _int_side(g["b"])
    refs = oracle.merge(A, B)
    assert _merged_values(A, B, refs) == g["values"]
    i = oracle.corank(refs, A.n, g["k"])
    assert i == g["corank"]
    assert (i, g["k"] - i) == (g["second_slice_starts_at"]["a"], g["second_slice_starts_at"]["b"])
    # provenance, not values: the first equal pair takes a before b
    assert [r < A.n for r in refs] == [True, True, False, False, False, True]


def test_corank_termination_case():
    g = _load("merge_path_ties_and_termination.json")["termination_case"]
    A, B = _int_side(g["a"]), _int_side(g["b"])
    refs = oracle.merge(A, B)
    assert oracle.corank(refs, A.n, g["k"]) == g["corank"]


# ---- closed forms ----

def test_eg0_closed_form_matches_textbook_code():
    # E(x) from the record grammar equals the length of the textbook order-0
    # Exp-Golomb code written out independently here.
    for x in list(range(0, 1 << 16)) + [2**20 - 1, 2**20, 2**30, 2**31 - 1]:
        y = bin(x + 1)[2:]
        code = "0" * (len(y) - 1) + y
        assert len(code) == eg0_length(x)


def _closed_form_lengths(records, W=15):
    """E(c)+E(k-l)+(k-l)+v per survivor, from the record grammar paragraph."""
    out = []
    prev = None
    for i, (k, _, v) in enumerate(records):
        kb = 8 * len(k)
        if i == 0:
            l = 0
        else:
            pb = "".join(f"{b:08b}" for b in prev)
            xb = "".join(f"{b:08b}" for b in k)
            l = 0
            while l < min(len(pb), len(xb)) and pb[l] == xb[l]:
                l += 1
        c = 1 + l if i % W == 0 else 8 * len(prev) - l
        vbits = 1 if v is None else 1 + eg0_length(len(v)) + 8 * len(v)
        out.append(eg0_length(c) + eg0_length(kb - l) + (kb - l) + vbits)
        prev = k
    return out


# ---- hand-derived payloads (readings of the record grammar, field by field) ----

def test_one_record_payload_bits():
    # key "a" (0x61), present empty value, first record:
    #   c0 = 1 + 0 = 1      EG0(1)  = 010
    #   k - l = 8           EG0(8)  = 0001001
    #   key bits 0..7       0x61    = 01100001
    #   present value       1, EG0(0) = 1
    bits = "010" + "0001001" + "01100001" + "1" + "1"
    A = gen.side_from_records([(b"a", b"")])
    B = gen.side_from_records([])
    r = oracle.run(A, B)
    assert r["T"] == len(bits) == 20
    padded = bits + "0" * (32 - len(bits))
    want = bytes(int(padded[i:i + 8], 2) for i in range(0, 32, 8))
    assert r["payload"].tobytes() == want == bytes.fromhex("42587000")


def test_merge_example_payload_bits():
    # A = {ab: "1", b: ""}, B = {ab: tombstone, abc: "Z"}; B's ab replaces A's.
    A = gen.side_from_records([(b"ab", b"1"), (b"b", b"")])
    B = gen.side_from_records([(b"ab", None), (b"abc", b"Z")])
    r = oracle.run(A, B)
    assert list(r["final"]) == [2, 3, 1]              # B0, B1, A1
    assert list(r["ord_A"]) == [oracle.NONE, 2] and list(r["ord_B"]) == [0, 1]
    rec0 = "010" + "000010001" + "0110000101100010" + "0"          # ab, l=0, c=1, tombstone
    rec1 = "1" + "0001001" + "01100011" + "1" + "010" + "01011010"  # abc, l=16, c=16-16=0, "Z"
    rec2 = "000010011" + "011" + "10" + "1" + "1"                  # b, l=6, c=24-6=18, ""
    assert [len(rec0), len(rec1), len(rec2)] == list(r["len_bits"]) == [29, 28, 16]
    assert list(r["lcp_bits"]) == [0, 16, 6]
    assert list(r["off"]) == [0, 29, 57, 73] and r["T"] == 73
    bits = rec0 + rec1 + rec2
    bits += "0" * (-len(bits) % 32)
    want = bytes(int(bits[i:i + 8], 2) for i in range(0, len(bits), 8))
    assert r["payload"].tobytes() == want
    assert want.hex() == "411616244b1d2d04dd800000"


def test_w15_phase_resets_control_to_absolute_length():
    # 17 records sharing long prefixes: records 0 and 15 carry c = 1 + l.
    keys = [b"prefix/" + bytes([0x41 + i]) + b"tail" for i in range(17)]
    A = gen.side_from_records([(k, b"v") for k in keys[::2]])
    B = gen.side_from_records([(k, None) for k in keys[1::2]])
    r = oracle.run(A, B)
    recs, info = decode(r["payload"].tobytes(), r["T"], r["S"])
    assert [k for k, _ in recs] == keys
    for i, d in enumerate(info):
        if i % 15 == 0:
            assert d["c"] == 1 + d["l"]
        else:
            assert d["c"] == info[i - 1]["k"] - d["l"]
    assert info[15]["l"] == 8 * len(b"prefix/") + 3  # 'O' 01001111 vs 'P' 01010000: bit 3
    assert info[15]["c"] == 1 + info[15]["l"]


# ---- brute force over tiny key universes ----

def _universe(alphabet, maxlen):
    keys = [b""]
    for L in range(1, maxlen + 1):
        keys += [bytes(t) for t in itertools.product(alphabet, repeat=L)]
    return sorted(keys)


def _check_case(a_recs, b_recs, items=3):
    A = gen.side_from_records(a_recs)
    B = gen.side_from_records(b_recs)
    r = oracle.run(A, B, items_per_part=items)
    # merge: stable, ties to A  (sort (key, side) pairs: A=0 before B=1)
    tagged = sorted([(k, 0, i) for i, (k, _) in enumerate(a_recs)]
                    + [(k, 1, j) for j, (k, _) in enumerate(b_recs)])
    want_refs = [i if s == 0 else A.n + i for _, s, i in tagged]
    assert list(r["refs"]) == want_refs
    for d, i in zip(oracle.diagonals(len(want_refs), items), r["splits"]):
        assert i == sum(1 for x in want_refs[:d] if x < A.n)
    # keep-newer: set semantics
    want = replace_merge(a_recs, b_recs)
    got = []
    for ref in r["final"]:
        if ref < A.n:
            got.append((A.key(ref), "A", A.value(ref)))
        else:
            got.append((B.key(ref - A.n), "B", B.value(ref - A.n)))
    assert got == want
    both = len({k for k, _ in a_recs} & {k for k, _ in b_recs})
    assert r["S"] == A.n + B.n - both
    # every B record survives; ordinals are positions in the final order
    assert all(o != oracle.NONE for o in r["ord_B"])
    for s, ref in enumerate(r["final"]):
        o = r["ord_A"][ref] if ref < A.n else r["ord_B"][ref - A.n]
        assert o == s
    assert sum(o == oracle.NONE for o in r["ord_A"]) == both
    # collision-bit formulas give the same ordinals and final order
    c = oracle.collision(A, B)
    assert np.array_equal(c["ord_A"], r["ord_A"]) and np.array_equal(c["ord_B"], r["ord_B"])
    assert np.array_equal(c["final"], r["final"]) and c["S"] == r["S"]
    assert int(c["R"][-1]) == both
    # decode the payload independently; lengths match the closed form
    recs, info = decode(r["payload"].tobytes(), r["T"], r["S"])
    assert recs == [(k, v) for k, _, v in want]
    assert list(r["len_bits"]) == _closed_form_lengths(want) == [d["length"] for d in info]
    assert list(r["off"][:-1]) == [d["start"] for d in info]
    assert r["T"] == sum(int(x) for x in r["len_bits"]) == int(r["off"][-1])
    assert len(r["payload"]) == 4 * ((r["T"] + 31) // 32)
    assert trailing_zero(r["payload"].tobytes(), r["T"])
    return r


def _rand_value(rng):
    if rng.random() < 0.2:
        return None
    return bytes(rng.randrange(256) for _ in range(rng.randrange(4)))


def test_brute_force_all_pairs_small_universe():
    # keys: "", 00, 61, FF: all 16 x 16 pairs of subsets
    U = _universe([0x00, 0x61, 0xFF], 1)
    rng = random.Random(7)
    for ma in range(1 << len(U)):
        for mb in range(1 << len(U)):
            a = [(k, _rand_value(rng)) for t, k in enumerate(U) if ma >> t & 1]
            b = [(k, _rand_value(rng)) for t, k in enumerate(U) if mb >> t & 1]
            _check_case(a, b)


def test_brute_force_random_subsets_larger_universe():
    # all strings of length <= 2 over {00, 61, FF}: 13 keys, proper prefixes, NUL bytes
    U = _universe([0x00, 0x61, 0xFF], 2)
    assert len(U) == 13
    rng = random.Random(11)
    for _ in range(600):
        a = [(k, _rand_value(rng)) for k in U if rng.random() < 0.5]
        b = [(k, _rand_value(rng)) for k in U if rng.random() < 0.5]
        _check_case(a, b, items=rng.choice([1, 2, 3, 5, 64]))


def test_edge_cases_empty_inputs():
    r = _check_case([], [])
    assert r["S"] == 0 and r["T"] == 0 and len(r["payload"]) == 0
    _check_case([(b"k", b"v")], [])
    _check_case([], [(b"k", None)])
    _check_case([(b"", b"")], [(b"", None)])   # the empty key, replaced by a tombstone


def test_random_workload_roundtrip():
    A, B = gen.make(gen.WORKLOADS[1].scaled(0.15))
    r = _check_case(A.records(), B.records(), items=37)
    assert r["S"] > 2000


def test_long_records_span_many_words():
    rng = random.Random(3)
    a = sorted({bytes(rng.randrange(256) for _ in range(rng.randrange(40, 300))) for _ in range(40)})
    recs = [(k, bytes(rng.randrange(256) for _ in range(rng.randrange(0, 600)))) for k in a]
    _check_case(recs[::2], [(k, None if i % 3 == 0 else v) for i, (k, v) in enumerate(recs[1::2])])


# ---- rank ----

def test_rank_scalar_prefix_counts():
    rng = np.random.default_rng(5)
    for nbits in (0, 1, 31, 32, 33, 63, 64, 65, 511, 512, 513, 2047, 2048, 2049):
        for fill in ("zero", "one", "sparse", "random"):
            bits = {"zero": np.zeros(nbits, np.uint8), "one": np.ones(nbits, np.uint8),
                    "sparse": (rng.random(nbits) < 0.01).astype(np.uint8),
                    "random": (rng.random(nbits) < 0.5).astype(np.uint8)}[fill]
            words = np.zeros((nbits + 31) // 32 + 1, np.uint32)
            for q in np.nonzero(bits)[0]:
                words[q >> 5] |= np.uint32(1 << (int(q) & 31))
            pos = list(range(nbits + 1))
            want = np.concatenate([[0], np.cumsum(bits)]).astype(np.uint32)
            assert np.array_equal(oracle.rank(words, pos), want)


def test_key_order_proper_prefix_and_unsigned_bytes():
    A = gen.side_from_records([(b"ab", b""), (b"a\x80", b""), (b"\xff", b"")])
    B = gen.side_from_records([(b"a", b""), (b"ab\x00", b""), (b"b", b"")])
    assert oracle.key_cmp(A, 0, B, 0) > 0      # "ab" > "a": proper prefix first
    assert oracle.key_cmp(A, 0, B, 1) < 0      # "ab" < "ab\0"
    assert oracle.key_cmp(A, 1, B, 2) < 0      # 0x61 < 0x62 regardless of later bytes
    assert oracle.key_cmp(A, 2, B, 2) > 0      # 0xff is large: unsigned bytes
    assert oracle.key_cmp(A, 0, A, 0) == 0


def test_key_lcp_bits_closed_forms_and_brute_force():
    """Bit LCP of two keys: hand values, then every pair of a small random
    set against a bit-string comparison written out here."""
    A = gen.side_from_records([(b"ab", b""), (b"\x80", b""), (b"abc", b"")])
    B = gen.side_from_records([(b"a", b""), (b"ab", b""), (b"\x00", b""), (b"abd", b""), (b"", b"")])
    assert oracle.key_lcp_bits(A, 0, B, 1) == 16   # identical keys: all their bits
    assert oracle.key_lcp_bits(A, 0, B, 0) == 8    # a proper prefix: the shorter key's bits
    assert oracle.key_lcp_bits(A, 1, B, 2) == 0    # the first bit differs
    assert oracle.key_lcp_bits(A, 2, B, 3) == 21   # 'c' = 0x63, 'd' = 0x64: six equal high bits
    assert oracle.key_lcp_bits(A, 0, B, 4) == 0    # an empty key
    rng = np.random.default_rng(5)
    keys = sorted({bytes(rng.integers(0, 3, int(rng.integers(0, 5)), dtype=np.uint8)) for _ in range(60)})
    X = gen.side_from_records([(k, b"") for k in keys])

    def bits(k):
        return "".join(format(c, "08b") for c in k)

    for i, ki in enumerate(keys):
        for j, kj in enumerate(keys):
            bi, bj = bits(ki), bits(kj)
            n = 0
            while n < min(len(bi), len(bj)) and bi[n] == bj[n]:
                n += 1
            assert oracle.key_lcp_bits(X, i, X, j) == n, (ki, kj)


# ---- output navigation: Elias-Fano sections of the sampled offsets ----

def test_ef_hand_examples():
    # e = 0, 5, 9, 20: (20 + 1) // 4 = 5 -> L = 2.  Lows 0, 1, 1, 0 at bits
    # 0, 2, 4, 6 -> 0b00010100.  Highs: e >> 2 = 0, 1, 2, 5, plus k -> bits
    # 0, 2, 4, 8 -> 0x115, 4 + 5 = 9 bits.  One group, span 9: dense.
    r = oracle.ef_encode(np.array([0, 5, 9, 20], np.uint64))
    assert (r["n"], r["L"], r["high_bits"], r["groups"], r["n_exceptions"]) == (4, 2, 9, 1, 0)
    assert [int(x) for x in r["lows"]] == [0x14] and [int(x) for x in r["highs"]] == [0x115]
    assert [int(x) for x in r["samples"]] == [0, 0]
    # repeated entries 0, 0, 1, 3: (3 + 1) // 4 = 1 -> L = 0, no low words;
    # highs at 0, 1, 3, 6 -> 0b1001011, 4 + 3 = 7 bits.
    r = oracle.ef_encode(np.array([0, 0, 1, 3], np.uint64))
    assert (r["L"], r["low_words"], r["high_bits"]) == (0, 0, 7)
    assert [int(x) for x in r["highs"]] == [0x4B]
    # a single entry (empty payload): L = 0, high bit 0
    r = oracle.ef_encode(np.array([0], np.uint64))
    assert (r["n"], r["L"], r["high_bits"], [int(x) for x in r["highs"]]) == (1, 0, 1, [1])


@pytest.mark.parametrize("n", [1, 2, 255, 256, 257, 700, 3000])
def test_ef_round_trip(n):
    from efdecode import popcount, select_all
    rng = np.random.default_rng(n)
    for shape in ("uniform", "clustered", "repeats"):
        if shape == "uniform":
            gaps = rng.integers(0, 1000, n)
        elif shape == "clustered":  # long quiet stretches, then bursts: sparse groups
            gaps = np.where(rng.random(n) < 0.02, rng.integers(10 ** 5, 10 ** 6, n), rng.integers(0, 3, n))
        else:
            gaps = rng.integers(0, 2, n)
        e = np.cumsum(gaps).astype(np.uint64)
        r = oracle.ef_encode(e)
        assert select_all(r) == [int(x) for x in e], f"n={n} {shape}"
        assert popcount(r["highs"]) == n
        # canonical padding: nothing set past the sections' lengths
        assert r["high_bits"] == n + (int(e[-1]) >> r["L"])
        if r["high_bits"] % 64:
            assert int(r["highs"][-1]) >> (r["high_bits"] % 64) == 0
        if (n * r["L"]) % 64:
            assert int(r["lows"][-1]) >> ((n * r["L"]) % 64) == 0
        # L = floor(log2((last + 1) // n)) from its definition
        q = (int(e[-1]) + 1) // n
        assert r["L"] == (q.bit_length() - 1 if q else 0)


@pytest.mark.parametrize("top", [3839, 3840])
def test_ef_sparse_threshold(top):
    # 2048 entries, all at most 3840, so (3840 + 1) // 2048 = 1 and L = 0:
    # position p_k = e_k + k.  Group 0 runs from e_0 = 0 to e_255 = top, so its
    # span is top + 255 + 1: 4095 (dense) or 4096 (sparse).  The other groups
    # sit on one value and span 256.
    e = np.concatenate([np.linspace(0, top, 256).round(), np.full(2048 - 256, 3840)]).astype(np.uint64)
    r = oracle.ef_encode(e)
    assert r["L"] == 0
    sparse = top + 256 >= 4096
    assert r["n_exceptions"] == (256 if sparse else 0)
    if sparse:
        assert [int(x) for x in r["exceptions"]] == [int(e[k]) + k for k in range(256)]
    assert [int(x) for x in r["samples"][1::2]] == [0] + [256 if sparse else 0] * 7
    from efdecode import select_all
    assert select_all(r) == [int(x) for x in e]


def test_ef_navigation_of_merged_payloads():
    # the hand-derived merge: widths 1 (tombstone), 1 + E(1) + 8 = 12 and
    # 1 + E(0) = 2 differ, so w = 0: entries off[0] = 0 and T = 73
    A = gen.side_from_records([(b"ab", b"1"), (b"b", b"")])
    B = gen.side_from_records([(b"ab", None), (b"abc", b"Z")])
    r = oracle.run(A, B)
    nav = oracle.ef_navigation(A, B, r["final"], r["off"], r["T"])
    assert nav["width"] == 0 and nav["n"] == 2
    from efdecode import select_all
    assert select_all(nav) == [0, 73]
    # fixed-width values: every record's value is 1 + E(16) + 128 = 138 bits,
    # read back from the payload by the independent decoder
    keys = [b"k%04d" % i for i in range(40)]
    A = gen.side_from_records([(k, bytes(16)) for k in keys[::2]])
    B = gen.side_from_records([(k, bytes([i]) * 16) for i, k in enumerate(keys[1::2])])
    r = oracle.run(A, B)
    recs, info = decode(r["payload"].tobytes(), r["T"], r["S"])
    widths = {i["length"] - eg0_length(i["c"]) - eg0_length(i["k"] - i["l"]) - (i["k"] - i["l"]) for i in info}
    assert widths == {138}
    nav = oracle.ef_navigation(A, B, r["final"], r["off"], r["T"])
    assert nav["width"] == 138 and nav["n"] == (40 + 14) // 15 + 1
    starts = [i["start"] for i in info]
    want = [starts[o] - 138 * o for o in range(0, 40, 15)] + [r["T"] - 138 * 40]
    assert select_all(nav) == want


# ---- compressed input: the payload decoded back into arenas ----

def _merged_records(A, B, final):
    nA = A.n
    return [(A.key(r), A.value(r)) if r < nA else (B.key(r - nA), B.value(r - nA)) for r in final]


def test_fc_decode_hand_example():
    payload = np.frombuffer(bytes.fromhex("411616244b1d2d04dd800000"), np.uint8)
    side = oracle.fc_decode(payload, 73, 3, 64, 64)
    assert side.records() == [(b"ab", None), (b"abc", b"Z"), (b"b", b"")]
    assert list(side.key_off) == [0, 2, 5, 6] and list(side.val_off) == [0, 0, 1, 1]
    with pytest.raises(ValueError):  # one bit short
        oracle.fc_decode(payload, 72, 3, 64, 64)
    with pytest.raises(ValueError):  # a bit left over after the last record
        oracle.fc_decode(payload, 74, 3, 64, 64)
    with pytest.raises(ValueError):  # key arena too small
        oracle.fc_decode(payload, 73, 3, 5, 64)


@pytest.mark.parametrize("seed", range(6))
def test_fc_decode_round_trip(seed):
    rng = random.Random(seed)
    alpha = [0x00, 0x01, 0x61, 0x7F, 0x80, 0xFF]
    keys = sorted({bytes(rng.choice(alpha) for _ in range(rng.randrange(0, 9))) for _ in range(400)})
    a, b = [], []
    for k in keys:
        u = rng.random()
        val = (lambda: None if rng.random() < 0.15 else bytes(rng.randrange(256) for _ in range(rng.randrange(0, 7))))
        if u < 0.3:
            a.append((k, val()))
            b.append((k, val()))
        elif u < 0.65:
            a.append((k, val()))
        else:
            b.append((k, val()))
    A, B = gen.side_from_records(a), gen.side_from_records(b)
    r = oracle.run(A, B)
    want = _merged_records(A, B, r["final"])
    side = oracle.fc_decode(r["payload"], r["T"], r["S"], 16 * len(want) + 16, 16 * len(want) + 16)
    assert side.records() == want
    # and the independent Python decoder reads the same records
    recs, _ = decode(r["payload"].tobytes(), r["T"], r["S"])
    assert recs == want


# ---- byte profile: LEB128 counts, byte literals, presence tags ----

def test_bp_hand_examples():
    # ab (tombstone), abc ("Z"), b (""): present lengths 1 and 0 differ, so
    # variable framing.  ab: c = 1, s = 2, 'ab', tag 0.  abc: l = 2,
    # c = 2 - 2 = 0, s = 1, 'c', tag 1, length 1, 'Z'.  b: l = 0, c = 3 - 0 = 3,
    # s = 1, 'b', tag 1, length 0.
    A = gen.side_from_records([(b"ab", b"1"), (b"b", b"")])
    B = gen.side_from_records([(b"ab", None), (b"abc", b"Z")])
    r = oracle.run(A, B)
    bp = oracle.bp_encode(A, B, r["final"])
    assert bp["width"] == 0
    assert bp["payload"].tobytes().hex() == "0102616200" + "00016301015a" + "0301620100"
    assert list(bp["off"]) == [0, 5, 11, 16] and bp["T"] == 16
    assert list(bp["lcp_bytes"]) == [0, 2, 0] and list(bp["len_bytes"]) == [5, 6, 5]
    # k1 (tombstone), k2 ("yy"): the one present length is 2, so width 3;
    # the tombstone's value is tag 0 and two zero bytes
    A = gen.side_from_records([(b"k1", b"xx"), (b"k2", b"yy")])
    B = gen.side_from_records([(b"k1", None)])
    r = oracle.run(A, B)
    bp = oracle.bp_encode(A, B, r["final"])
    assert bp["width"] == 3
    assert bp["payload"].tobytes().hex() == "01026b31000000" + "0101320179 79".replace(" ", "")
    # LEB128 at 128 and 200: a 200-byte key (s = 200 -> c8 01) and a 128-byte
    # value under variable framing (length -> 80 01)
    A = gen.side_from_records([(b"x" * 200, b"v" * 128), (b"y", b"")])
    r = oracle.run(A, gen.side_from_records([]))
    bp = oracle.bp_encode(A, gen.side_from_records([]), r["final"])
    p = bp["payload"].tobytes()
    assert bp["width"] == 0
    assert p[:3].hex() == "01c801" and p[203:206].hex() == "018001"


@pytest.mark.parametrize("seed", range(5))
def test_bp_round_trip(seed):
    from bpdecode import decode as bp_decode
    rng = random.Random(100 + seed)
    alpha = [0x00, 0x41, 0x7F, 0x80, 0xFF]
    keys = sorted({bytes(rng.choice(alpha) for _ in range(rng.randrange(0, 7))) for _ in range(300)}
                  | {b"L" * rng.randrange(120, 260) for _ in range(3)})
    fixed = seed % 2 == 0
    def val():
        if rng.random() < 0.15:
            return None
        return bytes(rng.randrange(256) for _ in range(16 if fixed else rng.randrange(0, 140)))
    a, b = [], []
    for k in keys:
        u = rng.random()
        if u < 0.3:
            a.append((k, val()))
            b.append((k, val()))
        elif u < 0.65:
            a.append((k, val()))
        else:
            b.append((k, val()))
    A, B = gen.side_from_records(a), gen.side_from_records(b)
    r = oracle.run(A, B)
    bp = oracle.bp_encode(A, B, r["final"])
    assert bp["width"] == (17 if fixed else 0)
    recs, starts = bp_decode(bp["payload"].tobytes(), r["S"], bp["width"])
    assert recs == _merged_records(A, B, r["final"])
    assert starts + [bp["T"]] == [int(x) for x in bp["off"]]
    # byte LCPs are the bit LCPs' whole bytes
    assert np.array_equal(bp["lcp_bytes"], r["lcp_bits"] // 8)
