"""Independent front-coding decoder and set-semantics reference, used as pins.

Written from the record grammar of Everett's "GPU construction experiment"
page (the c_i control equation and the paragraph that follows it), reading
the payload rather than producing it: it shares nothing with the oracle's
encoder.  Pure Python, for small payloads only.
"""
from __future__ import annotations


def eg0_length(x: int) -> int:
    """Closed form from the record grammar paragraph: E(x) = 2 floor(log2(x+1)) + 1."""
    return 2 * ((x + 1).bit_length() - 1) + 1


class BitReader:
    def __init__(self, payload: bytes, nbits: int):
        self.bits = "".join(f"{b:08b}" for b in payload)
        self.n = nbits
        self.pos = 0

    def bit(self) -> int:
        if self.pos >= self.n:
            raise ValueError("read past the end of the payload")
        b = self.bits[self.pos]
        self.pos += 1
        return 1 if b == "1" else 0

    def take(self, n: int) -> str:
        if self.pos + n > self.n:
            raise ValueError("read past the end of the payload")
        s = self.bits[self.pos:self.pos + n]
        self.pos += n
        return s

    def eg0(self) -> int:
        """Order-zero Exp-Golomb: count leading zeros z, then read z+1 bits as x+1."""
        z = 0
        while self.bit() == 0:
            z += 1
        rest = self.take(z)
        return int("1" + rest, 2) - 1


def decode(payload: bytes, T: int, S: int):
    """Decode S records -> list of (key bytes, value bytes or None), plus per-record info."""
    r = BitReader(payload, T)
    out, info = [], []
    prev_bits = ""
    for i in range(S):
        start = r.pos
        c = r.eg0()
        s = r.eg0()
        l = c - 1 if i % 15 == 0 else len(prev_bits) - c
        if l < 0 or l > len(prev_bits):
            raise ValueError(f"record {i}: inherited prefix {l} outside predecessor")
        key_bits = prev_bits[:l] + r.take(s)
        if len(key_bits) % 8:
            raise ValueError(f"record {i}: key is not a whole number of bytes")
        key = bytes(int(key_bits[t:t + 8], 2) for t in range(0, len(key_bits), 8))
        if r.bit():
            vlen = r.eg0()
            vb = r.take(8 * vlen)
            val = bytes(int(vb[t:t + 8], 2) for t in range(0, len(vb), 8))
        else:
            val = None
        out.append((key, val))
        info.append(dict(c=c, l=l, k=len(key_bits), start=start, length=r.pos - start))
        prev_bits = key_bits
    if r.pos != T:
        raise ValueError(f"decoded {r.pos} bits, payload holds {T}")
    return out, info


def trailing_zero(payload: bytes, T: int) -> bool:
    bits = "".join(f"{b:08b}" for b in payload)
    return set(bits[T:]) <= {"0"}


def replace_merge(a_records, b_records):
    """Set semantics of the replacement merge: every distinct key once, the
    newer side's record on a shared key (tombstones included), in unsigned
    bytewise order (Python's bytes order: a proper prefix first)."""
    m = {}
    for k, v in a_records:
        m[k] = ("A", v)
    for k, v in b_records:
        m[k] = ("B", v)
    return [(k, m[k][0], m[k][1]) for k in sorted(m)]
