"""Independent reader of the byte-profile payload, used as a pin.

Written from the byte-profile page ("Pipeline": byte LEB128 counts, byte FC
literals, optional-value tags, a common encoded value width) and the control
rule counted in bytes, reading the payload rather than producing it: it
shares nothing with the oracle's encoder.  Pure Python, small payloads only.
"""
from __future__ import annotations


def leb(data: bytes, at: int):
    """Unsigned little-endian base-128 value at `at` -> (value, next position)."""
    v, shift = 0, 0
    while True:
        b = data[at]
        at += 1
        v |= (b & 127) << shift
        shift += 7
        if b < 128:
            return v, at


def decode(payload: bytes, S: int, width: int):
    """S records -> list of (key, value or None) and the record start offsets."""
    out, starts = [], []
    at, prev = 0, b""
    for i in range(S):
        starts.append(at)
        c, at = leb(payload, at)
        s, at = leb(payload, at)
        l = c - 1 if i % 15 == 0 else len(prev) - c
        if l < 0 or l > len(prev):
            raise ValueError(f"record {i}: inherited prefix {l} outside the predecessor")
        key = prev[:l] + payload[at:at + s]
        at += s
        tag = payload[at]
        at += 1
        if width:
            body = payload[at:at + width - 1]
            at += width - 1
            val = body if tag else None
            if not tag and any(body):
                raise ValueError(f"record {i}: tombstone filler is not zero")
        elif tag:
            n, at = leb(payload, at)
            val = payload[at:at + n]
            at += n
        else:
            val = None
        out.append((key, val))
        prev = key
    if at != len(payload):
        raise ValueError(f"decoded {at} bytes, payload holds {len(payload)}")
    return out, starts
