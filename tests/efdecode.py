"""Independent reader of the output navigation sections, used as a pin.

Written from the section layout the design notes read out of Everett's "GPU
construction experiment" page (the KV03 paragraph and the output-EF
paragraph): it selects entries the way a reader of the file would -- a sparse
group's explicit positions, else a walk of the high bits from the group's
sample -- and shares nothing with the oracle's encoder.  Pure Python, for
small sections only.
"""
from __future__ import annotations


def _bit(words, b: int) -> int:
    return (int(words[b >> 6]) >> (b & 63)) & 1


def select_all(sec: dict) -> list[int]:
    """Every entry, in order, from the lows, highs, samples and exceptions."""
    n, L = sec["n"], sec["L"]
    samples, exc, highs, lows = sec["samples"], sec["exceptions"], sec["highs"], sec["lows"]
    G = (n + 255) // 256
    out = []
    for k in range(n):
        g, r = divmod(k, 256)
        p0, x0 = int(samples[2 * g]), int(samples[2 * g + 1])
        x1 = int(samples[2 * g + 3]) if g + 1 < G else len(exc)
        if x1 > x0:  # a sparse group: its positions are listed
            p = int(exc[x0 + r])
        else:  # a dense group: the r-th set bit from the group's first one
            p, seen = p0, 0
            while True:
                if _bit(highs, p):
                    if seen == r:
                        break
                    seen += 1
                p += 1
        low = 0
        for b in range(L):
            low |= _bit(lows, k * L + b) << b
        out.append(((p - k) << L) | low)
    return out


def popcount(words) -> int:
    return sum(bin(int(w)).count("1") for w in words)
