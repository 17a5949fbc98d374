"""Independent exact computations used to pin the oracle (tests only).

Nothing here shares code with ``oracle/``: these are from-the-definition
brute-force versions in exact arithmetic (Python integers and
``fractions.Fraction``), meant for tiny inputs.
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np


def bf16_fraction(bits: int) -> Fraction:
    """Exact rational value of a bf16 bit pattern (finite values)."""
    (f,) = struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))
    return Fraction(f)


def exact_projection(k_bits, P_bits, j) -> Fraction:
    """sum_i k_i * P_ij, exactly."""
    return sum((bf16_fraction(k_bits[i]) * bf16_fraction(P_bits[i, j])
                for i in range(len(k_bits))), Fraction(0))


def exact_sign_code(k_bits, P_bits) -> np.ndarray:
    """Bits [exact projection > 0], packed LSB-first into uint32 words."""
    d, b = P_bits.shape
    words = [0] * (b // 32)
    for j in range(b):
        if exact_projection(k_bits, P_bits, j) > 0:
            words[j // 32] |= 1 << (j % 32)
    return np.array(words, dtype=np.uint32)


def exact_radius_code(r2: Fraction) -> int:
    """Largest m in 1..255 with r2 >= 2^((m-64)/8) (true thresholds), else 0.

    Compares r2^8 with 2^(m-64) in exact rationals."""
    if r2 <= 0:
        return 0
    r2_8 = r2 ** 8
    for m in range(255, 0, -1):
        if r2_8 >= Fraction(2) ** (m - 64):
            return m
    return 0


def round_half_even(x: Fraction) -> int:
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def exact_query_int8(q_bits, P_bits) -> np.ndarray:
    """round_half_even(p*127/M) with exact p and M (one group)."""
    G, d = q_bits.shape
    b = P_bits.shape[1]
    p = [[sum((bf16_fraction(q_bits[h, i]) * bf16_fraction(P_bits[i, j])
               for i in range(d)), Fraction(0)) for j in range(b)] for h in range(G)]
    M = max(abs(v) for row in p for v in row)
    out = np.zeros((G, b), np.int64)
    if M == 0:
        return out
    for h in range(G):
        for j in range(b):
            out[h, j] = max(-127, min(127, round_half_even(p[h][j] * 127 / M)))
    return out


def brute_score(q8, code_words, r8) -> int:
    """r8 * max_h sum_j q8[h,j] * (+1 if bit j else -1), Python integers."""
    G, b = q8.shape
    best = None
    for h in range(G):
        s = 0
        for j in range(b):
            bit = (int(code_words[j // 32]) >> (j % 32)) & 1
            s += int(q8[h, j]) if bit else -int(q8[h, j])
        best = s if best is None else max(best, s)
    return int(r8) * best


def brute_select(S, k, w, sigma):
    """Sinks, window and top-k by a full Python sort on (-score, position)."""
    N = len(S)
    sinks = list(range(min(sigma, N)))
    window = list(range(max(min(sigma, N), N - w), N))
    cand = list(range(sigma, N - w))
    cand.sort(key=lambda i: (-int(S[i]), i))
    top = cand[:max(0, min(k, len(cand)))]
    return sinks, window, top


def brute_select_pages(S, k, w, sigma, page=16):
    """Sinks, window and the keys of the top k//page pages: each page of the
    candidate range scored by a Python max over its candidate keys, pages
    ranked by a full sort on (-page score, page index)."""
    N = len(S)
    sinks = list(range(min(sigma, N)))
    window = list(range(max(min(sigma, N), N - w), N))
    cand = range(sigma, N - w)
    pages = {}
    for i in cand:
        pages.setdefault(i // page, []).append(i)
    ranked = sorted(pages, key=lambda p: (-max(int(S[i]) for i in pages[p]), p))
    top = []
    for p in ranked[:max(0, k // page)]:
        top += pages[p]
    return sinks, window, top


def brute_lsh_bucket(code, t, m):
    """Bits t*m .. t*m+m-1 of a code (uint32 words), by Python integers."""
    big = 0
    for i, wd in enumerate(code):
        big |= int(wd) << (32 * i)
    return (big >> (t * m)) & ((1 << m) - 1)


def brute_select_lsh(S, codes, qbits, T, m, k, w, sigma):
    """Sinks, window and the top-k of the LSH candidates (Python sort)."""
    N = len(S)
    sinks = list(range(min(sigma, N)))
    window = list(range(max(min(sigma, N), N - w), N))
    cand = [i for i in range(sigma, N - w)
            if any(brute_lsh_bucket(codes[i], t, m) == brute_lsh_bucket(qb, t, m)
                   for t in range(T) for qb in qbits)]
    cand.sort(key=lambda i: (-int(S[i]), i))
    return sinks, window, cand[:max(0, k)]
