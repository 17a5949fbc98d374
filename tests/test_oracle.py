"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: a closed
form, an identity, a textbook special case, an exact-arithmetic brute force
(tests/exact.py) or a library routine (torch SDPA in fp64).  Together they
are chosen so that a dropped term, a wrong sign or index, a transposed
operand or a wrong rounding in any oracle step fails at least one test.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from exact import (bf16_fraction, brute_lsh_bucket, brute_score, brute_select,
                   brute_select_lsh, brute_select_pages, exact_projection,
                   exact_query_int8, exact_radius_code, exact_sign_code)
from helpers import bf16_bits, bits_to_float

D = 128


def rand_bits(rng, shape, scale=1.0):
    return bf16_bits(rng.standard_normal(shape).astype(np.float32) * scale)


# ---------------------------------------------------------------- E1 codes
@pytest.mark.parametrize("b", [64, 128, 256])
def test_code_one_hot_key_reads_row_of_P(b):
    """k = 2^e * e_i  =>  bit_j = [P_ij > 0] (closed form)."""
    rng = np.random.default_rng(1)
    P = rand_bits(rng, (D, b))
    Pf = bits_to_float(P)
    for i, e in [(0, 0), (5, 3), (77, -4), (127, 7)]:
        k = np.zeros(D, np.float32)
        k[i] = 2.0 ** e
        code = oracle.key_code(bf16_bits(k), P)
        want = np.zeros(b // 32, np.uint32)
        for j in range(b):
            if Pf[i, j] > 0:
                want[j // 32] |= np.uint32(1 << (j % 32))
        assert np.array_equal(code, want)


def test_code_identity_projection_is_sign_of_key():
    """P = [I_b; 0] (b <= d)  =>  bit_j = [k_j > 0]; also checks bit order."""
    b = 64
    P = np.zeros((D, b), np.float32)
    P[np.arange(b), np.arange(b)] = 1.0
    P = bf16_bits(P)
    rng = np.random.default_rng(2)
    for _ in range(5):
        k = rand_bits(rng, D)
        code = oracle.key_code(k, P)
        kf = bits_to_float(k)
        for j in range(b):
            assert ((int(code[j // 32]) >> (j % 32)) & 1) == int(kf[j] > 0)


def test_code_negation_and_power_of_two_scaling():
    rng = np.random.default_rng(3)
    b = 128
    P = rand_bits(rng, (D, b))
    for _ in range(4):
        kf = bits_to_float(rand_bits(rng, D)).astype(np.float32)
        c = oracle.key_code(bf16_bits(kf), P)
        cneg = oracle.key_code(bf16_bits(-kf), P)
        for e in (-5, 3):
            assert np.array_equal(oracle.key_code(bf16_bits(kf * 2.0 ** e), P), c)
        k_bits = bf16_bits(kf)
        for j in range(b):
            pj = exact_projection(k_bits, P, j)
            bit = (int(c[j // 32]) >> (j % 32)) & 1
            nbit = (int(cneg[j // 32]) >> (j % 32)) & 1
            if pj != 0:
                assert bit != nbit


def test_code_matches_exact_rational_sign():
    """Brute force: the fp64 index-order sign equals the exact sign."""
    rng = np.random.default_rng(4)
    b = 64
    P = rand_bits(rng, (D, b))
    for t in range(12):
        k = rand_bits(rng, D, scale=[1.0, 8.0, 0.01][t % 3])
        assert np.array_equal(oracle.key_code(k, P), exact_sign_code(k, P))


@pytest.mark.parametrize("b", [64, 128, 256])
def test_encode_keys_equals_each_row_and_exact_values(b):
    """The batched encoder (every parity test and the CPU baseline use it)
    returns, row by row, the single-key code and radius, at an odd row
    count; spot rows also match the exact-rational sign code and exact
    radius threshold, so a row or word stride mistake cannot pass."""
    rng = np.random.default_rng(40 + b)
    n = 37
    P = rand_bits(rng, (D, b))
    scales = np.array([[1.0], [8.0], [0.01], [300.0]], np.float32)
    K = bf16_bits(rng.standard_normal((n, D)).astype(np.float32) * scales[np.arange(n) % 4])
    K[5] = 0                                       # a zero row: code 0, radius 0
    codes, radii = oracle.encode_keys(K, P)
    assert codes.shape == (n, b // 32) and radii.shape == (n,)
    for t in range(n):
        assert np.array_equal(codes[t], oracle.key_code(K[t], P)), t
        assert radii[t] == oracle.radius_code(oracle.sq_norm(K[t])), t
    assert not codes[5].any() and radii[5] == 0
    for t in (0, 1, 18, n - 2, n - 1):
        assert np.array_equal(codes[t], exact_sign_code(K[t], P)), t
        r2 = sum((bf16_fraction(x) ** 2 for x in K[t]), Fraction(0))
        assert int(radii[t]) == exact_radius_code(r2), t


def test_code_zero_projection_is_clear_bit():
    b = 32 * 2
    P = np.zeros((D, b), np.float32)
    P[0, :] = 1.0
    P[1, :] = -1.0
    k = np.zeros(D, np.float32)
    k[0] = k[1] = 1.5          # projection exactly 0 on every column
    assert not oracle.key_code(bf16_bits(k), bf16_bits(P)).any()


def test_code_simhash_collision_rate():
    """Fraction of differing bits ~ angle/pi (random hyperplane identity)."""
    rng = np.random.default_rng(5)
    b = 256
    P = rand_bits(rng, (D, b))
    diffs, expected = 0, 0.0
    n_pairs = 40
    for _ in range(n_pairs):
        x = rng.standard_normal(D)
        y = 0.7 * x + 0.7 * rng.standard_normal(D)
        xb, yb = bf16_bits(x), bf16_bits(y)
        xf, yf = bits_to_float(xb), bits_to_float(yb)
        theta = math.acos(np.dot(xf, yf) / np.linalg.norm(xf) / np.linalg.norm(yf))
        expected += theta / math.pi * b
        cx, cy = oracle.key_code(xb, P), oracle.key_code(yb, P)
        diffs += sum(bin(int(a) ^ int(c)).count("1") for a, c in zip(cx, cy))
    # P is one fixed draw shared by all pairs; allow a wide band.
    assert abs(diffs - expected) < 0.1 * expected


# ---------------------------------------------------------------- E2 radius
def test_radius_constants_are_nearest_doubles():
    """C[f] is the double nearest 2^(f/8): checked in exact rationals."""
    for f in range(8):
        c = oracle.radius_threshold(64 + f)
        lo, hi = np.nextafter(c, 0.0), np.nextafter(c, 10.0)
        mid_lo = (Fraction(lo) + Fraction(c)) / 2
        mid_hi = (Fraction(c) + Fraction(hi)) / 2
        assert mid_lo ** 8 <= 2 ** f <= mid_hi ** 8


def test_radius_closed_form_powers_of_two():
    """|k|^2 = 4^e  =>  r8 = 64 + 16e (clamped to 0..255)."""
    for e in range(-3, 12):
        k = np.zeros(D, np.float32)
        k[3] = 2.0 ** e
        r2 = oracle.sq_norm(bf16_bits(k))
        assert r2 == 4.0 ** e
        assert oracle.radius_code(r2) == min(255, max(0, 64 + 16 * e))
    assert oracle.radius_code(0.0) == 0
    assert oracle.radius_code(1e300) == 255
    assert oracle.radius_code(2.0 ** -20) == 0


def test_radius_doubling_adds_sixteen_and_is_monotone():
    rng = np.random.default_rng(6)
    prev_r2, prev_m = -1.0, -1
    r2s = sorted(float(np.sum(bits_to_float(rand_bits(rng, D, s)) ** 2))
                 for s in np.geomspace(0.05, 50, 40))
    for r2 in r2s:
        m = oracle.radius_code(r2)
        assert m >= prev_m
        prev_m = m
        m2 = oracle.radius_code(4.0 * r2)
        assert m2 == min(255, m + 16) or m == 0


def test_radius_matches_exact_log_threshold():
    """Brute force: exact comparison r^2 >= 2^((m-64)/8) on random keys."""
    rng = np.random.default_rng(7)
    for s in np.geomspace(0.02, 300, 25):
        k = rand_bits(rng, D, s)
        r2 = oracle.sq_norm(k)
        assert r2 == float(sum(bf16_fraction(x) ** 2 for x in k))  # squares exact
        assert oracle.radius_code(r2) == exact_radius_code(Fraction(r2))


# ---------------------------------------------------------------- Q1 int8
@pytest.mark.parametrize("G", [1, 4])
def test_query_int8_textbook_properties(G):
    rng = np.random.default_rng(8 + G)
    b = 128
    P = rand_bits(rng, (D, b))
    q = rand_bits(rng, (G, D))
    q8 = oracle.query_int8(q, P)
    assert q8.dtype == np.int8
    assert np.abs(q8.astype(int)).max() == 127
    # signs preserved where nonzero
    for h in range(G):
        for j in range(0, b, 7):
            p = exact_projection(q[h], P, j)
            if q8[h, j] != 0:
                assert (q8[h, j] > 0) == (p > 0)
    # scaling the whole group by 2^e changes nothing
    qs = bf16_bits(bits_to_float(q) * 4.0)
    assert np.array_equal(oracle.query_int8(qs, P), q8)
    # zero query -> zero code
    assert not oracle.query_int8(np.zeros((G, D), np.uint16), P).any()


def test_query_int8_matches_exact_rounding():
    """Exact-rational round_half_even(p*127/M) agrees with the fp64 oracle."""
    rng = np.random.default_rng(9)
    b = 64
    P = rand_bits(rng, (32, b))
    q = rand_bits(rng, (2, 32))
    got = oracle.query_int8(q, P).astype(int)
    want = exact_query_int8(q, P)
    assert np.array_equal(got, want)


def test_query_int8_shares_scale_across_group():
    """Head 1 = head 0 / 2 exactly  =>  |q8_1| ~ |q8_0| / 2 (one group scale)."""
    rng = np.random.default_rng(10)
    b = 128
    P = rand_bits(rng, (D, b))
    q0 = bits_to_float(rand_bits(rng, D))
    q = bf16_bits(np.stack([q0, q0 / 2]))
    q8 = oracle.query_int8(q, P).astype(int)
    assert np.abs(q8[0]).max() == 127
    assert np.all(np.abs(q8[1] - q8[0] / 2) <= 0.5 + 1e-9)
    # per-head scaling would have made head 1 reach 127 too
    assert np.abs(q8[1]).max() <= 64


# ---------------------------------------------------------------- S1 scores
@pytest.mark.parametrize("G,b", [(1, 64), (4, 128), (2, 256)])
def test_score_matches_integer_brute_force(G, b):
    rng = np.random.default_rng(11 + b)
    for _ in range(30):
        q8 = rng.integers(-127, 128, size=(G, b)).astype(np.int8)
        code = rng.integers(0, 2 ** 32, size=b // 32, dtype=np.uint64).astype(np.uint32)
        r8 = int(rng.integers(0, 256))
        assert oracle.score(q8, code, r8) == brute_score(q8, code, r8)


def test_score_identities():
    rng = np.random.default_rng(12)
    b = 128
    q8 = rng.integers(-127, 128, size=(1, b)).astype(np.int8)
    qs = int(q8.astype(int).sum())
    ones = np.full(b // 32, 0xFFFFFFFF, np.uint32)
    zeros = np.zeros(b // 32, np.uint32)
    assert oracle.score(q8, ones, 1) == qs
    assert oracle.score(q8, zeros, 1) == -qs
    for _ in range(10):
        code = rng.integers(0, 2 ** 32, size=b // 32, dtype=np.uint64).astype(np.uint32)
        s = oracle.score(q8, code, 1)
        assert oracle.score(q8, ~code, 1) == -s
        set_sum = sum(int(q8[0, j]) for j in range(b) if (int(code[j // 32]) >> (j % 32)) & 1)
        assert s == 2 * set_sum - qs
        assert oracle.score(q8, code, 0) == 0
        assert oracle.score(q8, code, 200) == 200 * s
    # constant q8 = c: s = c * (2*popcount - b) (Hamming form)
    c = np.full((1, b), 3, np.int8)
    code = rng.integers(0, 2 ** 32, size=b // 32, dtype=np.uint64).astype(np.uint32)
    pop = sum(bin(int(x)).count("1") for x in code)
    assert oracle.score(c, code, 1) == 3 * (2 * pop - b)


def test_score_takes_group_maximum():
    b = 64
    q8 = np.zeros((4, b), np.int8)
    q8[2, :] = 5
    q8[0, :] = -5
    ones = np.full(b // 32, 0xFFFFFFFF, np.uint32)
    assert oracle.score(q8, ones, 2) == 2 * 5 * b       # head 2 wins
    assert oracle.score(q8, ~ones, 2) == 2 * 5 * b      # head 0 wins


# ---------------------------------------------------------- W1 radius weight
def _rne_pow2_sixteenth(r: int) -> int:
    """rne(2^(r/16)) from 60-digit decimal arithmetic (not libm)."""
    from decimal import ROUND_HALF_EVEN, Decimal, getcontext
    getcontext().prec = 60
    v = Decimal(2) ** (Decimal(r) / Decimal(16))
    return int(v.to_integral_value(rounding=ROUND_HALF_EVEN))


def test_radius_weight_log_mode_is_the_code():
    for r in range(256):
        assert oracle.radius_weight(r, 0) == r


def test_radius_weight_linear_matches_high_precision():
    """mode 1: w = rne(2^(r8/16)), checked against decimal arithmetic."""
    for r in range(256):
        assert oracle.radius_weight(r, 1) == _rne_pow2_sixteenth(r), r


def test_radius_weight_linear_closed_forms():
    w = [oracle.radius_weight(r, 1) for r in range(256)]
    # exact powers of two where 16 divides r8 (the code's zero point 64
    # stands for |k| = 1, weight 2^4)
    for m in range(16):
        assert w[16 * m] == 2 ** m
    assert w[64] == 16
    # linear in the radius: one octave of radius (16 codes) doubles the
    # weight up to the rounding of each side
    for r in range(240):
        assert abs(w[r + 16] - 2 * w[r]) <= 1
    assert all(a <= b for a, b in zip(w, w[1:]))
    # the largest score magnitude fits a signed 32-bit integer
    assert w[255] * 127 * 256 < 2 ** 31
    assert w[255] == 62757


def test_score_with_linear_weight_matches_brute_force():
    rng = np.random.default_rng(13)
    for G, b in [(1, 64), (4, 128), (8, 256)]:
        for _ in range(20):
            q8 = rng.integers(-127, 128, size=(G, b)).astype(np.int8)
            code = rng.integers(0, 2 ** 32, size=b // 32, dtype=np.uint64).astype(np.uint32)
            r8 = int(rng.integers(0, 256))
            wgt = _rne_pow2_sixteenth(r8)
            assert oracle.score(q8, code, oracle.radius_weight(r8, 1)) == \
                wgt * brute_score(q8, code, 1)
    # extreme magnitude: all q8 = 127, all bits set, b = 256, r8 = 255
    q8 = np.full((1, 256), 127, np.int8)
    ones = np.full(8, 0xFFFFFFFF, np.uint32)
    assert oracle.score(q8, ones, oracle.radius_weight(255, 1)) == 62757 * 127 * 256
    assert oracle.score(q8, ~ones, oracle.radius_weight(255, 1)) == -62757 * 127 * 256


# ---------------------------------------------------------------- T1 select
@pytest.mark.parametrize("N,k,w,sigma", [
    (500, 40, 16, 4), (1000, 64, 64, 4), (90, 10, 50, 4), (60, 10, 50, 4),
    (30, 10, 50, 4), (3, 2, 1, 4), (1, 5, 5, 4), (200, 500, 16, 4),
    (200, 0, 16, 4), (200, 10, 0, 0), (64, 8, 8, 60)])
def test_select_matches_brute_force(N, k, w, sigma):
    rng = np.random.default_rng(N + k)
    S = rng.integers(-50, 50, size=N).astype(np.int32)   # many ties
    got = oracle.select(S, k, w, sigma)
    sinks, window, top = brute_select(S, k, w, sigma)
    assert list(got) == sinks + window + top
    assert len(got) == min(N, sigma + w + k)
    assert len(set(got.tolist())) == len(got)


def test_select_all_equal_scores_take_lowest_positions():
    S = np.full(1000, 7, np.int32)
    got = oracle.select(S, 32, 16, 4)
    assert list(got[4 + 16:]) == list(range(4, 36))


def test_select_picks_largest_scores():
    N = 400
    S = np.zeros(N, np.int32)
    hot = [17, 99, 250, 301]
    S[hot] = [5, 9, 7, 9]
    got = oracle.select(S, 4, 10, 4)
    assert list(got[14:]) == [99, 301, 250, 17]   # score desc, then position


# ---------------------------------------------------------- T2 select pages
@pytest.mark.parametrize("N,k,w,sigma", [
    (500, 48, 16, 4), (1000, 64, 64, 5), (90, 16, 50, 4), (60, 16, 50, 4),
    (30, 16, 50, 4), (3, 16, 1, 4), (200, 500, 16, 4), (200, 15, 16, 4),
    (200, 0, 16, 4), (200, 40, 0, 0), (64, 16, 8, 60), (333, 37, 21, 19)])
def test_select_pages_matches_brute_force(N, k, w, sigma):
    rng = np.random.default_rng(N + 3 * k)
    S = rng.integers(-50, 50, size=N).astype(np.int32)   # many page ties
    got = oracle.select_pages(S, k, w, sigma)
    sinks, window, top = brute_select_pages(S, k, w, sigma)
    assert list(got) == sinks + window + top
    assert len(got) <= min(N, sigma + w + k)
    assert len(set(got.tolist())) == len(got)


@pytest.mark.parametrize("seed", range(4))
def test_select_pages_equals_select_on_page_constant_scores(seed):
    """Scores constant on each page, sigma, N - w and k multiples of 16:
    the token top-k takes whole pages in (score desc, page asc) order, so
    both selections are the same set (T1 is pinned independently)."""
    rng = np.random.default_rng(seed)
    npg = 64
    S = np.repeat(rng.integers(-20, 20, size=npg), 16).astype(np.int32)
    for k, w, sigma in [(160, 32, 16), (16, 0, 0), (480, 64, 48)]:
        pages = oracle.select_pages(S, k, w, sigma)
        tokens = oracle.select(S, k, w, sigma)
        assert sorted(pages.tolist()) == sorted(tokens.tolist())


def test_select_pages_limits():
    S = np.arange(1000, dtype=np.int32)
    # k below one page: sinks and window only
    assert list(oracle.select_pages(S, 15, 10, 4)) == list(range(4)) + list(range(990, 1000))
    # enough pages for the whole candidate range: dense
    assert sorted(oracle.select_pages(S, 1000, 10, 4).tolist()) == list(range(1000))
    # partial edge pages: the sinks' page and the window's page give only
    # their keys inside [sigma, N - w)
    got = oracle.select_pages(S, 2 * 16, 10, 4)[4 + 10:]
    assert list(got) == list(range(976, 990)) + list(range(960, 976))
    # a page's score is its best key: one hot key lifts its whole page
    S2 = np.zeros(1000, np.int32)
    S2[517] = 3
    got = oracle.select_pages(S2, 16, 10, 4)[14:]
    assert list(got) == list(range(512, 528))
    # equal page scores: the lowest page wins
    got = oracle.select_pages(np.zeros(1000, np.int32), 16, 10, 4)[14:]
    assert list(got) == list(range(4, 16))


# ------------------------------------------------------- H1/T3 LSH buckets
def test_lsh_bucket_matches_bit_extraction():
    rng = np.random.default_rng(21)
    for W in (2, 4, 8):
        for _ in range(20):
            code = rng.integers(0, 2 ** 32, size=W, dtype=np.uint64).astype(np.uint32)
            for m in (1, 3, 8, 12):
                for t in range(min(4, 32 * W // m)):
                    assert oracle.lsh_bucket(code, t, m) == brute_lsh_bucket(code, t, m)


@pytest.mark.parametrize("T,m,G", [(4, 3, 1), (6, 4, 4), (2, 8, 2), (10, 12, 4)])
def test_select_lsh_matches_brute_force(T, m, G):
    rng = np.random.default_rng(T * 100 + m)
    W = 4
    N, k, w, sigma = 700, 40, 30, 5
    S = rng.integers(-30, 30, size=N).astype(np.int32)
    codes = rng.integers(0, 2 ** 32, size=(N, W), dtype=np.uint64).astype(np.uint32)
    qbits = rng.integers(0, 2 ** 32, size=(G, W), dtype=np.uint64).astype(np.uint32)
    got = oracle.select_lsh(S, codes, qbits, T, m, k, w, sigma)
    sinks, window, top = brute_select_lsh(S, codes, qbits, T, m, k, w, sigma)
    assert list(got) == sinks + window + top


def test_select_lsh_all_candidates_equals_select():
    """Every key shares table 0's bucket with the query: the candidates are
    the whole range and T3 is T1."""
    rng = np.random.default_rng(22)
    N, W = 500, 4
    S = rng.integers(-20, 20, size=N).astype(np.int32)
    codes = rng.integers(0, 2 ** 32, size=(N, W), dtype=np.uint64).astype(np.uint32)
    qbits = rng.integers(0, 2 ** 32, size=(1, W), dtype=np.uint64).astype(np.uint32)
    codes[:, 0] = (codes[:, 0] & ~np.uint32(0xFF)) | (qbits[0, 0] & np.uint32(0xFF))
    for k in (0, 17, 300, 1000):
        assert list(oracle.select_lsh(S, codes, qbits, 3, 8, k, 20, 4)) == \
            list(oracle.select(S, k, 20, 4))


def test_select_lsh_no_candidates():
    N, W = 300, 4
    S = np.arange(N, dtype=np.int32)
    codes = np.zeros((N, W), np.uint32)
    qbits = np.full((2, W), 0xFFFFFFFF, np.uint32)
    got = oracle.select_lsh(S, codes, qbits, 5, 6, 64, 10, 4)
    assert list(got) == list(range(4)) + list(range(290, 300))


# ---------------------------------------------------------------- A1 attend
def _sdpa_fp64(qf, Kf, Vf):
    q = torch.from_numpy(qf)[None, :, None, :]          # [1, G, 1, d]
    k = torch.from_numpy(Kf)[None, None].expand(1, qf.shape[0], -1, -1)
    v = torch.from_numpy(Vf)[None, None].expand(1, qf.shape[0], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(q, k, v)[0, :, 0].numpy()


def test_attend_dense_case_equals_sdpa():
    """k + w + sigma >= N selects everything: the result is dense attention."""
    rng = np.random.default_rng(13)
    G, N = 4, 300
    q, K, V = rand_bits(rng, (G, D)), rand_bits(rng, (N, D), 3.0), rand_bits(rng, (N, D))
    sel = oracle.select(rng.integers(-9, 9, N).astype(np.int32), 500, 32, 4)
    assert sorted(sel.tolist()) == list(range(N))
    got = oracle.attend(q, K, V, sel)
    want = _sdpa_fp64(bits_to_float(q), bits_to_float(K), bits_to_float(V))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attend_single_key_and_identical_keys():
    rng = np.random.default_rng(14)
    q, K, V = rand_bits(rng, (2, D)), rand_bits(rng, (50, D)), rand_bits(rng, (50, D))
    got = oracle.attend(q, K, V, np.array([17], np.int32))
    np.testing.assert_array_equal(got, np.stack([bits_to_float(V[17])] * 2))
    K2 = np.repeat(K[:1], 50, axis=0)
    sel = np.array([3, 9, 20, 41], np.int32)
    got = oracle.attend(q, K2, V, sel)
    want = bits_to_float(V[sel]).mean(axis=0)
    np.testing.assert_allclose(got, np.stack([want] * 2), rtol=1e-13, atol=1e-13)


def test_attend_uses_one_over_sqrt_d_scale():
    """Two keys with logits differing by a known amount: closed-form weight."""
    q = np.zeros((1, D), np.float32)
    q[0, 0] = 1.0
    K = np.zeros((2, D), np.float32)
    K[0, 0] = 4.0
    V = np.zeros((2, D), np.float32)
    V[0, 1] = 1.0
    V[1, 2] = 1.0
    out = oracle.attend(bf16_bits(q), bf16_bits(K), bf16_bits(V), np.array([0, 1], np.int32))
    a0 = 1.0 / (1.0 + math.exp(-4.0 / math.sqrt(D)))
    assert abs(out[0, 1] - a0) < 1e-15 and abs(out[0, 2] - (1 - a0)) < 1e-15
