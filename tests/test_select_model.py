"""CPU model of the workgroup k-th-largest search (the bin arithmetic of
wg_kth_largest in hashed_top_sparse_amd/csrc/select_common.h).

The device search histograms (v - vmin) >> shift over 4096 bins, shift
chosen so the value range fits, then refines inside the bin found, at most
12 bits per pass, until the bins are single values.  This model repeats that
bin arithmetic with numpy (same shifts, masks, prefixes and counts) and
checks it against a full sort, for value ranges from a few values up to all
32 bits: biased scores u = S + 2^31 under the linear radius weight span up
to about 2^32.  It checks the algorithm, not the device code; the GPU tests
reach the device code with wide ranges.
"""
import numpy as np
import pytest

HIST_BITS = 12


def find_bin(hist, kneed):
    """Scanning from the top bin: the bin where the running count reaches
    kneed, and the count of the bins above it."""
    above = 0
    for b in range(len(hist) - 1, -1, -1):
        if above + hist[b] >= kneed:
            return b, above
        above += hist[b]
    raise AssertionError("kneed exceeds the element count")


def kth_largest_model(v, kneed):
    v = np.asarray(v, np.uint64)
    vmin, vmax = int(v.min()), int(v.max())
    rng = vmax - vmin
    bits = rng.bit_length()
    shift = bits - HIST_BITS if bits > HIST_BITS else 0
    d = v - np.uint64(vmin)
    hist = np.bincount((d >> np.uint64(shift)).astype(np.int64), minlength=1 << HIST_BITS)
    assert len(hist) == 1 << HIST_BITS   # every first-pass bin index fits
    b, above = find_bin(hist, kneed)
    prefix, kleft, n_eq = b, kneed - above, int(hist[b])
    passes = 1
    while shift > 0:
        nxt = shift - HIST_BITS if shift > HIST_BITS else 0
        width = shift - nxt
        inbin = d[(d >> np.uint64(shift)) == np.uint64(prefix)]
        idx = ((inbin >> np.uint64(nxt)) & np.uint64((1 << width) - 1)).astype(np.int64)
        assert idx.max() < 1 << HIST_BITS
        hist = np.bincount(idx, minlength=1 << HIST_BITS)
        b, above = find_bin(hist, kleft)
        prefix = (prefix << width) | b
        kleft -= above
        n_eq = int(hist[b])
        shift = nxt
        passes += 1
    return vmin + prefix, kleft, n_eq, passes


def reference(v, kneed):
    s = np.sort(np.asarray(v, np.uint64))[::-1]
    T = int(s[kneed - 1])
    n_gt = int((s > T).sum())
    return T, kneed - n_gt, int((s == T).sum())


@pytest.mark.parametrize("bits", [0, 3, 12, 13, 20, 24, 25, 28, 31, 32])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_model_matches_sort(bits, seed):
    rng = np.random.default_rng(1000 * bits + seed)
    n = 3000
    lo = int(rng.integers(0, (1 << 32) - (1 << bits) + 1))
    v = lo + rng.integers(0, 1 << bits, size=n, dtype=np.uint64) if bits else np.full(n, lo)
    v = np.asarray(v, np.uint64)
    # repeated values: ties at the k-th element
    v[rng.integers(0, n, 200)] = v[rng.integers(0, n)]
    for kneed in (1, 2, 17, n // 3, n // 2, n - 1, n):
        T, take, n_eq, passes = kth_largest_model(v, kneed)
        assert (T, take, n_eq) == reference(v, kneed), (bits, kneed)
        assert 1 <= take <= n_eq
        assert passes == 1 + max(0, (max(0, bits - HIST_BITS) + HIST_BITS - 1) // HIST_BITS) \
            or bits == 0


def test_full_32_bit_range_takes_three_passes():
    v = np.array([0, 1, 2, (1 << 31) + 5, (1 << 32) - 1, (1 << 32) - 2], np.uint64)
    for kneed in range(1, len(v) + 1):
        T, take, n_eq, passes = kth_largest_model(v, kneed)
        assert (T, take, n_eq) == reference(v, kneed)
        assert passes == 3


def test_scores_of_the_linear_weight_span_more_than_24_bits():
    """Scores w * max_h s_h with the linear weight (w up to 62757) and b = 256
    (|s| up to 127 * 256), biased by 2^31: the range the device search must
    handle exceeds a two-pass 24-bit search."""
    w_max, s_max = 62757, 127 * 256
    lo = (-w_max * s_max) + (1 << 31)
    hi = (w_max * s_max) + (1 << 31)
    assert 0 <= lo and hi < 1 << 32
    assert (hi - lo).bit_length() > 24
    rng = np.random.default_rng(7)
    v = rng.integers(lo, hi + 1, size=5000, dtype=np.uint64)
    for kneed in (1, 100, 2500, 5000):
        T, take, n_eq, _ = kth_largest_model(v, kneed)
        assert (T, take, n_eq) == reference(v, kneed)
