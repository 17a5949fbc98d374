"""Method-level checks of the oracle pipeline on the seeded workloads (CPU).

* every planted needle key is selected (recall 1.0) -- the needle-in-a-
  haystack idea at several depths and several needles;
* with k + w + sigma >= N the pipeline reduces to dense softmax attention
  (checked against torch SDPA in fp64);
* the composition decode_unit == query_int8 -> score -> select -> attend.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import bits_to_float, logical_rows, tensor_bits


def _units(name):
    wl = workloads.get(name)
    inp = workloads.make_inputs(wl, "cpu")
    bt = inp["block_table"].numpy()
    lens = inp["seq_lens"].numpy()
    P = tensor_bits(inp["proj"])
    q = tensor_bits(inp["q"])
    G = wl.group
    for s in range(wl.batch):
        for g in range(wl.num_kv_heads):
            N = int(lens[s])
            K = logical_rows(inp["k_pool"], bt, s, N, g)
            V = logical_rows(inp["v_pool"], bt, s, N, g)
            yield wl, s, g, q[s, g * G:(g + 1) * G], P, K, V, inp["needles"][s][g]


@pytest.mark.parametrize("name", ["mha1_n4k_b64", "gqa32x8_bs1_n32k_b128",
                                  "small_mha_b64", "small_gqa_b128",
                                  "small_gqa_b256_lognormal", "small_ragged_b128"])
def test_needle_recall_is_one(name):
    n_checked = 0
    for wl, s, g, q, P, K, V, nd in _units(name):
        codes, radii = oracle.encode_keys(K, P)
        r = oracle.decode_unit(q, P, codes, radii, K, V, wl.top_k, wl.window, wl.sinks)
        assert len(r["sel"]) == min(K.shape[0], wl.sinks + wl.window + wl.top_k)
        if len(nd):
            assert np.isin(nd, r["sel"]).all(), (s, g)
            n_checked += len(nd)
    assert n_checked > 0


def test_pipeline_dense_limit_equals_sdpa():
    wl = workloads.get("small_gqa_b128")
    for _, s, g, q, P, K, V, _ in _units("small_gqa_b128"):
        N = K.shape[0]
        codes, radii = oracle.encode_keys(K, P)
        r = oracle.decode_unit(q, P, codes, radii, K, V, N, 16, 4)
        assert sorted(r["sel"].tolist()) == list(range(N))
        qf = torch.from_numpy(bits_to_float(q))[None, :, None, :]
        Kf = torch.from_numpy(bits_to_float(K))[None, None].expand(1, q.shape[0], -1, -1)
        Vf = torch.from_numpy(bits_to_float(V))[None, None].expand(1, q.shape[0], -1, -1)
        want = torch.nn.functional.scaled_dot_product_attention(qf, Kf, Vf)[0, :, 0].numpy()
        np.testing.assert_allclose(r["out"], want, rtol=1e-11, atol=1e-12)
        break


def test_decode_unit_lsh_is_the_composition():
    """With LSH tables: query bits are the E1 code of each query row, the
    selection is T3 over the scores."""
    for wl, s, g, q, P, K, V, _ in _units("small_gqa_b128"):
        codes, radii = oracle.encode_keys(K, P)
        for lsh in [(8, 6), (4, 10)]:
            r = oracle.decode_unit(q, P, codes, radii, K, V, wl.top_k, wl.window, wl.sinks,
                                   radius_mode=1, lsh=lsh)
            qbits = np.stack([oracle.key_code(q[h], P) for h in range(q.shape[0])])
            S = oracle.scores(oracle.query_int8(q, P), codes, radii, radius_mode=1)
            sel = oracle.select_lsh(S, codes, qbits, lsh[0], lsh[1], wl.top_k, wl.window,
                                    wl.sinks)
            assert np.array_equal(r["scores"], S)
            assert np.array_equal(r["sel"], sel)
            assert np.array_equal(r["out"], oracle.attend(q, K, V, sel))
        if s >= 1:
            break


@pytest.mark.parametrize("mode,pages", [(0, False), (1, False), (0, True), (1, True)])
def test_decode_unit_is_the_composition(mode, pages):
    for wl, s, g, q, P, K, V, _ in _units("small_ragged_b128"):
        codes, radii = oracle.encode_keys(K, P)
        r = oracle.decode_unit(q, P, codes, radii, K, V, wl.top_k, wl.window, wl.sinks,
                               radius_mode=mode, pages=pages)
        q8 = oracle.query_int8(q, P)
        S = oracle.scores(q8, codes, radii, radius_mode=mode)
        pick = oracle.select_pages if pages else oracle.select
        sel = pick(S, wl.top_k, wl.window, wl.sinks)
        out = oracle.attend(q, K, V, sel)
        assert np.array_equal(r["q8"], q8)
        assert np.array_equal(r["scores"], S)
        assert np.array_equal(r["sel"], sel)
        assert np.array_equal(r["out"], out)
        if s >= 1:
            break


@pytest.mark.parametrize("mode,pages", [(0, False), (1, False), (0, True)])
def test_decode_units_batch_equals_single_units(mode, pages):
    units = list(_units("small_gqa_b128"))[:3]
    wl = units[0][0]
    Nmax = max(u[5].shape[0] for u in units)
    U, G, d = len(units), units[0][3].shape[0], 128
    b = wl.code_bits
    q = np.stack([u[3] for u in units])
    P = units[0][4]
    K = np.zeros((U, Nmax, d), np.uint16)
    V = np.zeros((U, Nmax, d), np.uint16)
    codes = np.zeros((U, Nmax, b // 32), np.uint32)
    radii = np.zeros((U, Nmax), np.uint8)
    N = np.zeros(U, np.int32)
    for i, u in enumerate(units):
        n = u[5].shape[0]
        K[i, :n], V[i, :n], N[i] = u[5], u[6], n
        codes[i, :n], radii[i, :n] = oracle.encode_keys(u[5], P)
    r = oracle.decode_units(q, P, codes, radii, K, V, N, wl.top_k, wl.window, wl.sinks,
                            radius_mode=mode, pages=pages)
    for i, u in enumerate(units):
        n = N[i]
        one = oracle.decode_unit(q[i], P, codes[i, :n], radii[i, :n], K[i, :n], V[i, :n],
                                 wl.top_k, wl.window, wl.sinks, radius_mode=mode,
                                 pages=pages)
        assert np.array_equal(r["sel"][i], one["sel"])
        assert np.array_equal(r["out"][i], one["out"])
        assert np.array_equal(r["scores"][i, :n], one["scores"])
