"""GPU-vs-oracle parity driver shared by the GPU tests and the smoke check.

Inputs come from ``workloads`` (drawn on the GPU); the GPU path runs through
the C ABI (``hashed_top_sparse_amd``); the oracle gets host copies of the
very same input bytes for the (sequence, KV head) units under test and
computes its own codes, radii, query codes, scores, selection and output.
Nothing the GPU computed is ever fed to the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import hashed_top_sparse_amd as dkv
import oracle
import workloads
from helpers import (PAGE, logical_codes, logical_radii, logical_rows,
                     tensor_bits)

ATOL, RTOL = 2e-3, 1e-2


def config_of(wl: workloads.Workload, **over) -> dkv.Config:
    kw = dict(num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
              code_bits=wl.code_bits, top_k=wl.top_k, window=wl.window,
              sinks=wl.sinks)
    kw.update(over)
    return dkv.Config(**kw)


def gpu_encode_all(cfg: dkv.Config, inp: dict):
    """Encode every cached token of every sequence with dkv_encode."""
    dev = inp["k_pool"].device
    nb = inp["k_pool"].shape[0]
    codes = torch.zeros((nb, cfg.num_kv_heads, PAGE, cfg.code_bits // 32),
                        dtype=torch.int32, device=dev)
    radii = torch.zeros((nb, cfg.num_kv_heads, PAGE), dtype=torch.uint8, device=dev)
    B = inp["block_table"].shape[0]
    start = torch.zeros(B, dtype=torch.int32, device=dev)
    dkv.encode(cfg, inp["k_pool"], inp["block_table"], start, inp["seq_lens"],
               inp["max_seq_len"], inp["proj"], codes, radii)
    return codes, radii


def gpu_decode(cfg: dkv.Config, inp: dict, codes, radii, debug: bool = True,
               seq_lens=None, max_seq_len=None):
    dev = inp["k_pool"].device
    B = inp["block_table"].shape[0]
    seq_lens = inp["seq_lens"] if seq_lens is None else seq_lens
    max_seq_len = inp["max_seq_len"] if max_seq_len is None else max_seq_len
    ws = torch.empty(dkv.decode_workspace_size(cfg, B, max_seq_len),
                     dtype=torch.uint8, device=dev)
    out = torch.full((B, cfg.num_q_heads, cfg.head_dim), float("nan"), device=dev)
    sel = torch.full((B, cfg.num_kv_heads, cfg.select_cap), -7, dtype=torch.int32,
                     device=dev)
    cnt = torch.full((B, cfg.num_kv_heads), -7, dtype=torch.int32, device=dev)
    res = {"out": out, "sel": sel, "cnt": cnt}
    if debug:
        q8 = torch.zeros((B, cfg.num_q_heads, cfg.code_bits), dtype=torch.int8, device=dev)
        sc = torch.zeros((B, cfg.num_kv_heads, max(1, max_seq_len)), dtype=torch.int32,
                         device=dev)
        if max_seq_len == 0:
            sc = None
        dkv.decode_debug(cfg, inp["q"], inp["k_pool"], inp["v_pool"], codes, radii,
                         inp["block_table"], seq_lens, max_seq_len, inp["proj"], out,
                         ws, sel, cnt, q8, sc)
        res.update(q8=q8, scores=sc)
    else:
        dkv.decode(cfg, inp["q"], inp["k_pool"], inp["v_pool"], codes, radii,
                   inp["block_table"], seq_lens, max_seq_len, inp["proj"], out, ws,
                   sel, cnt)
    torch.cuda.synchronize()
    return res


def gpu_decode_lsh(cfg: dkv.Config, inp: dict, codes, radii, index_lens=None):
    """dkv_lsh_build over [0, index_lens) (default: every cached token), then
    dkv_decode_lsh over the full lengths."""
    dev = inp["k_pool"].device
    B = inp["block_table"].shape[0]
    T = inp["max_seq_len"]
    index = torch.empty(dkv.lsh_index_size(cfg, B, T), dtype=torch.uint8, device=dev)
    lens = inp["seq_lens"] if index_lens is None else index_lens
    dkv.lsh_build(cfg, codes, inp["block_table"], lens, T, index)
    ws = torch.empty(dkv.decode_workspace_size(cfg, B, T), dtype=torch.uint8, device=dev)
    out = torch.full((B, cfg.num_q_heads, cfg.head_dim), float("nan"), device=dev)
    sel = torch.full((B, cfg.num_kv_heads, cfg.select_cap), -7, dtype=torch.int32,
                     device=dev)
    cnt = torch.full((B, cfg.num_kv_heads), -7, dtype=torch.int32, device=dev)
    dkv.decode_lsh(cfg, inp["q"], inp["k_pool"], inp["v_pool"], codes, radii,
                   inp["block_table"], inp["seq_lens"], T, inp["proj"], index, out, ws,
                   sel, cnt)
    torch.cuda.synchronize()
    return {"out": out, "sel": sel, "cnt": cnt}


def gpu_decode_append(cfg: dkv.Config, inp: dict):
    """dkv_encode over [0, N-1) of every sequence into sentinel-filled pools,
    then dkv_decode_append (which must encode position N-1 itself).  Returns
    (result dict, codes, radii)."""
    dev = inp["k_pool"].device
    nb = inp["k_pool"].shape[0]
    Hkv, B = cfg.num_kv_heads, inp["block_table"].shape[0]
    codes = torch.full((nb, Hkv, PAGE, cfg.code_bits // 32), 0x5A5A5A5A,
                       dtype=torch.int32, device=dev)
    radii = torch.full((nb, Hkv, PAGE), 0xA5, dtype=torch.uint8, device=dev)
    start = torch.zeros(B, dtype=torch.int32, device=dev)
    end = torch.clamp(inp["seq_lens"] - 1, min=0).to(torch.int32)
    dkv.encode(cfg, inp["k_pool"], inp["block_table"], start, end,
               inp["max_seq_len"], inp["proj"], codes, radii)
    ws = torch.empty(dkv.decode_workspace_size(cfg, B, inp["max_seq_len"]),
                     dtype=torch.uint8, device=dev)
    out = torch.full((B, cfg.num_q_heads, cfg.head_dim), float("nan"), device=dev)
    sel = torch.full((B, Hkv, cfg.select_cap), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device=dev)
    dkv.decode_append(cfg, inp["q"], inp["k_pool"], inp["v_pool"], codes, radii,
                      inp["block_table"], inp["seq_lens"], inp["max_seq_len"],
                      inp["proj"], out, ws, sel, cnt)
    torch.cuda.synchronize()
    return {"out": out, "sel": sel, "cnt": cnt}, codes, radii


def check_unit(cfg: dkv.Config, inp: dict, gpu: dict, codes, radii, s: int, g: int,
               check_codes: bool = True, needles=None, code_pool=None) -> dict:
    """Compares one (sequence s, KV head g) unit with the oracle.  code_pool:
    the key pool the codes were built from, when it is not the attended one."""
    bt = inp["block_table"].cpu().numpy()
    N = int(inp["seq_lens"][s].item())
    G = cfg.group
    P = tensor_bits(inp["proj"])
    q = tensor_bits(inp["q"][s, g * G:(g + 1) * G])
    K = logical_rows(inp["k_pool"], bt, s, N, g)
    V = logical_rows(inp["v_pool"], bt, s, N, g)
    Kc = K if code_pool is None else logical_rows(code_pool, bt, s, N, g)
    o_codes, o_radii = oracle.encode_keys(Kc, P)
    if check_codes:
        g_codes = logical_codes(codes, bt, s, N, g)
        g_radii = logical_radii(radii, bt, s, N, g)
        bad = np.nonzero((g_codes != o_codes).any(axis=1))[0]
        assert len(bad) == 0, f"codes differ at {len(bad)} keys, first {bad[:5]}"
        assert np.array_equal(g_radii, o_radii), "radii differ"
    r = oracle.decode_unit(q, P, o_codes, o_radii, K, V, cfg.top_k, cfg.window,
                           cfg.sinks, radius_mode=cfg.radius_weight,
                           pages=cfg.select_pages, lsh=(cfg.lsh_tables, cfg.lsh_bits))
    if "q8" in gpu:
        g_q8 = gpu["q8"][s, g * G:(g + 1) * G].cpu().numpy()
        assert np.array_equal(g_q8, r["q8"]), "query codes differ"
    if gpu.get("scores") is not None:
        g_sc = gpu["scores"][s, g, :N].cpu().numpy()
        bad = np.nonzero(g_sc != r["scores"])[0]
        assert len(bad) == 0, f"scores differ at {len(bad)} keys, first {bad[:5]}"
    cnt = int(gpu["cnt"][s, g].item())
    assert cnt == len(r["sel"]), (cnt, len(r["sel"]))
    g_sel = gpu["sel"][s, g].cpu().numpy()
    assert np.array_equal(np.sort(g_sel[:cnt]), np.sort(r["sel"])), "selection differs"
    assert (g_sel[cnt:] == -1).all(), "selection list not -1 past the count"
    g_out = gpu["out"][s, g * G:(g + 1) * G].double().cpu().numpy()
    err = np.abs(g_out - r["out"])
    ok = err <= ATOL + RTOL * np.abs(r["out"])
    assert ok.all(), f"out: max abs err {err.max():.3g}"
    rec = None
    if needles is not None and len(needles):
        rec = float(np.isin(needles, g_sel[:cnt]).mean())
    big = np.abs(r["out"]) >= 0.2
    return {"max_abs": float(err.max()) if err.size else 0.0,
            "max_rel": float((err[big] / np.abs(r["out"][big])).max()) if big.any() else 0.0,
            "recall": rec}


def oracle_check_units(cfg: dkv.Config, inp: dict, gpu: dict, codes, radii, units,
                       debug: dict = None, chunk: int = 16, log=None) -> dict:
    """Compares many (sequence, KV head) units with the oracle at once.

    The oracle encodes every unit's keys itself (one call over all rows of a
    chunk of units) and decodes the chunk with OpenMP over units.  Checked
    per unit: codes and radii of all N keys (bit-exact), the selection as a
    set and its count (bit-exact), entries past the count (-1), and the
    outputs (within the tolerance) of ``gpu``; with ``debug`` (a
    dkv_decode_debug result) also its query codes and every key's score.
    Returns the largest absolute output error and the needle recalls."""
    bt = inp["block_table"].cpu().numpy()
    lens = inp["seq_lens"].cpu().numpy()
    G, b, d = cfg.group, cfg.code_bits, cfg.head_dim
    P = tensor_bits(inp["proj"])
    qall = tensor_bits(inp["q"])
    g_cnt = gpu["cnt"].cpu().numpy()
    g_sel = gpu["sel"].cpu().numpy()
    g_out = gpu["out"].double().cpu().numpy()
    d_q8 = debug["q8"].cpu().numpy() if debug is not None else None
    max_abs, recalls, checked = 0.0, [], 0
    for c0 in range(0, len(units), chunk):
        part = units[c0:c0 + chunk]
        U = len(part)
        Ns = np.array([int(lens[s]) for s, _ in part], np.int32)
        Nmax = max(1, int(Ns.max()))
        K = np.zeros((U, Nmax, d), np.uint16)
        V = np.zeros((U, Nmax, d), np.uint16)
        q = np.zeros((U, G, d), np.uint16)
        for i, (s, g) in enumerate(part):
            n = int(Ns[i])
            K[i, :n] = logical_rows(inp["k_pool"], bt, s, n, g)
            V[i, :n] = logical_rows(inp["v_pool"], bt, s, n, g)
            q[i] = qall[s, g * G:(g + 1) * G]
        rows = np.concatenate([K[i, :int(Ns[i])] for i in range(U)], axis=0)
        oc, orad = oracle.encode_keys(rows, P)
        o_codes = np.zeros((U, Nmax, b // 32), np.uint32)
        o_radii = np.zeros((U, Nmax), np.uint8)
        off = 0
        for i, (s, g) in enumerate(part):
            n = int(Ns[i])
            o_codes[i, :n], o_radii[i, :n] = oc[off:off + n], orad[off:off + n]
            off += n
            gc = logical_codes(codes, bt, s, n, g)
            bad = np.nonzero((gc != o_codes[i, :n]).any(axis=1))[0]
            assert len(bad) == 0, f"unit {(s, g)}: codes differ at {len(bad)} keys, first {bad[:5]}"
            assert np.array_equal(logical_radii(radii, bt, s, n, g), o_radii[i, :n]), \
                f"unit {(s, g)}: radii differ"
        r = oracle.decode_units(q, P, o_codes, o_radii, K, V, Ns, cfg.top_k, cfg.window,
                                cfg.sinks, want_scores=debug is not None,
                                radius_mode=cfg.radius_weight, pages=cfg.select_pages,
                                lsh=(cfg.lsh_tables, cfg.lsh_bits))
        for i, (s, g) in enumerate(part):
            n = int(Ns[i])
            if debug is not None:
                assert np.array_equal(d_q8[s, g * G:(g + 1) * G], r["q8"][i]), \
                    f"unit {(s, g)}: query codes differ"
                ds = debug["scores"][s, g, :n].cpu().numpy()
                bad = np.nonzero(ds != r["scores"][i, :n])[0]
                assert len(bad) == 0, f"unit {(s, g)}: scores differ at {len(bad)} keys"
            sel = r["sel"][i]
            cnt = int(g_cnt[s, g])
            assert cnt == len(sel), (s, g, cnt, len(sel))
            assert np.array_equal(np.sort(g_sel[s, g, :cnt]), np.sort(sel)), \
                f"unit {(s, g)}: selection differs"
            assert (g_sel[s, g, cnt:] == -1).all(), f"unit {(s, g)}: list not -1 past count"
            ref = r["out"][i]
            err = np.abs(g_out[s, g * G:(g + 1) * G] - ref)
            ok = err <= ATOL + RTOL * np.abs(ref)
            assert ok.all(), f"unit {(s, g)}: out max abs err {err.max():.3g}"
            max_abs = max(max_abs, float(err.max()) if err.size else 0.0)
            nd = inp["needles"][s][g]
            if len(nd):
                recalls.append(float(np.isin(nd, g_sel[s, g, :cnt]).mean()))
            checked += 1
        if log is not None:
            log(f"  oracle checked {checked}/{len(units)} units")
    return {"max_abs": max_abs, "recalls": recalls, "units": checked}
