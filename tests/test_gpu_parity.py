"""GPU parity: libdkv (through the C ABI) against the CPU oracle.

Bit-exact: key codes, radii, query codes, scores, selected index sets and
counts.  Within |err| <= 2e-3 + 1e-2*|ref|: attention outputs (fp32
accumulation on the GPU, fp64 in the oracle).

Small workloads compare every (sequence, KV head) unit; so do the five
full-size workloads, which run at their real shapes through the entry points
the benchmark times.  Option paths (linear weight, pages, LSH) compare
sampled units at full size.
"""
import numpy as np
import pytest
import torch

import workloads
import hashed_top_sparse_amd as dkv
import oracle
from helpers import PAGE, logical_codes, logical_radii, logical_rows, tensor_bits
from parity import (check_unit, config_of, gpu_decode, gpu_decode_append, gpu_decode_lsh,
                    gpu_encode_all, oracle_check_units)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run(wl, units=None, **cfg_over):
    print(f"[case] {wl.name} {cfg_over}", flush=True)
    cfg = config_of(wl, **cfg_over)
    inp = workloads.make_inputs(wl, DEV)
    codes, radii = gpu_encode_all(cfg, inp)
    gpu = gpu_decode(cfg, inp, codes, radii, debug=True)
    if units is None:
        units = [(s, g) for s in range(wl.batch) for g in range(wl.num_kv_heads)]
    stats = []
    for s, g in units:
        nd = inp["needles"][s][g] if "top_k" not in cfg_over else None
        stats.append(check_unit(cfg, inp, gpu, codes, radii, s, g, needles=nd))
    return stats


@pytest.mark.parametrize("name", sorted(workloads.SMALL))
def test_small_workloads_every_unit(name):
    stats = _run(workloads.get(name))
    recalls = [st["recall"] for st in stats if st["recall"] is not None]
    assert all(r == 1.0 for r in recalls)


@pytest.mark.parametrize("name,over", [
    ("small_mha_b64", {}),
    ("small_gqa_b128", {}),
    ("small_gqa_b256_lognormal", {}),
    ("small_gqa_b128", dict(num_q_heads=32, num_kv_heads=8)),
])
def test_append_encode_writes_exactly_its_range(name, over):
    """dkv_encode over a per-sequence range [start, end): the one-token
    append of a decode step and ragged chunks.  Codes and radii inside the
    range are bit-exact to the oracle; every other slot keeps its old
    contents."""
    import dataclasses
    wl = dataclasses.replace(workloads.get(name), **over)
    print(f"[case] append {wl.name} {over}", flush=True)
    cfg = config_of(wl)
    inp = workloads.make_inputs(wl, DEV)
    nb, Hkv, W = inp["k_pool"].shape[0], wl.num_kv_heads, wl.code_bits // 32
    sentinel_code, sentinel_r = 0x5A5A5A5A, 0xA5
    codes = torch.full((nb, Hkv, PAGE, W), sentinel_code, dtype=torch.int32, device=DEV)
    radii = torch.full((nb, Hkv, PAGE), sentinel_r, dtype=torch.uint8, device=DEV)
    lens = inp["seq_lens"].cpu().numpy()
    # sequence 0: the newest token only; sequence 1: a chunk that starts and
    # ends inside pages and spans more than one 16-token tile
    ranges = [(int(lens[0]) - 1, int(lens[0])),
              (int(lens[1]) // 3 + 5, int(lens[1]) - 7)]
    start = torch.tensor([a for a, _ in ranges], dtype=torch.int32, device=DEV)
    end = torch.tensor([e for _, e in ranges], dtype=torch.int32, device=DEV)
    dkv.encode(cfg, inp["k_pool"], inp["block_table"][:2], start, end,
               max(e - a for a, e in ranges), inp["proj"], codes, radii)
    torch.cuda.synchronize()
    bt = inp["block_table"].cpu().numpy()
    P = tensor_bits(inp["proj"])
    written = 0
    for s, (a, e) in enumerate(ranges):
        N = int(lens[s])
        for g in range(Hkv):
            K = logical_rows(inp["k_pool"], bt, s, N, g)
            o_codes, o_radii = oracle.encode_keys(K[a:e], P)
            g_codes = logical_codes(codes, bt, s, N, g)
            g_radii = logical_radii(radii, bt, s, N, g)
            assert np.array_equal(g_codes[a:e], o_codes), (s, g)
            assert np.array_equal(g_radii[a:e], o_radii), (s, g)
            written += e - a
    c = codes.cpu().numpy().view(np.uint32)
    r = radii.cpu().numpy()
    assert int((c != sentinel_code).any(axis=-1).sum()) <= written
    # no slot outside the ranges was written: count untouched radius bytes,
    # allowing for encoded radii that happen to equal the sentinel
    hits = sum(int((logical_radii(radii, bt, s, int(lens[s]), g)[a:e] == sentinel_r).sum())
               for s, (a, e) in enumerate(ranges) for g in range(Hkv))
    assert int((r == sentinel_r).sum()) == r.size - written + hits


@pytest.mark.parametrize("over", [
    dict(top_k=5000, window=16, sinks=4),      # dense: selection = everything
    dict(top_k=0, window=64, sinks=4),         # window + sinks only
    dict(top_k=64, window=0, sinks=0),         # top-k only
    dict(top_k=1, window=1, sinks=1),
])
def test_small_selection_edge_configs(over):
    _run(workloads.get("small_gqa_b128"), **over)


def test_short_and_empty_sequences():
    """N = 0, 1, <= sinks, <= sinks + window, and a one-page tail."""
    wl = workloads.get("small_gqa_b128")
    cfg = config_of(wl)
    inp = workloads.make_inputs(wl, DEV)
    codes, radii = gpu_encode_all(cfg, inp)
    for lens in ([0, 1], [3, 4], [5, 68], [69, 17]):
        sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
        sub = dict(inp, seq_lens=sl, max_seq_len=int(max(lens)))
        print(f"[case] lens={lens}", flush=True)
        gpu = gpu_decode(cfg, sub, codes, radii, debug=True,
                         seq_lens=sl, max_seq_len=int(max(lens)))
        for s in range(2):
            for g in range(wl.num_kv_heads):
                if lens[s] == 0:
                    assert int(gpu["cnt"][s, g]) == 0
                    assert (gpu["out"][s, g * cfg.group:(g + 1) * cfg.group] == 0).all()
                    continue
                check_unit(cfg, sub, gpu, codes, radii, s, g)


@pytest.mark.parametrize("append", [False, True])
def test_many_units_window_in_split_kernel(append):
    """More (sequence, KV head) units than half the compute units: the window
    rows are attended by the split kernel's own splits (taken from the
    positions and the block table) instead of beside the query prep.  Ragged
    short lengths put sequences below sinks + window too."""
    import dataclasses
    wl = dataclasses.replace(workloads.get("small_ragged_b128"), name="many_units_ragged",
                             batch=160, ragged=(3, 900), seed=21)
    cfg = config_of(wl)
    inp = workloads.make_inputs(wl, DEV)
    print(f"[case] {wl.name} units={wl.batch * wl.num_kv_heads} append={append}", flush=True)
    if append:
        gpu, codes, radii = gpu_decode_append(cfg, inp)
    else:
        codes, radii = gpu_encode_all(cfg, inp)
        gpu = gpu_decode(cfg, inp, codes, radii, debug=True)
    for s in range(wl.batch):
        for g in range(wl.num_kv_heads):
            check_unit(cfg, inp, gpu, codes, radii, s, g)


def test_forced_ties_go_to_lowest_positions():
    """Identical keys everywhere: every score ties, the lowest positions win."""
    wl = workloads.get("small_gqa_b128")
    cfg = config_of(wl)
    inp = workloads.make_inputs(wl, DEV)
    inp["k_pool"][:] = inp["k_pool"][0, 0]
    codes, radii = gpu_encode_all(cfg, inp)
    gpu = gpu_decode(cfg, inp, codes, radii, debug=True)
    for s in range(wl.batch):
        for g in range(wl.num_kv_heads):
            check_unit(cfg, inp, gpu, codes, radii, s, g)
            sel = np.sort(gpu["sel"][s, g, :int(gpu["cnt"][s, g])].cpu().numpy())
            top = sel[(sel >= wl.sinks) & (sel < int(inp["seq_lens"][s]) - wl.window)]
            assert np.array_equal(top, np.arange(wl.sinks, wl.sinks + wl.top_k))


def _run_append(wl, units=None):
    """The newest key of every sequence must be encoded by
    dkv_decode_append itself, and the step must match the oracle."""
    print(f"[case] append-decode {wl.name}", flush=True)
    cfg = config_of(wl)
    inp = workloads.make_inputs(wl, DEV)
    gpu, codes, radii = gpu_decode_append(cfg, inp)
    if units is None:
        units = [(s, g) for s in range(wl.batch) for g in range(wl.num_kv_heads)]
    for s, g in units:
        check_unit(cfg, inp, gpu, codes, radii, s, g)  # codes of all N keys
    return gpu, codes, radii, inp, cfg


@pytest.mark.parametrize("name", sorted(workloads.SMALL))
def test_decode_append_encodes_newest_key(name):
    _run_append(workloads.get(name))


def test_decode_append_equals_encode_then_decode():
    wl = workloads.get("small_ragged_b128")
    gpu, codes, radii, inp, cfg = _run_append(wl)
    ref = gpu_decode(cfg, inp, codes, radii, debug=False)
    assert torch.equal(gpu["out"], ref["out"])
    assert torch.equal(gpu["cnt"], ref["cnt"])
    assert torch.equal(torch.sort(gpu["sel"], dim=-1).values,
                       torch.sort(ref["sel"], dim=-1).values)


@pytest.mark.parametrize("copies_before,copies_after", [(3, 3), (0, 5), (6, 0)])
def test_ties_at_the_cut_split_by_position(copies_before, copies_after):
    """A few exact copies of the key that sits at rank k_eff (same code, same
    radius, so the same score) are planted before and after it: the ties at
    the threshold fall in a small score bin and must be split by position."""
    wl = workloads.get("small_gqa_b128")
    print(f"[case] ties at cut {copies_before}+{copies_after}", flush=True)
    cfg = config_of(wl)
    inp = workloads.make_inputs(wl, DEV)
    s, g = 0, 1
    N = int(inp["seq_lens"][s])
    bt = inp["block_table"].cpu().numpy()
    P = tensor_bits(inp["proj"])
    K = logical_rows(inp["k_pool"], bt, s, N, g)
    codes0, radii0 = oracle.encode_keys(K, P)
    G = cfg.group
    q = tensor_bits(inp["q"][s, g * G:(g + 1) * G])
    V = logical_rows(inp["v_pool"], bt, s, N, g)
    r = oracle.decode_unit(q, P, codes0, radii0, K, V, cfg.top_k, cfg.window, cfg.sinks)
    cand = np.arange(cfg.sinks, N - cfg.window)
    order = cand[np.lexsort((cand, -r["scores"][cand].astype(np.int64)))]
    keff = min(cfg.top_k, len(cand))
    pstar = int(order[keff - 1])
    # copy targets: candidate positions well away from pstar, not already in
    # the top k_eff + 20 (so they really add ties)
    top = set(order[:keff + 20].tolist())
    before = [p for p in range(cfg.sinks + 5, pstar) if p not in top][::37][:copies_before]
    after = [p for p in range(pstar + 1, N - cfg.window) if p not in top][::37][:copies_after]
    src_blk, src_slot = int(bt[s, pstar // PAGE]), pstar % PAGE
    for p in before + after:
        blk, slot = int(bt[s, p // PAGE]), p % PAGE
        inp["k_pool"][blk, slot, g] = inp["k_pool"][src_blk, src_slot, g]
    codes, radii = gpu_encode_all(cfg, inp)
    gpu = gpu_decode(cfg, inp, codes, radii, debug=True)
    st = check_unit(cfg, inp, gpu, codes, radii, s, g)
    sc = gpu["scores"][s, g, :N].cpu().numpy()
    assert (sc[before + after] == sc[pstar]).all()   # the ties are real
    for gg in range(wl.num_kv_heads):
        check_unit(cfg, inp, gpu, codes, radii, 1, gg)


def test_decode_is_deterministic():
    wl = workloads.get("small_ragged_b128")
    cfg = config_of(wl)
    inp = workloads.make_inputs(wl, DEV)
    codes, radii = gpu_encode_all(cfg, inp)
    a = gpu_decode(cfg, inp, codes, radii, debug=False)
    b = gpu_decode(cfg, inp, codes, radii, debug=False)
    assert torch.equal(a["out"], b["out"])
    for x, y in ((a["sel"], b["sel"]), (a["cnt"], b["cnt"])):
        assert torch.equal(torch.sort(x, dim=-1).values, torch.sort(y, dim=-1).values)


# ---------------------------------------------------------------- full size
def _same_result(a, b, what):
    assert torch.equal(a["out"], b["out"]), f"{what}: outputs differ"
    assert torch.equal(a["cnt"], b["cnt"]), f"{what}: counts differ"
    assert torch.equal(torch.sort(a["sel"], dim=-1).values,
                       torch.sort(b["sel"], dim=-1).values), f"{what}: selections differ"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_full_size_every_unit(name):
    """The five workloads at their real shapes, in the benchmark's launch
    configuration, every (sequence, KV head) unit compared with the oracle.

    The prefix [0, N-1) of every sequence is encoded with dkv_encode into
    sentinel-filled pools, then dkv_decode_append (the benchmarked step)
    encodes each sequence's newest key itself and decodes.  dkv_decode over
    the same codes and dkv_decode_debug (which also returns the query codes
    and every key's score) must agree with it bit for bit.  Against the
    oracle: codes and radii of every key, query codes, every score, the
    selected sets and counts (bit-exact), outputs within tolerance, and
    needle recall 1.0 where needles are planted."""
    wl = workloads.get(name)
    print(f"[case] full size every unit {name}", flush=True)
    cfg = config_of(wl)
    inp = workloads.make_inputs(wl, DEV)
    app, codes, radii = gpu_decode_append(cfg, inp)
    plain = gpu_decode(cfg, inp, codes, radii, debug=False)
    dbg = gpu_decode(cfg, inp, codes, radii, debug=True)
    _same_result(plain, app, "dkv_decode vs dkv_decode_append")
    _same_result(dbg, app, "dkv_decode_debug vs dkv_decode_append")
    units = [(s, g) for s in range(wl.batch) for g in range(wl.num_kv_heads)]
    st = oracle_check_units(cfg, inp, app, codes, radii, units, debug=dbg,
                            log=lambda m: print(m, flush=True))
    assert st["units"] == len(units)
    if wl.needles:
        assert st["recalls"] and all(r == 1.0 for r in st["recalls"])
    print(name, "units", st["units"], "max abs err", st["max_abs"], flush=True)
    del app, plain, dbg, codes, radii, inp
    torch.cuda.empty_cache()


def _sample_stride(keff: int, n: int, w: int, sigma: int) -> int:
    """The page-sample stride the threshold pass uses: the largest power of
    two <= 64 with 2*SP <= k_eff/16 (at least 1), doubled until the sample
    holds at most 512 of the candidate pages (every SP-th from page
    sigma/16)."""
    sp = 1
    while sp < 64 and 2 * sp <= keff // 16:
        sp *= 2
    ncp = (n - w + PAGE - 1) // PAGE - sigma // PAGE
    while (ncp + sp - 1) // sp > 512:
        sp *= 2
    return sp


def _scale_pages(inp, wl, pred, factor):
    bt = inp["block_table"].cpu().numpy()
    lens = inp["seq_lens"].cpu().numpy()
    for s in range(wl.batch):
        npg = (int(lens[s]) + 15) // 16
        pages = [p for p in range(npg) if pred(p)]
        blocks = torch.as_tensor(bt[s, pages].astype(np.int64), device=DEV)
        inp["k_pool"][blocks] = (inp["k_pool"][blocks].float() * factor).to(torch.bfloat16)


@pytest.mark.parametrize("factor", [4.0, 0.125])
def test_threshold_fallback_stays_exact(factor):
    """Keys on the sampled pages scaled up (the sampled threshold lets too
    few keys through: underflow) or down (far too many: overflow).  Either
    way the merge must rescan and stay exact."""
    import dataclasses
    base = workloads.get("small_gqa_b128")
    # long enough that the overflow case exceeds the candidate list room
    wl = dataclasses.replace(base, name="adversarial", batch=1, seq_len=40000,
                             needles=0)
    print(f"[case] adversarial factor={factor}", flush=True)
    cfg = config_of(wl)
    inp = workloads.make_inputs(wl, DEV)
    keff = min(wl.top_k, wl.seq_len - wl.window - wl.sinks)
    sp = _sample_stride(keff, wl.seq_len, wl.window, wl.sinks)
    _scale_pages(inp, wl, lambda p: p % sp == 0, factor)
    codes, radii = gpu_encode_all(cfg, inp)
    gpu = gpu_decode(cfg, inp, codes, radii, debug=True)
    for g in range(wl.num_kv_heads):
        check_unit(cfg, inp, gpu, codes, radii, 0, g)


# ---------------------------------------------------- linear radius weight
LIN = dict(radius_weight=dkv.RADIUS_LINEAR)


@pytest.mark.parametrize("name", sorted(workloads.SMALL))
def test_linear_radius_weight_small_every_unit(name):
    """Scores w(r8) * max_h s_h with w = rne(2^(r8/16)): bit-exact scores,
    selection and counts, outputs within tolerance, on every unit."""
    stats = _run(workloads.get(name), **LIN)
    rec = [st["recall"] for st in stats if st["recall"] is not None]
    print(name, "needle recall (linear weight)", np.mean(rec) if rec else None)


@pytest.mark.parametrize("name,units", [
    ("gqa32x8_bs16_n128k_b128", [(0, 0), (15, 7)]),
    ("gqa32x8_bs4_n256k_b256_lognormal", [(1, 2)]),
])
def test_full_size_linear_radius_weight(name, units):
    _run(workloads.get(name), units, **LIN)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("factor", [4.0, 0.125])
def test_linear_weight_threshold_fallback_stays_exact(factor):
    """The adversarial sample of the fallback test under the linear weight
    (the merge's rescan scores with the same weight)."""
    import dataclasses
    base = workloads.get("small_gqa_b128")
    wl = dataclasses.replace(base, name="adversarial", batch=1, seq_len=40000,
                             needles=0)
    print(f"[case] adversarial linear factor={factor}", flush=True)
    cfg = config_of(wl, **LIN)
    inp = workloads.make_inputs(wl, DEV)
    keff = min(wl.top_k, wl.seq_len - wl.window - wl.sinks)
    sp = _sample_stride(keff, wl.seq_len, wl.window, wl.sinks)
    _scale_pages(inp, wl, lambda p: p % sp == 0, factor)
    codes, radii = gpu_encode_all(cfg, inp)
    gpu = gpu_decode(cfg, inp, codes, radii, debug=True)
    for g in range(wl.num_kv_heads):
        check_unit(cfg, inp, gpu, codes, radii, 0, g)


@pytest.mark.parametrize("mode", ["rescan", "unstaged"])
def test_linear_weight_wide_score_range_stays_exact(mode):
    """Scores spanning far more than 2^24 reach the merge's exact k-th
    largest search.  Codes come from keys scaled x64 (radius codes near the
    top, linear weights in the tens of thousands); then either the sampled
    pages are scaled x4 more, so too few keys pass the sampled threshold and
    the merge rescans every key (a score range near 2^28), or the top-k is
    so large that the candidates do not fit the merge's LDS staging and the
    search runs over the lists in global memory.  Attention runs over the
    unscaled pool."""
    import dataclasses
    base = workloads.get("small_gqa_b128")
    over = dict(top_k=7000) if mode == "unstaged" else {}
    wl = dataclasses.replace(base, name=f"wide_{mode}", batch=1, seq_len=40000,
                             needles=0, **over)
    print(f"[case] wide score range, linear weight, {mode}", flush=True)
    cfg = config_of(wl, **LIN)
    inp = workloads.make_inputs(wl, DEV)
    k_big = dict(inp, k_pool=(inp["k_pool"].float() * 64.0).to(torch.bfloat16))
    if mode == "rescan":
        keff = min(wl.top_k, wl.seq_len - wl.window - wl.sinks)
        sp = _sample_stride(keff, wl.seq_len, wl.window, wl.sinks)
        _scale_pages(k_big, wl, lambda p: p % sp == 0, 4.0)
    codes, radii = gpu_encode_all(cfg, k_big)
    gpu = gpu_decode(cfg, inp, codes, radii, debug=True)
    n = int(inp["seq_lens"][0].item())
    for g in range(wl.num_kv_heads):
        check_unit(cfg, inp, gpu, codes, radii, 0, g, code_pool=k_big["k_pool"])
        sc = gpu["scores"][0, g, wl.sinks:n - wl.window].long()
        assert int(sc.max() - sc.min()) > 2 ** 26   # far past a 24-bit search
    torch.cuda.empty_cache()


def test_linear_weight_largest_radii():
    """Codes built from keys scaled so most radius codes clamp at 255
    (weight 62757, the largest) at b = 256: scores far beyond the exact
    range of a float product stay exact and ordered.  (Attention runs over
    the unscaled pool, so the outputs keep ordinary logits.)"""
    import dataclasses
    wl = dataclasses.replace(workloads.get("small_gqa_b256_lognormal"), name="big_radii",
                             needles=0)
    print("[case] big radii linear", flush=True)
    cfg = config_of(wl, **LIN)
    inp = workloads.make_inputs(wl, DEV)
    k_big = (inp["k_pool"].float() * 512.0).to(torch.bfloat16)
    codes, radii = gpu_encode_all(cfg, dict(inp, k_pool=k_big))
    assert (radii == 255).float().mean().item() > 0.5
    gpu = gpu_decode(cfg, inp, codes, radii, debug=True)
    big = 0
    for s in range(wl.batch):
        for g in range(wl.num_kv_heads):
            check_unit(cfg, inp, gpu, codes, radii, s, g, code_pool=k_big)
            n = int(inp["seq_lens"][s].item())
            big = max(big, int(gpu["scores"][s, g, :n].abs().max().item()))
    # far past 2^24, where a float product would no longer be exact
    assert big > 2 ** 26, big


# ------------------------------------------------ page-granular selection
PAGES = dict(select_pages=True)


@pytest.mark.parametrize("name", sorted(workloads.SMALL))
def test_page_selection_small_every_unit(name):
    """The top top_k/16 pages, each scored by its best candidate key: bit-exact
    scores, selected sets and counts, outputs within tolerance."""
    stats = _run(workloads.get(name), **PAGES)
    rec = [st["recall"] for st in stats if st["recall"] is not None]
    print(name, "needle recall (pages)", np.mean(rec) if rec else None)


@pytest.mark.parametrize("over", [
    dict(top_k=5000, window=16, sinks=4),      # every page of the range
    dict(top_k=15, window=64, sinks=4),        # below one page: window + sinks
    dict(top_k=64, window=0, sinks=0),
    dict(top_k=33, window=21, sinks=19),       # partial edge pages
    dict(top_k=64, window=64, sinks=4, radius_weight=dkv.RADIUS_LINEAR),
])
def test_page_selection_edge_configs(over):
    _run(workloads.get("small_gqa_b128"), **PAGES, **over)


def test_page_selection_ties_go_to_lowest_pages():
    """Identical keys everywhere: every page ties, the lowest pages win."""
    wl = workloads.get("small_gqa_b128")
    cfg = config_of(wl, **PAGES)
    inp = workloads.make_inputs(wl, DEV)
    inp["k_pool"][:] = inp["k_pool"][0, 0]
    codes, radii = gpu_encode_all(cfg, inp)
    gpu = gpu_decode(cfg, inp, codes, radii, debug=True)
    kp = wl.top_k // PAGE
    for s in range(wl.batch):
        for g in range(wl.num_kv_heads):
            check_unit(cfg, inp, gpu, codes, radii, s, g)
            sel = np.sort(gpu["sel"][s, g, :int(gpu["cnt"][s, g])].cpu().numpy())
            top = sel[(sel >= wl.sinks) & (sel < int(inp["seq_lens"][s]) - wl.window)]
            assert np.array_equal(top, np.arange(wl.sinks, kp * PAGE))


def test_page_selection_short_sequences():
    wl = workloads.get("small_gqa_b128")
    cfg = config_of(wl, **PAGES)
    inp = workloads.make_inputs(wl, DEV)
    codes, radii = gpu_encode_all(cfg, inp)
    for lens in ([0, 1], [5, 68], [69, 17], [400, 333]):
        sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
        sub = dict(inp, seq_lens=sl, max_seq_len=int(max(lens)))
        print(f"[case] pages lens={lens}", flush=True)
        gpu = gpu_decode(cfg, sub, codes, radii, debug=True,
                         seq_lens=sl, max_seq_len=int(max(lens)))
        for s in range(2):
            for g in range(wl.num_kv_heads):
                if lens[s] == 0:
                    assert int(gpu["cnt"][s, g]) == 0
                    continue
                check_unit(cfg, sub, gpu, codes, radii, s, g)


@pytest.mark.parametrize("name,units,over", [
    ("gqa32x8_bs16_n128k_b128", [(0, 0), (15, 7)], {}),
    ("gqa32x8_ragged64_4k-128k_b128", [(0, 0), (17, 5), (40, 2)], {}),
    # more pages than the merge stages in LDS (its global-memory path)
    ("gqa32x8_bs4_n256k_b256_lognormal", [(1, 2)], dict(radius_weight=dkv.RADIUS_LINEAR)),
])
def test_full_size_page_selection(name, units, over):
    _run(workloads.get(name), units, **PAGES, **over)
    torch.cuda.empty_cache()



# ------------------------------------------------------ LSH candidates
def _run_lsh(wl, units=None, index_back=0, **cfg_over):
    """Index over [0, N - index_back) of every sequence, decode over N: the
    positions past the index are tested from their codes."""
    print(f"[case] lsh {wl.name} {cfg_over} index_back={index_back}", flush=True)
    cfg = config_of(wl, **cfg_over)
    inp = workloads.make_inputs(wl, DEV)
    codes, radii = gpu_encode_all(cfg, inp)
    lens = torch.clamp(inp["seq_lens"] - index_back, min=0).to(torch.int32)
    gpu = gpu_decode_lsh(cfg, inp, codes, radii, index_lens=lens)
    if units is None:
        units = [(s, g) for s in range(wl.batch) for g in range(wl.num_kv_heads)]
    cnts = []
    for s, g in units:
        check_unit(cfg, inp, gpu, codes, radii, s, g)
        cnts.append(int(gpu["cnt"][s, g]))
    return cnts


@pytest.mark.parametrize("name", sorted(workloads.SMALL))
def test_lsh_small_every_unit(name):
    _run_lsh(workloads.get(name), lsh_tables=8, lsh_bits=6)


@pytest.mark.parametrize("over", [
    dict(lsh_tables=8, lsh_bits=6, index_back=700),    # a long unindexed tail
    dict(lsh_tables=1, lsh_bits=12),                   # few candidates: all kept
    dict(lsh_tables=16, lsh_bits=2),                   # almost every key
    dict(lsh_tables=12, lsh_bits=10, radius_weight=dkv.RADIUS_LINEAR),
    dict(lsh_tables=8, lsh_bits=6, top_k=0, window=64, sinks=4),
])
def test_lsh_edge_configs(over):
    over = dict(over)
    back = over.pop("index_back", 0)
    _run_lsh(workloads.get("small_gqa_b128"), index_back=back, **over)


def test_lsh_index_of_nothing():
    """An index built over empty prefixes: every key is tested directly."""
    wl = workloads.get("small_ragged_b128")
    _run_lsh(wl, index_back=1 << 20, lsh_tables=6, lsh_bits=8)


@pytest.mark.parametrize("name,units,over", [
    ("gqa32x8_bs16_n128k_b128", [(0, 0), (15, 7)], dict(lsh_tables=8, lsh_bits=10)),
    ("gqa32x8_bs4_n256k_b256_lognormal", [(1, 2)], dict(lsh_tables=16, lsh_bits=12)),
])
def test_full_size_lsh(name, units, over):
    _run_lsh(workloads.get(name), units, index_back=100, **over)
    torch.cuda.empty_cache()


# ------------------------------------------- every code width x group size
@pytest.mark.parametrize("b", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_every_code_width_and_group_size(b, G):
    """Each (b, G) pair runs its own kernel instantiations: a small batch of
    two sequences, two KV heads, every unit checked."""
    import dataclasses
    wl = dataclasses.replace(workloads.get("small_gqa_b128"), name=f"b{b}_g{G}",
                             code_bits=b, num_q_heads=2 * G, num_kv_heads=2,
                             seq_len=2500, needles=4, top_k=160, window=48)
    stats = _run(wl)
    rec = [st["recall"] for st in stats if st["recall"] is not None]
    assert rec and all(r == 1.0 for r in rec)


@pytest.mark.parametrize("G", [2, 8])
@pytest.mark.parametrize("mode", ["pages", "lsh"])
def test_group_sizes_in_page_and_lsh_modes(G, mode):
    import dataclasses
    wl = dataclasses.replace(workloads.get("small_gqa_b128"), name=f"{mode}_g{G}",
                             num_q_heads=2 * G, num_kv_heads=2, seq_len=3000,
                             needles=4, top_k=160, window=48)
    if mode == "pages":
        _run(wl, **PAGES)
    else:
        _run_lsh(wl, index_back=40, lsh_tables=8, lsh_bits=7)
