"""dkv_decode_append_noalloc (the workspace is the library's static per-GPU
scratch array) against dkv_decode_append with a caller workspace: two calls
in a row on one GPU, the second with a smaller input, each bit-identical to
the regular entry point (codes, radii, selections, counts, outputs)."""
import dataclasses

import pytest
import torch

import hashed_top_sparse_amd as dkv
import workloads
from helpers import PAGE
from parity import config_of, gpu_decode_append

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _noalloc(cfg, inp):
    """The same steps as parity.gpu_decode_append, through the no-alloc call."""
    nb = inp["k_pool"].shape[0]
    Hkv, B = cfg.num_kv_heads, inp["block_table"].shape[0]
    codes = torch.full((nb, Hkv, PAGE, cfg.code_bits // 32), 0x5A5A5A5A,
                       dtype=torch.int32, device=DEV)
    radii = torch.full((nb, Hkv, PAGE), 0xA5, dtype=torch.uint8, device=DEV)
    start = torch.zeros(B, dtype=torch.int32, device=DEV)
    end = torch.clamp(inp["seq_lens"] - 1, min=0).to(torch.int32)
    dkv.encode(cfg, inp["k_pool"], inp["block_table"], start, end,
               inp["max_seq_len"], inp["proj"], codes, radii)
    out = torch.full((B, cfg.num_q_heads, cfg.head_dim), float("nan"), device=DEV)
    sel = torch.full((B, Hkv, cfg.select_cap), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device=DEV)
    dkv.decode_append_noalloc(cfg, inp["q"], inp["k_pool"], inp["v_pool"], codes, radii,
                              inp["block_table"], inp["seq_lens"], inp["max_seq_len"],
                              inp["proj"], out, sel, cnt)
    torch.cuda.synchronize()
    return {"out": out, "sel": sel, "cnt": cnt}, codes, radii


def test_noalloc_equals_decode_append_twice_shrinking():
    first = workloads.get("gqa32x8_bs1_n32k_b128")
    second = dataclasses.replace(workloads.get("small_ragged_b128"), name="second")
    for wl in (first, second):
        print(f"[case] noalloc {wl.name}", flush=True)
        cfg = config_of(wl)
        inp = workloads.make_inputs(wl, DEV)
        assert dkv.decode_workspace_size(cfg, wl.batch, inp["max_seq_len"]) \
            <= dkv.NOALLOC_SCRATCH_BYTES
        ref, rc, rr = gpu_decode_append(cfg, inp)
        got, gc, gr = _noalloc(cfg, inp)
        assert torch.equal(gc, rc) and torch.equal(gr, rr)
        assert torch.equal(got["cnt"], ref["cnt"])
        assert torch.equal(torch.sort(got["sel"], dim=-1).values,
                           torch.sort(ref["sel"], dim=-1).values)
        assert torch.equal(got["out"], ref["out"])


def test_noalloc_rejects_a_step_beyond_its_scratch():
    wl = workloads.get("small_gqa_b128")
    cfg = config_of(wl, top_k=64)
    inp = workloads.make_inputs(wl, DEV)
    big = 1 << 22   # max_seq_len whose workspace exceeds the scratch
    assert dkv.decode_workspace_size(cfg, wl.batch, big) > dkv.NOALLOC_SCRATCH_BYTES
    nb = inp["k_pool"].shape[0]
    codes = torch.zeros((nb, cfg.num_kv_heads, PAGE, cfg.code_bits // 32),
                        dtype=torch.int32, device=DEV)
    radii = torch.zeros((nb, cfg.num_kv_heads, PAGE), dtype=torch.uint8, device=DEV)
    out = torch.zeros((wl.batch, cfg.num_q_heads, cfg.head_dim), device=DEV)
    with pytest.raises(dkv.DkvError) as e:
        dkv.decode_append_noalloc(cfg, inp["q"], inp["k_pool"], inp["v_pool"], codes,
                                  radii, inp["block_table"], inp["seq_lens"], big,
                                  inp["proj"], out)
    assert e.value.status == 3
