"""Seeded synthetic decode workloads (inputs only).

This module draws the random inputs that both the GPU library and the CPU
oracle consume: queries, paged K/V pools, the Gaussian projection, block
tables, sequence lengths and planted needle keys.  It holds none of the
method's arithmetic: it draws numbers, scales them, places them and rounds
them to bf16.  Whoever calls it hands the very same bytes to both sides.

Recipe (every workload):
  * projection P [d][b]: i.i.d. N(0,1), rounded to bf16 (one P per layer,
    shared by all KV heads);
  * queries q [B][Hq][d]: N(0,1) -> bf16, no outliers;
  * keys and values: N(0,1); when ``outliers`` is set, 4 channels per KV
    head (distinct, seeded, drawn separately for K and V) are scaled x8;
  * when ``lognormal_sigma`` > 0, every non-needle key row is multiplied by
    exp(sigma*z), z ~ N(0,1) (heavy-tailed radii);
  * needles: per (sequence, KV head g) ``needles`` positions, uniform without
    replacement in [sinks, N - window); needle j becomes
    3*q[s, g*G + (j mod G)] + (the regular key row drawn there);
  * pages of 16 tokens; physical block ids are a seeded permutation of all
    blocks, so consecutive pages of a sequence are scattered in the pools;
    unused block-table entries hold -1;
  * lengths: fixed, or rounded exp(U(ln lo, ln hi)) per sequence (ragged).

Small arrays (P, q, channels, positions, lengths, the permutation) come from
numpy's PCG64 seeded through ``SeedSequence``; the bulk K/V draws come from a
torch generator on the target device seeded from the same sequence.  Draws
are fp32, rounded to bf16 with round-to-nearest-even (torch ``.to``).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np
import torch

PAGE = 16


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    code_bits: int
    top_k: int
    window: int
    sinks: int
    seq_len: int = 0                       # fixed length (when not ragged)
    ragged: Optional[Tuple[int, int]] = None  # (lo, hi) log-uniform lengths
    needles: int = 0                       # per (sequence, KV head)
    outliers: bool = True
    lognormal_sigma: float = 0.0
    head_dim: int = 128
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def config_dict(self) -> dict:
        d = dataclasses.asdict(self)
        d["workload"] = d.pop("name")
        return d


# The five workloads, shaped like the pages' up-to-128K-token contexts on a
# Llama-3-8B-shaped GQA layer (32 query heads, 8 KV heads, d = 128).
WORKLOADS = {
    "mha1_n4k_b64": Workload(
        "mha1_n4k_b64", batch=1, num_q_heads=1, num_kv_heads=1, code_bits=64,
        top_k=64, window=64, sinks=4, seq_len=4096, needles=8, seed=1001),
    "gqa32x8_bs1_n32k_b128": Workload(
        "gqa32x8_bs1_n32k_b128", batch=1, num_q_heads=32, num_kv_heads=8,
        code_bits=128, top_k=1024, window=256, sinks=4, seq_len=32768,
        needles=16, seed=1002),
    "gqa32x8_bs16_n128k_b128": Workload(
        "gqa32x8_bs16_n128k_b128", batch=16, num_q_heads=32, num_kv_heads=8,
        code_bits=128, top_k=2048, window=512, sinks=4, seq_len=131072,
        seed=1003),
    "gqa32x8_ragged64_4k-128k_b128": Workload(
        "gqa32x8_ragged64_4k-128k_b128", batch=64, num_q_heads=32,
        num_kv_heads=8, code_bits=128, top_k=1024, window=256, sinks=4,
        ragged=(4096, 131072), seed=1004),
    "gqa32x8_bs4_n256k_b256_lognormal": Workload(
        "gqa32x8_bs4_n256k_b256_lognormal", batch=4, num_q_heads=32,
        num_kv_heads=8, code_bits=256, top_k=4096, window=1024, sinks=4,
        seq_len=262144, needles=64, outliers=False, lognormal_sigma=0.5,
        seed=1005),
}

# Reduced shapes for parity at sizes the oracle finishes in seconds; they
# keep the real head layout and code widths, span many 16-token pages and
# end on a ragged (partial) page.
SMALL = {
    "small_mha_b64": Workload(
        "small_mha_b64", batch=2, num_q_heads=1, num_kv_heads=1, code_bits=64,
        top_k=64, window=64, sinks=4, seq_len=3001, needles=8, seed=11),
    "small_gqa_b128": Workload(
        "small_gqa_b128", batch=2, num_q_heads=8, num_kv_heads=2,
        code_bits=128, top_k=200, window=64, sinks=4, seq_len=5003,
        needles=12, seed=12),
    "small_gqa_b256_lognormal": Workload(
        "small_gqa_b256_lognormal", batch=2, num_q_heads=8, num_kv_heads=2,
        code_bits=256, top_k=300, window=100, sinks=4, seq_len=4099,
        needles=16, outliers=False, lognormal_sigma=0.5, seed=13),
    "small_ragged_b128": Workload(
        "small_ragged_b128", batch=5, num_q_heads=8, num_kv_heads=2,
        code_bits=128, top_k=128, window=48, sinks=4, ragged=(200, 6000),
        needles=4, seed=14),
}


def get(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    return SMALL[name]


def _bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def seq_lengths(wl: Workload) -> np.ndarray:
    """Per-sequence cached lengths (the current token included)."""
    ss = np.random.SeedSequence(wl.seed)
    rng = np.random.default_rng(ss.spawn(8)[7])
    if wl.ragged is None:
        return np.full(wl.batch, wl.seq_len, np.int32)
    lo, hi = wl.ragged
    u = rng.uniform(math.log(lo), math.log(hi), size=wl.batch)
    return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)


def make_inputs(wl: Workload, device: str = "cpu", seed: Optional[int] = None) -> dict:
    """Draws one decode workload.  Returns a dict of tensors on ``device``:

    q [B][Hq][d] bf16; k_pool, v_pool [num_blocks][16][Hkv][d] bf16;
    proj [d][b] bf16; block_table [B][max_blocks] int32 (-1 = unused);
    seq_lens [B] int32; plus host-side numpy ``needles`` [B][Hkv] lists of
    positions and the scalars num_blocks, max_blocks, max_seq_len."""
    seed = wl.seed if seed is None else seed
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(8)
    r_proj, r_q, r_chan, r_needle, r_perm = (np.random.default_rng(k) for k in kids[:5])
    torch_seed_k = int(kids[5].generate_state(1, np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)
    torch_seed_v = int(kids[6].generate_state(1, np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)
    B, Hq, Hkv, d, b = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.code_bits
    G = Hq // Hkv

    lens = seq_lengths(wl) if seed == wl.seed else _lengths_with_seed(wl, seed)
    nblk_seq = (lens.astype(np.int64) + PAGE - 1) // PAGE
    num_blocks = int(nblk_seq.sum())
    max_blocks = int(nblk_seq.max())
    perm = r_perm.permutation(num_blocks).astype(np.int32)
    bt = np.full((B, max_blocks), -1, np.int32)
    off = 0
    for s in range(B):
        n = int(nblk_seq[s])
        bt[s, :n] = perm[off:off + n]
        off += n

    proj = _bf16(torch.from_numpy(r_proj.standard_normal((d, b), dtype=np.float32))).to(device)
    q32 = torch.from_numpy(r_q.standard_normal((B, Hq, d), dtype=np.float32))
    q = _bf16(q32)

    gk = torch.Generator(device=device)
    gk.manual_seed(torch_seed_k)
    gv = torch.Generator(device=device)
    gv.manual_seed(torch_seed_v)
    shape = (num_blocks, PAGE, Hkv, d)
    k32 = torch.randn(shape, generator=gk, device=device, dtype=torch.float32)
    v32 = torch.randn(shape, generator=gv, device=device, dtype=torch.float32)
    if wl.outliers:
        for pool in (k32, v32):
            scale = torch.ones(Hkv, d, dtype=torch.float32)
            for h in range(Hkv):
                ch = r_chan.choice(d, size=4, replace=False)
                scale[h, torch.from_numpy(ch)] = 8.0
            pool.mul_(scale.to(device))

    # Needle placement (host), physical (block, slot) of each needle.
    needles = [[np.zeros(0, np.int64) for _ in range(Hkv)] for _ in range(B)]
    needle_rows = []  # (block, slot, head, s, query head)
    if wl.needles > 0:
        for s in range(B):
            lo, hi = wl.sinks, int(lens[s]) - wl.window
            for g in range(Hkv):
                if hi - lo < wl.needles:
                    continue
                pos = np.sort(r_needle.choice(np.arange(lo, hi), size=wl.needles,
                                              replace=False))
                needles[s][g] = pos
                for j, p in enumerate(pos):
                    needle_rows.append((int(bt[s, p // PAGE]), int(p % PAGE), g, s,
                                        g * G + (j % G)))

    if wl.lognormal_sigma > 0:
        z = torch.randn((num_blocks, PAGE, Hkv), generator=gk, device=device,
                        dtype=torch.float32)
        fac = torch.exp(wl.lognormal_sigma * z)
        if needle_rows:
            idx = torch.tensor([[r[0], r[1], r[2]] for r in needle_rows], dtype=torch.long)
            fac[idx[:, 0].to(device), idx[:, 1].to(device), idx[:, 2].to(device)] = 1.0
        k32.mul_(fac.unsqueeze(-1))

    if needle_rows:
        idx = torch.tensor([[r[0], r[1], r[2]] for r in needle_rows], dtype=torch.long)
        src = torch.tensor([[r[3], r[4]] for r in needle_rows], dtype=torch.long)
        qsel = q.float()[src[:, 0], src[:, 1]].to(device)   # exact bf16 values
        bi, si, hi_ = (idx[:, i].to(device) for i in range(3))
        k32[bi, si, hi_] = 3.0 * qsel + k32[bi, si, hi_]

    k_pool = _bf16(k32)
    del k32
    v_pool = _bf16(v32)
    del v32
    return {
        "q": q.to(device),
        "k_pool": k_pool,
        "v_pool": v_pool,
        "proj": proj,
        "block_table": torch.from_numpy(bt).to(device),
        "seq_lens": torch.from_numpy(lens.astype(np.int32)).to(device),
        "needles": needles,
        "num_blocks": num_blocks,
        "max_blocks": max_blocks,
        "max_seq_len": int(lens.max()),
    }


def _lengths_with_seed(wl: Workload, seed: int) -> np.ndarray:
    return seq_lengths(dataclasses.replace(wl, seed=seed))
