"""How well the code-domain score finds the keys exact attention weighs most
(a diagnostic of the method, computed with the oracle only; CPU).

TEST INFRASTRUCTURE: uses the oracle and the seeded workload generator,
never the GPU library.

For each selection (keys; 16-token pages scored by their best key; the
top-k among multi-table LSH candidates, T tables of m bits), each radius
weight (the log code r8, or the linear rne(2^(r8/16)); pages and LSH with
the linear weight only),
each code width b in {64, 128, 256} and two key distributions (N(0,1) with
4 outlier channels x8; log-normal radii, sigma = 0.5), on every KV head of
one sequence of the 32K-token GQA shape (32 query / 8 KV heads, k = 1024,
window 256, 4 sinks):

  recall@k   |selected candidates ∩ top-k by the exact logit| / k, over
             the candidates [sinks, N - window); the exact logit of a key
             for a KV group is the largest q_h.k / sqrt(d) over the group's
             query heads (the same max aggregation the score uses);
  mass       the share of dense softmax attention (over all N keys) that
             falls on the selected keys, averaged over query heads;
  out err    |o_selected - o_dense| / |o_dense| per query head, averaged;
  needles    share of planted needle keys selected (16 per KV head, in a
             second draw of the same shape: a needle, 3 q + noise, takes
             almost all of the softmax, so the other columns use inputs
             without needles).

Usage:  python -m oracle.recall_study [--seq-len N] [--heads H]
"""
from __future__ import annotations

import argparse
import dataclasses
import os
import sys
import time

import numpy as np
import torch

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def _bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> its uint16 bit patterns."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _logical_rows(pool, bt, s, N, g):
    """Rows [N][d] (bf16 bits) of KV head g of sequence s, position order."""
    pos = np.arange(N)
    blk = bt[s, pos // workloads.PAGE]
    return pool[blk, pos % workloads.PAGE, g]


def needle_recall(wl, q, P, K, V, needles, mode, sel):
    codes, radii = oracle.encode_keys(K, P)
    r = oracle.decode_unit(q, P, codes, radii, K, V, wl.top_k, wl.window,
                           wl.sinks, radius_mode=mode, **sel)
    return float(np.isin(needles, r["sel"]).mean())


def study_unit(wl, q, P, K, V, mode, sel):
    G, d = q.shape
    N = K.shape[0]
    codes, radii = oracle.encode_keys(K, P)
    r = oracle.decode_unit(q, P, codes, radii, K, V, wl.top_k, wl.window,
                           wl.sinks, radius_mode=mode, **sel)
    qf, Kf, Vf = _bf16_to_f64(q), _bf16_to_f64(K), _bf16_to_f64(V)
    logits = qf @ Kf.T / np.sqrt(d)                     # [G][N]
    c0, c1 = wl.sinks, N - wl.window
    keff = min(wl.top_k, c1 - c0)
    exact = logits[:, c0:c1].max(axis=0)
    top_exact = c0 + np.argsort(-exact, kind="stable")[:keff]
    sel = r["sel"]
    in_c = sel[(sel >= c0) & (sel < c1)]
    recall = len(np.intersect1d(in_c, top_exact)) / keff
    a = np.exp(logits - logits.max(axis=1, keepdims=True))
    a /= a.sum(axis=1, keepdims=True)
    mass = float(a[:, sel].sum(axis=1).mean())
    o_dense = a @ Vf
    err = float((np.linalg.norm(r["out"] - o_dense, axis=1) /
                 np.linalg.norm(o_dense, axis=1)).mean())
    return recall, mass, err


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--seq-len", type=int, default=32768)
    ap.add_argument("--heads", type=int, default=8, help="KV heads studied")
    args = ap.parse_args(argv)
    base = workloads.get("gqa32x8_bs1_n32k_b128")
    dists = {
        "outliers": dict(outliers=True, lognormal_sigma=0.0),
        "lognormal": dict(outliers=False, lognormal_sigma=0.5),
    }
    print("| keys | b | select | weight | recall@k | mass | out err | needles |")
    print("|---|---|---|---|---|---|---|---|")
    t0 = time.time()
    def units(wl):
        inp = workloads.make_inputs(wl, "cpu")
        bt = inp["block_table"].numpy()
        kpool, vpool = _bits(inp["k_pool"]), _bits(inp["v_pool"])
        P, Q = _bits(inp["proj"]), _bits(inp["q"])
        N = int(inp["seq_lens"][0])
        G = wl.group
        for g in range(min(args.heads, wl.num_kv_heads)):
            yield (Q[0, g * G:(g + 1) * G], P, _logical_rows(kpool, bt, 0, N, g),
                   _logical_rows(vpool, bt, 0, N, g), np.asarray(inp["needles"][0][g]))

    for dname, dkw in dists.items():
        for b in (64, 128, 256):
            plain = dataclasses.replace(base, code_bits=b, seq_len=args.seq_len,
                                        needles=0, **dkw)
            with_nd = dataclasses.replace(plain, needles=16)
            variants = [("keys", 0, {}), ("keys", 1, {}), ("pages", 1, dict(pages=True)),
                        ("lsh 8x8", 1, dict(lsh=(8, 8))), ("lsh 8x10", 1, dict(lsh=(8, 10)))]
            for sname, mode, sel in variants:
                mname = "linear" if mode else "log r8"
                m = np.array([study_unit(plain, q, P, K, V, mode, sel)
                              for q, P, K, V, _ in units(plain)]).mean(axis=0)
                nd = np.mean([needle_recall(with_nd, q, P, K, V, n, mode, sel)
                              for q, P, K, V, n in units(with_nd)])
                print(f"| {dname} | {b} | {sname} | {mname} | {m[0]:.3f} | "
                      f"{m[1]:.3f} | {m[2]:.3f} | {nd:.3f} |", flush=True)
    print(f"\n({time.time() - t0:.0f} s; seq_len {args.seq_len}, "
          f"{args.heads} KV heads per row, seed {base.seed})")


if __name__ == "__main__":
    main()
