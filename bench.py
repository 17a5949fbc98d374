#!/usr/bin/env python
"""Decode-step benchmark of score-then-select sparse attention on one MI355X.

One step = the whole hot path for one batch: one dkv_decode_append call,
which encodes the current token of every sequence (sign code + radius of
B x Hkv keys) and runs the decode (query codes, score of every cached key,
selection of sinks + window + top-k, attention over the selection, split
merge).  The prefix codes are built once before timing; with
--encode-prefix each step also re-encodes every cached key first (dkv_encode
over the whole prefix, then the decode: the "encode + decode" workload).
Inputs are seeded synthetic tensors resident in HBM (see workloads/).

Timing.  After W warm-up steps, K steps are timed one by one, each after a
1 GiB read that evicts the 256 MB last-level cache (outside its HIP events),
so every step streams its codes and rows from HBM; ``ms_per_step`` and
``value`` come from the median of those K step times.  Beside it: the same K
steps back to back without flushes ("warm", where the cache can carry part
of the working set from one step to the next), per-stage medians from cold
steps with an event before every stage, and cold steps after a 1 GiB write
("cold_dirty": the write-back of the dirty lines competes with the step).

Prints ONE JSON line: scored keys per second (every (key, KV head) pair of
every sequence is scored once per step), the step latency, per-stage times,
the roofline of the dominant kernel (the score stage: it streams every key's
code and radius), and the CPU oracle timed on a bounded sample of the same
workload on this host's cores (its encode and its decode step).

    python bench.py [--gpus 1] [--steps 50] [--warmup 10]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("scored keys/s and decode-step latency at 128K ctx; "
          "achieved HBM GB/s vs peak")
DEFAULT_WORKLOAD = "gqa32x8_bs16_n128k_b128"
HBM_PEAK_GBS = 8000.0
PAGE = 16


class HipEvents:
    """hipEvent_t handles through ctypes (timing on the launch stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(h.value)
        return out

    def record(self, ev, stream_handle):
        if self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream_handle)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                        ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(ctypes.c_void_p(e))


def algorithmic_bytes(wl, lens, cfg) -> dict:
    """Bytes the method itself must move per step (not the dense K/V)."""
    Hkv, Hq, d, b = wl.num_kv_heads, wl.num_q_heads, wl.head_dim, wl.code_bits
    keys = int(sum(int(n) for n in lens)) * Hkv          # scored (key, KV head)
    sel_rows = sum(min(int(n), cfg.select_cap) for n in lens) * Hkv
    pages = sum((int(n) + PAGE - 1) // PAGE for n in lens)
    score = keys * (b // 8 + 1)
    attend = sel_rows * 4 * d                            # K + V bf16 rows
    io = len(lens) * Hq * (2 * d + 4 * d) + 4 * pages    # q in, out, table
    encode = len(lens) * Hkv * (2 * d + b // 8 + 1)      # current token
    return {"keys": keys, "score": score, "attend": attend, "io": io,
            "encode": encode, "total": score + attend + io + encode}


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel_src_digest: str, workload: str):
    """HBM bytes per launch of the score kernel from committed rocprofv3 PMC
    counters (profiles/score_traffic.json), or None when absent or taken for a
    different kernel source."""
    path = os.path.join(ROOT, "profiles", "score_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != kernel_src_digest or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, inp, units: int, seconds: float, radius_mode: int = 0,
                 pages: bool = False, lsh=(0, 0), with_prefix_encode: bool = False) -> dict:
    """The CPU oracle (as it stands) on a bounded sample of the workload: its
    encode of the sampled units' keys (timed once) and its decode step over
    them (repeated for about `seconds`)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import numpy as np

    import oracle
    from helpers import logical_rows, tensor_bits

    bt = inp["block_table"].cpu().numpy()
    lens = inp["seq_lens"].cpu().numpy()
    P = tensor_bits(inp["proj"])
    G, d, b = wl.group, wl.head_dim, wl.code_bits
    picks = [(s, g) for s in range(wl.batch) for g in range(wl.num_kv_heads)][:units]
    Nmax = max(int(lens[s]) for s, _ in picks)
    U = len(picks)
    q = np.zeros((U, G, d), np.uint16)
    K = np.zeros((U, Nmax, d), np.uint16)
    V = np.zeros((U, Nmax, d), np.uint16)
    codes = np.zeros((U, Nmax, b // 32), np.uint32)
    radii = np.zeros((U, Nmax), np.uint8)
    N = np.zeros(U, np.int32)
    qall = tensor_bits(inp["q"])
    for i, (s, g) in enumerate(picks):
        n = int(lens[s])
        N[i] = n
        q[i] = qall[s, g * G:(g + 1) * G]
        K[i, :n] = logical_rows(inp["k_pool"], bt, s, n, g)
        V[i, :n] = logical_rows(inp["v_pool"], bt, s, n, g)
    # the oracle's encode (E1 + E2) of the sampled units' keys, timed once
    rows = np.concatenate([K[i, :int(N[i])] for i in range(U)], axis=0)
    t0 = time.perf_counter()
    c_all, r_all = oracle.encode_keys(rows, P)
    enc_s = time.perf_counter() - t0
    off = 0
    for i in range(U):
        n = int(N[i])
        codes[i, :n], radii[i, :n] = c_all[off:off + n], r_all[off:off + n]
        off += n
    enc_rate = rows.shape[0] / enc_s
    # repeat the decode step until about `seconds` of CPU work is timed
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.decode_units(q, P, codes, radii, K, V, N, wl.top_k, wl.window,
                            wl.sinks, want_scores=False, radius_mode=radius_mode,
                            pages=pages, lsh=lsh)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds or reps >= 100000:
            break
    keys = float(N.sum()) * reps
    dec_rate = keys / dt
    total_rows = int(lens.sum()) * wl.num_kv_heads
    sample = (f"{U} of {wl.batch * wl.num_kv_heads} (sequence, KV head) units of "
              f"{wl.name} at full length: the oracle's encode of their "
              f"{rows.shape[0]} key rows once, then its decode step (query codes, "
              f"scores, select, attention) x{reps}")
    out = {"value": dec_rate, "unit": "scored keys/s", "cores": oracle.num_threads(),
           "kind": "oracle", "sample": sample, "seconds": dt + enc_s,
           "decode_keys_per_s": dec_rate,
           "encode": {"key_rows_per_s": enc_rate, "seconds": enc_s,
                      "sample_key_rows": int(rows.shape[0]),
                      # the whole cached prefix of the workload at that rate
                      "prefix_key_rows": total_rows,
                      "prefix_s_estimate": total_rows / enc_rate}}
    if with_prefix_encode:
        # a step that encodes every cached key and then decodes: both rates
        # per scored (key, KV head) pair
        out["value"] = 1.0 / (1.0 / enc_rate + 1.0 / dec_rate)
        out["sample"] += "; value combines both rates (encode + decode per key)"
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-units", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cold-steps", type=int, default=-1,
                    help="steps of the stage and dirty-flush measurements "
                         "(default: --steps; 0 skips them)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--encode-prefix", action="store_true",
                    help="each step first encodes every cached key of the batch "
                         "(dkv_encode over the whole prefix), then decodes")
    ap.add_argument("--select", choices=("keys", "pages"), default="keys",
                    help="select the top_k keys, or the top top_k/16 pages "
                         "(each scored by its best candidate key)")
    ap.add_argument("--lsh", default="",
                    help="T,m: select among multi-table LSH candidates (T tables "
                         "of m code bits; the index is built before timing)")
    ap.add_argument("--radius-weight", choices=("log", "linear"), default="log",
                    help="score weight of the radius code: the code r8 itself "
                         "(log) or rne(2^(r8/16)) (linear)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for "
                         "scaling PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not "
              "supported (units of (sequence, KV head) are independent, so the "
              "path would shard by KV head or sequence with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    if args.encode_prefix and args.lsh:
        print("bench.py: --encode-prefix and --lsh do not combine", file=sys.stderr)
        sys.exit(2)
    cold_steps = args.steps if args.cold_steps < 0 else args.cold_steps

    import statistics

    import torch

    import hashed_top_sparse_amd as dkv
    import workloads

    torch.cuda.set_device(0)
    wl = workloads.get(args.workload)
    cfg = dkv.Config(num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                     code_bits=wl.code_bits, top_k=wl.top_k, window=wl.window,
                     sinks=wl.sinks,
                     radius_weight=(dkv.RADIUS_LINEAR if args.radius_weight == "linear"
                                    else dkv.RADIUS_LOG),
                     select_pages=args.select == "pages",
                     lsh_tables=int(args.lsh.split(",")[0]) if args.lsh else 0,
                     lsh_bits=int(args.lsh.split(",")[1]) if args.lsh else 0)
    print(f"[bench] drawing {wl.name}", file=sys.stderr, flush=True)
    inp = workloads.make_inputs(wl, "cuda")
    B, Hkv = wl.batch, wl.num_kv_heads
    nb = inp["k_pool"].shape[0]
    dev = inp["k_pool"].device
    codes = torch.zeros((nb, Hkv, PAGE, wl.code_bits // 32), dtype=torch.int32, device=dev)
    radii = torch.zeros((nb, Hkv, PAGE), dtype=torch.uint8, device=dev)
    zeros = torch.zeros(B, dtype=torch.int32, device=dev)
    # the prefix: every cached token but each sequence's newest, which the
    # step's dkv_decode_append encodes itself
    prefix_end = torch.clamp(inp["seq_lens"] - 1, min=0).to(torch.int32)
    max_len = inp["max_seq_len"]
    dkv.encode(cfg, inp["k_pool"], inp["block_table"], zeros, inp["seq_lens"],
               max_len, inp["proj"], codes, radii)
    # the encode of every cached token once more, timed (A1 + A2)
    torch.cuda.synchronize()
    hip = HipEvents()
    eev = hip.create(2)
    hip.record(eev[0], torch.cuda.current_stream().cuda_stream)
    dkv.encode(cfg, inp["k_pool"], inp["block_table"], zeros, inp["seq_lens"],
               max_len, inp["proj"], codes, radii)
    hip.record(eev[1], torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    enc_us = hip.elapsed_ms(eev[0], eev[1]) * 1e3
    hip.destroy(eev)
    enc_rows = int(inp["seq_lens"].sum().item()) * Hkv
    enc_bytes = enc_rows * (2 * wl.head_dim + wl.code_bits // 8 + 1)
    enc_flop = enc_rows * 2 * wl.head_dim * wl.code_bits
    ws = torch.empty(dkv.decode_workspace_size(cfg, B, max_len), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    index = None
    if cfg.lsh_tables > 0:
        # the bucket index of the cached prefix (untimed, like the encode);
        # each step's newest key is past it and is tested from its code
        index = torch.empty(dkv.lsh_index_size(cfg, B, max_len), dtype=torch.uint8,
                            device=dev)
        dkv.lsh_build(cfg, codes, inp["block_table"], prefix_end, max_len, index)
    torch.cuda.synchronize()
    print("[bench] prefix encoded", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    names = dkv.decode_stage_names()
    n_ev = len(names) + 1

    def step(evs=None, enc_evs=None):
        """One step: dkv_decode_append encodes the newest key of every
        sequence and decodes (with --encode-prefix, dkv_encode of the whole
        prefix first).  With evs, HIP events bracket every decode stage."""
        if index is not None:
            dkv.decode_lsh(cfg, inp["q"], inp["k_pool"], inp["v_pool"], codes, radii,
                           inp["block_table"], inp["seq_lens"], max_len, inp["proj"],
                           index, out, ws, events=evs, stream=stream)
            return
        if args.encode_prefix:
            if enc_evs is not None:
                hip.record(enc_evs[0], sh)
            dkv.encode(cfg, inp["k_pool"], inp["block_table"], zeros, prefix_end,
                       max_len, inp["proj"], codes, radii, stream=stream)
        dkv.decode_append(cfg, inp["q"], inp["k_pool"], inp["v_pool"], codes, radii,
                          inp["block_table"], inp["seq_lens"], max_len, inp["proj"],
                          out, ws, events=evs, stream=stream)

    # 1 GiB read (evicts the last-level cache) or write (also leaves it
    # full of dirty lines)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def flush(mode):
        if mode == "read":
            flush_buf.sum()
        else:
            flush_buf.fill_(1.0)

    def median_us(pairs):
        return statistics.median(hip.elapsed_ms(a, b) for a, b in pairs) * 1e3

    for _ in range(args.warmup):
        flush("read")
        step()
    torch.cuda.synchronize()

    # ---- the timed steps: each after a read flush, timed by its own events
    edges = [hip.create(2) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush("read")
        hip.record(edges[i][0], sh)
        step()
        hip.record(edges[i][1], sh)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_times = sorted(hip.elapsed_ms(a, b) * 1e3 for a, b in edges)
    step_us = statistics.median(step_times)
    for e in edges:
        hip.destroy(e)
    print(f"[bench] {args.steps} cold steps timed", file=sys.stderr, flush=True)

    # ---- warm: the same steps back to back, no flush
    warm_edge = hip.create(2)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    hip.record(warm_edge[0], sh)
    for _ in range(args.steps):
        step()
    hip.record(warm_edge[1], sh)
    torch.cuda.synchronize()
    warm_us = hip.elapsed_ms(warm_edge[0], warm_edge[1]) * 1e3 / args.steps
    hip.destroy(warm_edge)

    # ---- stage breakdown (cold steps, an event before every stage; each
    # record adds a little to the stage it opens) and the dirty flush
    stage_med, stage_mean, dirty = {}, {}, {}
    enc_step_us = None
    if cold_steps > 0:
        evs = [hip.create(n_ev) for _ in range(cold_steps)]
        eevs = [hip.create(1) for _ in range(cold_steps)] if args.encode_prefix else None
        for i in range(cold_steps):
            flush("read")
            step(evs[i], eevs[i] if eevs else None)
        torch.cuda.synchronize()
        for j, nm in enumerate(names):
            t = [hip.elapsed_ms(e[j], e[j + 1]) * 1e3 for e in evs]
            stage_med[nm] = statistics.median(t)
            stage_mean[nm] = sum(t) / len(t)
        if eevs:
            enc_step_us = statistics.median(
                hip.elapsed_ms(eevs[i][0], evs[i][0]) * 1e3 for i in range(cold_steps))
        for e in evs + (eevs or []):
            hip.destroy(e)
        dedges = [hip.create(2) for _ in range(cold_steps)]
        for i in range(cold_steps):
            flush("write")
            hip.record(dedges[i][0], sh)
            step()
            hip.record(dedges[i][1], sh)
        torch.cuda.synchronize()
        dirty = {"step_us_median": median_us(dedges)}
        for e in dedges:
            hip.destroy(e)
        print(f"[bench] {cold_steps} staged and dirty-flush steps timed", file=sys.stderr,
              flush=True)
    del flush_buf

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    lens = inp["seq_lens"].cpu().tolist()
    ab = algorithmic_bytes(wl, lens, cfg)
    score_src = [os.path.join(ROOT, "hashed_top_sparse_amd", "csrc", f)
                 for f in ("score_filter.h", "score_keys_log.hip", "score_common.h",
                           "internal.h")]
    # the counters were taken for the key-selecting, log-weight kernel
    traffic = (counter_traffic(source_digest(score_src), wl.name)
               if args.radius_weight == "log" and args.select == "keys" and not args.lsh
               else None)
    roofline = None
    if "score" in stage_mean:
        score_s = stage_mean["score"] * 1e-6
        roofline = {"bound": "hbm", "kernel": "score",
                    "achieved": ab["score"] / score_s / 1e9, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": ab["score"] / score_s / 1e9 / HBM_PEAK_GBS,
                    "traffic": traffic,
                    "algorithmic_bytes_per_launch": ab["score"],
                    "launch_us_mean": stage_mean["score"]}
    step_bytes = ab["total"] + (enc_bytes if args.encode_prefix else 0)
    result = {
        "metric": METRIC,
        "value": ab["keys"] / (step_us * 1e-6),
        "unit": "scored keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_us * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "seq_len": max_len,
                   "q_heads": wl.num_q_heads, "kv_heads": Hkv, "head_dim": wl.head_dim,
                   "code_bits": wl.code_bits, "top_k": wl.top_k, "window": wl.window,
                   "sinks": wl.sinks, "page": PAGE, "radius_weight": args.radius_weight,
                   "select": args.select, "lsh": args.lsh or None,
                   "step": ("encode of every cached key + decode" if args.encode_prefix
                            else "decode with the newest key's encode"),
                   "parallelism": "single GPU"},
        "timing": ("median of K steps, each after a 1 GiB read flush, HIP events "
                   "on the launch stream"),
        "latency_us": step_us,
        "step_us_min": step_times[0],
        "step_us_max": step_times[-1],
        "timed_wall_s": t1 - t0,
        "warm_step_us": warm_us,
        "cold_dirty": dirty,
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_gbs": step_bytes / (step_us * 1e-6) / 1e9,
        "step_frac_of_peak": step_bytes / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "stages_us_median": stage_med,
        "stages_us_mean": stage_mean,
        # the encode of every cached key of the batch, timed once with HIP
        # events: algorithmic bytes (2d bf16 read + b/8 + 1 written per key
        # row) and matrix-core flop (2 d b per key row) over its time
        "prefix_encode": {"us": enc_us, "key_rows": enc_rows,
                          "gbs": enc_bytes / (enc_us * 1e-6) / 1e9,
                          "frac_of_hbm_peak": enc_bytes / (enc_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                          "tflops": enc_flop / (enc_us * 1e-6) / 1e12},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if enc_step_us is not None:
        result["encode_in_step_us_median"] = enc_step_us
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_units, args.cpu_seconds,
                                              cfg.radius_weight, cfg.select_pages,
                                              (cfg.lsh_tables, cfg.lsh_bits),
                                              with_prefix_encode=args.encode_prefix)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
