"""CPU oracle for score-then-select sparse decode attention.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg are the only callers.  The GPU library
(``hashed_top_sparse_amd``) never imports this package and this package never
imports it; they share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64, index-order sums, a full
sort for the top-k); this module only marshals numpy arrays to it.  bf16
values travel as ``uint16`` bit patterns.  Per-function citations are in the
C source.

Parity status of each function (what pins it is listed in the tests):
  key_code / encode_keys   pinned (closed forms, exact-rational brute force)
  radius_code              pinned (closed form, exact-rational constants)
  query_int8               pinned (textbook symmetric int8 properties,
                           exact-rational rounding bound)
  radius_weight            pinned (mode 1: 60-digit decimal 2^(r/16) rounded,
                           exact powers of two at r = 16m, monotone)
  score                    pinned (Python-integer brute force, identities)
  select                   pinned (brute-force sort, special cases)
  select_pages             pinned (brute-force page sort, equals select when
                           scores are constant on aligned pages, limits)
  lsh_bucket, select_lsh   pinned (Python bit extraction and brute-force
                           candidate sort; all-candidate case equals select)
  attend                   pinned (dense softmax attention special case,
                           single-key and identical-key closed forms)
  decode_unit(s)           composition of the above; whole-pipeline values
                           are otherwise parity unpinned (the pages print no
                           worked example)
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.orc_key_code.argtypes = [P, P, i32, i32, P]
    lib.orc_key_code.restype = None
    lib.orc_radius_threshold.argtypes = [i32]
    lib.orc_radius_threshold.restype = f64
    lib.orc_sq_norm.argtypes = [P, i32]
    lib.orc_sq_norm.restype = f64
    lib.orc_radius_code.argtypes = [f64]
    lib.orc_radius_code.restype = i32
    lib.orc_encode_keys.argtypes = [i64, i32, i32, P, P, P, P]
    lib.orc_encode_keys.restype = None
    lib.orc_query_int8.argtypes = [P, i32, P, i32, i32, P]
    lib.orc_query_int8.restype = None
    lib.orc_radius_weight.argtypes = [i32, i32]
    lib.orc_radius_weight.restype = ctypes.c_int32
    lib.orc_score.argtypes = [P, i32, i32, P, ctypes.c_int32]
    lib.orc_score.restype = ctypes.c_int32
    lib.orc_select.argtypes = [P, i32, i32, i32, i32, P]
    lib.orc_select.restype = i32
    lib.orc_select_pages.argtypes = [P, i32, i32, i32, i32, P]
    lib.orc_select_pages.restype = i32
    lib.orc_lsh_bucket.argtypes = [P, i32, i32]
    lib.orc_lsh_bucket.restype = i32
    lib.orc_select_lsh.argtypes = [P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, P]
    lib.orc_select_lsh.restype = i32
    lib.orc_attend.argtypes = [P, i32, P, P, i32, P, i32, P]
    lib.orc_attend.restype = None
    lib.orc_decode_unit.argtypes = [i32] * 10 + [P] * 6 + [i32] + [P] * 4
    lib.orc_decode_unit.restype = i32
    lib.orc_decode_units.argtypes = [i32] * 11 + [P] * 7 + [i32, P, P, P, i32, P, P]
    lib.orc_decode_units.restype = None
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = i32
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def radius_threshold(m: int) -> float:
    return float(_load().orc_radius_threshold(int(m)))


def radius_code(r2: float) -> int:
    return int(_load().orc_radius_code(float(r2)))


def sq_norm(k: np.ndarray) -> float:
    k = _c(k, np.uint16)
    return float(_load().orc_sq_norm(_p(k), k.shape[-1]))


def key_code(k: np.ndarray, P: np.ndarray) -> np.ndarray:
    """E1 for one key row k [d] (bf16 bits) and P [d][b] -> uint32 [b/32]."""
    k = _c(k, np.uint16)
    P = _c(P, np.uint16)
    d, b = P.shape
    out = np.zeros(b // 32, np.uint32)
    _load().orc_key_code(_p(k), _p(P), d, b, _p(out))
    return out


def encode_keys(K: np.ndarray, P: np.ndarray):
    """E1+E2 for rows K [n][d] -> (codes uint32 [n][b/32], radii uint8 [n])."""
    K = _c(K, np.uint16)
    P = _c(P, np.uint16)
    d, b = P.shape
    n = K.shape[0]
    codes = np.zeros((n, b // 32), np.uint32)
    radii = np.zeros(n, np.uint8)
    _load().orc_encode_keys(n, d, b, _p(K), _p(P), _p(codes), _p(radii))
    return codes, radii


def query_int8(q: np.ndarray, P: np.ndarray) -> np.ndarray:
    """Q1 for one KV group: q [G][d] (bf16 bits) -> int8 [G][b]."""
    q = _c(q, np.uint16)
    P = _c(P, np.uint16)
    G, d = q.shape
    b = P.shape[1]
    out = np.zeros((G, b), np.int8)
    _load().orc_query_int8(_p(q), G, _p(P), d, b, _p(out))
    return out


def radius_weight(r8: int, mode: int = 0) -> int:
    """W1: the score weight of radius code r8 (mode 0: r8; mode 1: linear)."""
    return int(_load().orc_radius_weight(int(r8), int(mode)))


def score(q8: np.ndarray, code: np.ndarray, wgt: int) -> int:
    """S1 for one key: q8 [G][b], code uint32 [b/32], radius weight -> int."""
    q8 = _c(q8, np.int8)
    code = _c(code, np.uint32)
    G, b = q8.shape
    return int(_load().orc_score(_p(q8), G, b, _p(code), int(wgt)))


def scores(q8: np.ndarray, codes: np.ndarray, radii: np.ndarray,
           radius_mode: int = 0) -> np.ndarray:
    """S1 for every key: codes [N][b/32], radii [N] -> int32 [N]."""
    lib = _load()
    q8 = _c(q8, np.int8)
    codes = _c(codes, np.uint32)
    G, b = q8.shape
    out = np.empty(codes.shape[0], np.int32)
    for i in range(codes.shape[0]):
        wgt = lib.orc_radius_weight(int(radii[i]), int(radius_mode))
        out[i] = lib.orc_score(_p(q8), G, b, _p(codes[i]), wgt)
    return out


def select(S: np.ndarray, k: int, w: int, sigma: int) -> np.ndarray:
    """T1 over scores S [N] -> int32 positions (sinks, window, top-k)."""
    S = _c(S, np.int32)
    N = S.shape[0]
    cap = max(1, min(N, sigma + w + k))
    sel = np.full(cap, -1, np.int32)
    n = _load().orc_select(_p(S), N, k, w, sigma, _p(sel))
    return sel[:n].copy()


def select_pages(S: np.ndarray, k: int, w: int, sigma: int) -> np.ndarray:
    """T2 over scores S [N] -> int32 positions (sinks, window, top pages)."""
    S = _c(S, np.int32)
    N = S.shape[0]
    cap = max(1, min(N, sigma + w + k))
    sel = np.full(cap, -1, np.int32)
    n = _load().orc_select_pages(_p(S), N, k, w, sigma, _p(sel))
    return sel[:n].copy()


def lsh_bucket(code: np.ndarray, t: int, m: int) -> int:
    """H1: bucket of code (uint32 [W]) in table t of m bits."""
    code = _c(code, np.uint32)
    return int(_load().orc_lsh_bucket(_p(code), int(t), int(m)))


def select_lsh(S: np.ndarray, codes: np.ndarray, qbits: np.ndarray, T: int, m: int,
               k: int, w: int, sigma: int) -> np.ndarray:
    """T3 over scores S [N], codes [N][W], query bits [G][W] -> positions."""
    S = _c(S, np.int32)
    codes = _c(codes, np.uint32)
    qbits = _c(qbits, np.uint32)
    N, W = codes.shape
    G = qbits.shape[0]
    cap = max(1, min(N, sigma + w + k))
    sel = np.full(cap, -1, np.int32)
    n = _load().orc_select_lsh(_p(S), _p(codes), W, _p(qbits), G, T, m, N, k, w, sigma,
                               _p(sel))
    return sel[:n].copy()


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, sel: np.ndarray) -> np.ndarray:
    """A1: q [G][d], K/V [N][d] (bf16 bits), sel positions -> fp64 [G][d]."""
    q = _c(q, np.uint16)
    K = _c(K, np.uint16)
    V = _c(V, np.uint16)
    sel = _c(sel, np.int32)
    G, d = q.shape
    out = np.zeros((G, d), np.float64)
    _load().orc_attend(_p(q), G, _p(K), _p(V), d, _p(sel), sel.shape[0], _p(out))
    return out


def decode_unit(q, P, codes, radii, K, V, k: int, w: int, sigma: int,
                radius_mode: int = 0, pages: bool = False, lsh=(0, 0)):
    """One (sequence, KV head) decode step.

    q [G][d]; P [d][b]; codes [N][b/32]; radii [N]; K, V [N][d] (logical
    order).  Returns dict(q8, scores, sel, out)."""
    q = _c(q, np.uint16)
    P = _c(P, np.uint16)
    codes = _c(codes, np.uint32)
    radii = _c(radii, np.uint8)
    K = _c(K, np.uint16)
    V = _c(V, np.uint16)
    G, d = q.shape
    b = P.shape[1]
    N = K.shape[0]
    q8 = np.zeros((G, b), np.int8)
    S = np.zeros(max(N, 1), np.int32)
    cap = max(1, min(N, sigma + w + k))
    sel = np.full(cap, -1, np.int32)
    out = np.zeros((G, d), np.float64)
    n = _load().orc_decode_unit(G, d, b, k, w, sigma, radius_mode, int(pages),
                                int(lsh[0]), int(lsh[1]), _p(q), _p(P),
                                _p(codes),
                                _p(radii), _p(K), _p(V), N, _p(q8), _p(S),
                                _p(sel), _p(out))
    return {"q8": q8, "scores": S[:N].copy(), "sel": sel[:n].copy(), "out": out}


def decode_units(q, P, codes, radii, K, V, N, k: int, w: int, sigma: int,
                 want_scores: bool = True, radius_mode: int = 0, pages: bool = False,
                 lsh=(0, 0)):
    """Many units at once (OpenMP over units).

    q [U][G][d]; codes [U][Nmax][b/32]; radii [U][Nmax]; K, V [U][Nmax][d];
    N [U].  Returns dict(q8 [U][G][b], scores [U][Nmax] or None,
    sel list of arrays, out [U][G][d])."""
    q = _c(q, np.uint16)
    P = _c(P, np.uint16)
    codes = _c(codes, np.uint32)
    radii = _c(radii, np.uint8)
    K = _c(K, np.uint16)
    V = _c(V, np.uint16)
    N = _c(N, np.int32)
    U, G, d = q.shape
    b = P.shape[1]
    Nmax = K.shape[1]
    cap = max(1, sigma + w + k)
    q8 = np.zeros((U, G, b), np.int8)
    S = np.zeros((U, Nmax), np.int32) if want_scores else None
    sel = np.full((U, cap), -1, np.int32)
    cnt = np.zeros(U, np.int32)
    out = np.zeros((U, G, d), np.float64)
    _load().orc_decode_units(U, G, d, b, k, w, sigma, radius_mode, int(pages),
                             int(lsh[0]), int(lsh[1]), _p(q), _p(P),
                             _p(codes),
                             _p(radii), _p(K), _p(V), _p(N), Nmax, _p(q8),
                             _p(S) if S is not None else None, _p(sel), cap,
                             _p(cnt), _p(out))
    return {"q8": q8, "scores": S, "sel": [sel[u, :cnt[u]].copy() for u in range(U)],
            "out": out}
