"""hashed_top_sparse_amd -- Python binding of libdkv (MI355X / gfx950).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of ``libdkv.so``; this module checks tensor dtypes, devices and
shapes, passes ``data_ptr()`` values and the current HIP stream to the C ABI
declared in ``include/dkv.h``, and turns a non-OK status into an exception.
There is no CPU fallback: when the library is not built, importing the
binding's functions raises.

PyTorch only provides device memory and streams.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

__all__ = ["Config", "DkvError", "encode", "decode", "decode_debug",
           "decode_profiled", "decode_append", "decode_append_noalloc",
           "decode_stage_names",
           "decode_workspace_size",
           "library_path", "load_library", "EXPORTED_SYMBOLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdkv.so")
_lib = None

# Every symbol include/dkv.h declares.
EXPORTED_SYMBOLS = ("dkv_encode", "dkv_decode_workspace_size", "dkv_decode",
                    "dkv_decode_debug", "dkv_decode_profiled", "dkv_decode_append",
                    "dkv_decode_num_stages", "dkv_decode_stage_name",
                    "dkv_status_string", "dkv_abi_version", "dkv_lsh_index_size",
                    "dkv_lsh_build", "dkv_decode_lsh", "dkv_decode_append_noalloc")
# bytes of the static scratch array dkv_decode_append_noalloc uses
NOALLOC_SCRATCH_BYTES = 64 << 20
ABI_VERSION = 6
RADIUS_LOG = 0
RADIUS_LINEAR = 1

STATUS = {0: "DKV_OK", 1: "DKV_ERR_INVALID_ARG", 2: "DKV_ERR_UNSUPPORTED",
          3: "DKV_ERR_WORKSPACE", 4: "DKV_ERR_LAUNCH"}


class DkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class _CConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "head_dim", "num_q_heads", "num_kv_heads", "code_bits", "page_size",
        "top_k", "window", "sinks", "radius_weight", "select_pages", "lsh_tables",
        "lsh_bits")]


@dataclasses.dataclass(frozen=True)
class Config:
    num_q_heads: int
    num_kv_heads: int
    code_bits: int
    top_k: int
    window: int
    sinks: int
    head_dim: int = 128
    page_size: int = 16
    # score weight of the radius code: RADIUS_LOG (w = r8) or RADIUS_LINEAR
    # (w = rne(2^(r8/16)))
    radius_weight: int = 0
    # select the top top_k/16 pages (scored by their best candidate key)
    # instead of the top_k keys
    select_pages: bool = False
    # multi-table LSH candidates (decode with decode_lsh): tables and bits
    # per table (0 tables: none)
    lsh_tables: int = 0
    lsh_bits: int = 0

    def _c(self) -> _CConfig:
        return _CConfig(self.head_dim, self.num_q_heads, self.num_kv_heads,
                        self.code_bits, self.page_size, self.top_k, self.window,
                        self.sinks, self.radius_weight, int(self.select_pages),
                        self.lsh_tables, self.lsh_bits)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def select_cap(self) -> int:
        return self.top_k + self.window + self.sinks


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Loads libdkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with "
            "`python -m hashed_top_sparse_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(_CConfig)
    lib.dkv_encode.argtypes = [cfgp, P, i64, P, i32, i32, P, P, i32, P, P, P, P]
    lib.dkv_encode.restype = ctypes.c_int
    lib.dkv_decode_workspace_size.argtypes = [cfgp, i32, i32]
    lib.dkv_decode_workspace_size.restype = sz
    dec = [cfgp, P, P, P, P, P, i64, P, i32, P, i32, i32, P, P, P, P, P, sz]
    lib.dkv_decode.argtypes = dec + [P]
    lib.dkv_decode.restype = ctypes.c_int
    lib.dkv_decode_debug.argtypes = dec + [P, P, P]
    lib.dkv_decode_debug.restype = ctypes.c_int
    lib.dkv_decode_profiled.argtypes = dec + [P, P]
    lib.dkv_decode_profiled.restype = ctypes.c_int
    lib.dkv_decode_append.argtypes = dec + [P, P]
    lib.dkv_decode_append.restype = ctypes.c_int
    lib.dkv_decode_append_noalloc.argtypes = dec[:16] + [P]
    lib.dkv_decode_append_noalloc.restype = ctypes.c_int
    lib.dkv_lsh_index_size.argtypes = [cfgp, i32, i32]
    lib.dkv_lsh_index_size.restype = sz
    lib.dkv_lsh_build.argtypes = [cfgp, P, i64, P, i32, i32, P, i32, P, sz, P]
    lib.dkv_lsh_build.restype = ctypes.c_int
    lib.dkv_decode_lsh.argtypes = dec[:13] + [P, sz] + dec[13:] + [P, P]
    lib.dkv_decode_lsh.restype = ctypes.c_int
    lib.dkv_decode_num_stages.argtypes = []
    lib.dkv_decode_num_stages.restype = i32
    lib.dkv_decode_stage_name.argtypes = [i32]
    lib.dkv_decode_stage_name.restype = ctypes.c_char_p
    lib.dkv_status_string.argtypes = [ctypes.c_int]
    lib.dkv_status_string.restype = ctypes.c_char_p
    lib.dkv_abi_version.argtypes = []
    lib.dkv_abi_version.restype = i32
    if lib.dkv_abi_version() != ABI_VERSION:
        raise ImportError("libdkv.so ABI version mismatch: rebuild it")
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load_library().dkv_status_string(status).decode()
        raise DkvError(status, msg)


def _ptr(t: Optional[torch.Tensor], name: str, dtypes, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


_BF16 = (torch.bfloat16,)
_I32 = (torch.int32,)
_U32 = (torch.int32, torch.uint32)
_U8 = (torch.uint8,)


def _expect(t: torch.Tensor, name: str, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")


def encode(cfg: Config, k_pool, block_table, enc_start, enc_end,
           max_encode_len: int, proj, codes, radii, stream=None) -> None:
    """dkv_encode: codes/radii of tokens [enc_start[s], enc_end[s])."""
    lib = load_library()
    nb = k_pool.shape[0]
    B, max_blocks = block_table.shape
    _expect(k_pool, "k_pool", (nb, cfg.page_size, cfg.num_kv_heads, cfg.head_dim))
    _expect(proj, "proj", (cfg.head_dim, cfg.code_bits))
    _expect(codes, "codes", (nb, cfg.num_kv_heads, cfg.page_size, cfg.code_bits // 32))
    _expect(radii, "radii", (nb, cfg.num_kv_heads, cfg.page_size))
    _expect(enc_start, "enc_start", (B,))
    _expect(enc_end, "enc_end", (B,))
    c = cfg._c()
    _check(lib.dkv_encode(
        ctypes.byref(c), _ptr(k_pool, "k_pool", _BF16), nb,
        _ptr(block_table, "block_table", _I32), max_blocks, B,
        _ptr(enc_start, "enc_start", _I32), _ptr(enc_end, "enc_end", _I32),
        int(max_encode_len), _ptr(proj, "proj", _BF16),
        _ptr(codes, "codes", _U32), _ptr(radii, "radii", _U8), _stream(stream)))


def decode_workspace_size(cfg: Config, batch: int, max_seq_len: int) -> int:
    lib = load_library()
    c = cfg._c()
    n = lib.dkv_decode_workspace_size(ctypes.byref(c), int(batch), int(max_seq_len))
    if n == 0:
        raise DkvError(1, "invalid configuration for the workspace size")
    return int(n)


def _decode_args(cfg, q, k_pool, v_pool, codes, radii, block_table, seq_lens,
                 max_seq_len, proj, out, workspace, sel_idx, sel_cnt):
    nb = k_pool.shape[0]
    B, max_blocks = block_table.shape
    Hq, Hkv, d, b = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.code_bits
    _expect(q, "q", (B, Hq, d))
    _expect(k_pool, "k_pool", (nb, cfg.page_size, Hkv, d))
    _expect(v_pool, "v_pool", (nb, cfg.page_size, Hkv, d))
    _expect(codes, "codes", (nb, Hkv, cfg.page_size, b // 32))
    _expect(radii, "radii", (nb, Hkv, cfg.page_size))
    _expect(seq_lens, "seq_lens", (B,))
    _expect(proj, "proj", (d, b))
    _expect(out, "out", (B, Hq, d))
    if sel_idx is not None:
        _expect(sel_idx, "sel_idx", (B, Hkv, cfg.select_cap))
    if sel_cnt is not None:
        _expect(sel_cnt, "sel_cnt", (B, Hkv))
    c = cfg._c()
    args = [
        ctypes.byref(c), _ptr(q, "q", _BF16), _ptr(k_pool, "k_pool", _BF16),
        _ptr(v_pool, "v_pool", _BF16), _ptr(codes, "codes", _U32),
        _ptr(radii, "radii", _U8), nb, _ptr(block_table, "block_table", _I32),
        max_blocks, _ptr(seq_lens, "seq_lens", _I32), B, int(max_seq_len),
        _ptr(proj, "proj", _BF16), _ptr(out, "out", (torch.float32,)),
        _ptr(sel_idx, "sel_idx", _I32), _ptr(sel_cnt, "sel_cnt", _I32)]
    if workspace is None:     # dkv_decode_append_noalloc: no workspace arguments
        return c, args
    if workspace.dtype not in (torch.uint8, torch.int8):
        raise TypeError("workspace must be a uint8/int8 tensor")
    return c, args + [_ptr(workspace, "workspace", (torch.uint8, torch.int8)),
                      workspace.numel() * workspace.element_size()]


def decode(cfg: Config, q, k_pool, v_pool, codes, radii, block_table, seq_lens,
           max_seq_len: int, proj, out, workspace, sel_idx=None, sel_cnt=None,
           stream=None) -> None:
    """dkv_decode: one decode step; writes ``out`` (and the optional lists)."""
    lib = load_library()
    c, args = _decode_args(cfg, q, k_pool, v_pool, codes, radii, block_table,
                           seq_lens, max_seq_len, proj, out, workspace, sel_idx,
                           sel_cnt)
    _check(lib.dkv_decode(*args, _stream(stream)))


def decode_debug(cfg: Config, q, k_pool, v_pool, codes, radii, block_table,
                 seq_lens, max_seq_len: int, proj, out, workspace, sel_idx=None,
                 sel_cnt=None, q8_out=None, scores_out=None, stream=None) -> None:
    """dkv_decode_debug: dkv_decode plus the query codes and all scores."""
    lib = load_library()
    B = block_table.shape[0]
    if q8_out is not None:
        _expect(q8_out, "q8_out", (B, cfg.num_q_heads, cfg.code_bits))
    if scores_out is not None:
        _expect(scores_out, "scores_out", (B, cfg.num_kv_heads, max_seq_len))
    c, args = _decode_args(cfg, q, k_pool, v_pool, codes, radii, block_table,
                           seq_lens, max_seq_len, proj, out, workspace, sel_idx,
                           sel_cnt)
    _check(lib.dkv_decode_debug(*args, _ptr(q8_out, "q8_out", (torch.int8,)),
                                _ptr(scores_out, "scores_out", _I32),
                                _stream(stream)))


def decode_append(cfg: Config, q, k_pool, v_pool, codes, radii, block_table,
                  seq_lens, max_seq_len: int, proj, out, workspace, sel_idx=None,
                  sel_cnt=None, events=None, stream=None) -> None:
    """dkv_decode_append: encode every sequence's newest key (position
    seq_lens-1) into ``codes``/``radii``, then one decode step.  ``events``:
    optional num_stages+1 hipEvent_t handles, as for decode_profiled."""
    lib = load_library()
    arr = None
    if events is not None:
        n = lib.dkv_decode_num_stages()
        if len(events) < n + 1:
            raise ValueError(f"need {n + 1} events, got {len(events)}")
        arr = (ctypes.c_void_p * len(events))(*events)
    c, args = _decode_args(cfg, q, k_pool, v_pool, codes, radii, block_table,
                           seq_lens, max_seq_len, proj, out, workspace, sel_idx,
                           sel_cnt)
    _check(lib.dkv_decode_append(
        *args, ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None,
        _stream(stream)))


def decode_append_noalloc(cfg: Config, q, k_pool, v_pool, codes, radii, block_table,
                          seq_lens, max_seq_len: int, proj, out, sel_idx=None,
                          sel_cnt=None, stream=None) -> None:
    """dkv_decode_append_noalloc: decode_append whose workspace is the
    library's static per-GPU scratch array (no allocation in the call;
    calls that overlap on one GPU race)."""
    lib = load_library()
    c, args = _decode_args(cfg, q, k_pool, v_pool, codes, radii, block_table,
                           seq_lens, max_seq_len, proj, out, None, sel_idx, sel_cnt)
    _check(lib.dkv_decode_append_noalloc(*args, _stream(stream)))


def lsh_index_size(cfg: Config, batch: int, max_seq_len: int) -> int:
    """Bytes of the LSH index (dkv_lsh_index_size)."""
    lib = load_library()
    c = cfg._c()
    n = lib.dkv_lsh_index_size(ctypes.byref(c), int(batch), int(max_seq_len))
    if n == 0:
        raise DkvError(1, "invalid configuration for an LSH index")
    return int(n)


def lsh_build(cfg: Config, codes, block_table, seq_lens, max_seq_len: int, index,
              stream=None) -> None:
    """dkv_lsh_build: bucket index of positions [0, seq_lens) of every sequence."""
    lib = load_library()
    nb = codes.shape[0]
    B, max_blocks = block_table.shape
    _expect(codes, "codes", (nb, cfg.num_kv_heads, cfg.page_size, cfg.code_bits // 32))
    _expect(seq_lens, "seq_lens", (B,))
    if index.dtype not in (torch.uint8, torch.int8):
        raise TypeError("index must be a uint8/int8 tensor")
    c = cfg._c()
    _check(lib.dkv_lsh_build(
        ctypes.byref(c), _ptr(codes, "codes", _U32), nb,
        _ptr(block_table, "block_table", _I32), max_blocks, B,
        _ptr(seq_lens, "seq_lens", _I32), int(max_seq_len),
        _ptr(index, "index", (torch.uint8, torch.int8)), index.numel(), _stream(stream)))


def decode_lsh(cfg: Config, q, k_pool, v_pool, codes, radii, block_table, seq_lens,
               max_seq_len: int, proj, index, out, workspace, sel_idx=None,
               sel_cnt=None, events=None, stream=None) -> None:
    """dkv_decode_lsh: one decode step whose top-k runs over the LSH
    candidates found through ``index`` (built by lsh_build)."""
    lib = load_library()
    arr = None
    if events is not None:
        n = lib.dkv_decode_num_stages()
        if len(events) < n + 1:
            raise ValueError(f"need {n + 1} events, got {len(events)}")
        arr = (ctypes.c_void_p * len(events))(*events)
    c, args = _decode_args(cfg, q, k_pool, v_pool, codes, radii, block_table,
                           seq_lens, max_seq_len, proj, out, workspace, sel_idx,
                           sel_cnt)
    if index.dtype not in (torch.uint8, torch.int8):
        raise TypeError("index must be a uint8/int8 tensor")
    args = args[:13] + [_ptr(index, "index", (torch.uint8, torch.int8)), index.numel()] + \
        args[13:]
    _check(lib.dkv_decode_lsh(
        *args, ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None,
        _stream(stream)))


def decode_stage_names():
    """Names of the decode stages dkv_decode_profiled brackets with events."""
    lib = load_library()
    return [lib.dkv_decode_stage_name(i).decode() for i in range(lib.dkv_decode_num_stages())]


def decode_profiled(cfg: Config, q, k_pool, v_pool, codes, radii, block_table,
                    seq_lens, max_seq_len: int, proj, out, workspace, events,
                    sel_idx=None, sel_cnt=None, stream=None) -> None:
    """dkv_decode_profiled: ``events`` holds num_stages+1 hipEvent_t handles
    (ints) that the library records before each stage and after the last."""
    lib = load_library()
    n = lib.dkv_decode_num_stages()
    if len(events) < n + 1:
        raise ValueError(f"need {n + 1} events, got {len(events)}")
    arr = (ctypes.c_void_p * len(events))(*events)
    c, args = _decode_args(cfg, q, k_pool, v_pool, codes, radii, block_table,
                           seq_lens, max_seq_len, proj, out, workspace, sel_idx,
                           sel_cnt)
    _check(lib.dkv_decode_profiled(*args, ctypes.cast(arr, ctypes.c_void_p),
                                   _stream(stream)))
