"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any launch (no GPU needed: every call below
fails validation, so no kernel is ever enqueued)."""
import ctypes
import os
import re

import pytest

import hashed_top_sparse_amd as dkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dkv.h")
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dkv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = dkv.load_library()
    names = declared_functions()
    assert set(names) == set(dkv.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.dkv_abi_version() == dkv.ABI_VERSION


def test_config_struct_matches_header():
    """The binding's dkv_config fields are the header's, in order."""
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} dkv_config;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"int32_t\s+(\w+)\s*;", body)
    assert fields == [f for f, _ in dkv._CConfig._fields_]


def test_status_strings():
    lib = dkv.load_library()
    for code, name in dkv.STATUS.items():
        assert lib.dkv_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.dkv_status_string(99)


def _cfg(**over):
    kw = dict(head_dim=128, num_q_heads=32, num_kv_heads=8, code_bits=128,
              page_size=16, top_k=64, window=16, sinks=4, radius_weight=0,
              select_pages=0, lsh_tables=0, lsh_bits=0)
    kw.update(over)
    return dkv._CConfig(*[kw[f] for f, _ in dkv._CConfig._fields_])


def _decode(cfg, ws_bytes=1 << 30, workspace=FAKE, q=FAKE, batch=2, max_seq_len=1000,
            num_blocks=200, max_blocks=64):
    lib = dkv.load_library()
    c = cfg
    return lib.dkv_decode(ctypes.byref(c) if c is not None else None, q, FAKE, FAKE,
                          FAKE, FAKE, num_blocks, FAKE, max_blocks, FAKE, batch,
                          max_seq_len, FAKE, FAKE, None, None, workspace, ws_bytes, None)


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=64), 2), (dict(code_bits=96), 2), (dict(code_bits=512), 2),
    (dict(page_size=32), 2), (dict(num_q_heads=24, num_kv_heads=8), 2),  # G = 3
    (dict(num_q_heads=30, num_kv_heads=8), 1), (dict(top_k=-1), 1),
    (dict(window=-5), 1), (dict(sinks=-1), 1), (dict(num_kv_heads=0), 1),
    (dict(top_k=1 << 20), 2), (dict(radius_weight=2), 2), (dict(radius_weight=-1), 2),
    (dict(select_pages=2), 2), (dict(select_pages=-1), 2),
    (dict(lsh_tables=-1), 2), (dict(lsh_tables=4, lsh_bits=13), 2),
    (dict(lsh_tables=4, lsh_bits=0), 2), (dict(lsh_tables=17, lsh_bits=8), 2),  # 136 > b
    (dict(lsh_tables=4, lsh_bits=8, select_pages=1), 2),
    (dict(lsh_tables=4, lsh_bits=8), 1),   # an LSH config needs dkv_decode_lsh
])
def test_decode_rejects_bad_config(over, status):
    assert _decode(_cfg(**over)) == status


def test_decode_rejects_bad_arguments():
    assert _decode(None) == 1
    assert _decode(_cfg(), q=None) == 1
    assert _decode(_cfg(), batch=0) == 1
    assert _decode(_cfg(), max_seq_len=-1) == 1
    assert _decode(_cfg(), num_blocks=0) == 1
    assert _decode(_cfg(), max_blocks=0) == 1
    assert _decode(_cfg(), max_seq_len=(1 << 24) + 1) == 2
    assert _decode(_cfg(), workspace=None) == 3
    assert _decode(_cfg(), ws_bytes=16) == 3
    assert _decode(_cfg(), workspace=ctypes.c_void_p(0x10004)) == 3   # misaligned
    assert _decode(_cfg(), q=ctypes.c_void_p(0x10008)) == 1           # q not 16-byte aligned


def test_decode_append_rejects_bad_arguments():
    lib = dkv.load_library()
    c = _cfg()
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 200, FAKE, 64, FAKE, 2, 1000, FAKE,
            FAKE, None, None, FAKE, 1 << 30]
    assert lib.dkv_decode_append(None, *args, None, None) == 1
    a2 = list(args)
    a2[0] = None       # q
    assert lib.dkv_decode_append(ctypes.byref(c), *a2, None, None) == 1
    a3 = list(args)
    a3[3] = ctypes.c_void_p(0x10004)   # codes not 16-byte aligned
    assert lib.dkv_decode_append(ctypes.byref(c), *a3, None, None) == 1
    events = (ctypes.c_void_p * 8)(*([0x1000] * 3 + [0] * 5))   # a null event
    assert lib.dkv_decode_append(ctypes.byref(c), *args,
                                 ctypes.cast(events, ctypes.c_void_p), None) == 1


def test_workspace_size():
    lib = dkv.load_library()
    c = _cfg()
    a = lib.dkv_decode_workspace_size(ctypes.byref(c), 4, 4096)
    b = lib.dkv_decode_workspace_size(ctypes.byref(c), 4, 65536)
    assert 0 < a < b and a % 256 == 0
    bad = _cfg(code_bits=7)
    assert lib.dkv_decode_workspace_size(ctypes.byref(bad), 4, 4096) == 0
    assert lib.dkv_decode_workspace_size(ctypes.byref(c), 0, 4096) == 0


def test_encode_rejects_bad_arguments():
    lib = dkv.load_library()
    c = _cfg()
    args = [FAKE, 100, FAKE, 8, 2, FAKE, FAKE, 128, FAKE, FAKE, FAKE, None]
    assert lib.dkv_encode(None, *args) == 1
    bad = _cfg(code_bits=100)
    assert lib.dkv_encode(ctypes.byref(bad), *args) == 2
    a2 = list(args)
    a2[1] = 0          # num_blocks
    assert lib.dkv_encode(ctypes.byref(c), *a2) == 1
    a3 = list(args)
    a3[7] = -1         # max_encode_len
    assert lib.dkv_encode(ctypes.byref(c), *a3) == 1
    a4 = list(args)
    a4[0] = None       # k_pool
    assert lib.dkv_encode(ctypes.byref(c), *a4) == 1
    a6 = list(args)
    a6[3] = (1 << 20) + 1   # max_blocks_per_seq: positions past DKV_MAX_SEQ_LEN
    assert lib.dkv_encode(ctypes.byref(c), *a6) == 2
    a6[3] = 1 << 20         # the largest accepted; still fails later (null range ptr)
    a6[5] = None
    assert lib.dkv_encode(ctypes.byref(c), *a6) == 1
    for i in (0, 8, 9, 10):  # k_pool, proj, codes, radii not 16-byte aligned
        a5 = list(args)
        a5[i] = ctypes.c_void_p(0x10002)
        assert lib.dkv_encode(ctypes.byref(c), *a5) == 1


def test_python_binding_refuses_host_tensors():
    import torch
    cfg = dkv.Config(num_q_heads=1, num_kv_heads=1, code_bits=64, top_k=4,
                     window=4, sinks=1)
    kp = torch.zeros((2, 16, 1, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dkv.encode(cfg, kp, torch.zeros((1, 2), dtype=torch.int32),
                   torch.zeros(1, dtype=torch.int32), torch.ones(1, dtype=torch.int32),
                   1, torch.zeros((128, 64), dtype=torch.bfloat16),
                   torch.zeros((2, 1, 2, 16), dtype=torch.int32),
                   torch.zeros((2, 1, 16), dtype=torch.uint8), stream=0)


def test_lsh_entry_points_reject_bad_arguments():
    lib = dkv.load_library()
    c = _cfg(lsh_tables=4, lsh_bits=8)
    size = lib.dkv_lsh_index_size(ctypes.byref(c), 2, 1000)
    assert size > 0
    assert lib.dkv_lsh_index_size(ctypes.byref(_cfg()), 2, 1000) == 0       # no tables
    assert lib.dkv_lsh_index_size(ctypes.byref(c), 2, (1 << 19) + 1) == 0   # too long
    build = lambda cfg, **kw: lib.dkv_lsh_build(
        ctypes.byref(cfg), kw.get("codes", FAKE), 200, FAKE, 64, 2, FAKE,
        kw.get("max_seq_len", 1000), kw.get("index", FAKE), kw.get("bytes", size), None)
    assert build(_cfg()) == 1                                  # config without tables
    assert build(c, codes=None) == 1
    assert build(c, bytes=size - 1) == 3
    assert build(c, index=ctypes.c_void_p(0x10010)) == 3       # misaligned index
    assert build(c, max_seq_len=(1 << 19) + 1) == 2

    def dec(cfg, index=FAKE, nbytes=size, max_seq_len=1000):
        return lib.dkv_decode_lsh(ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, FAKE, 200, FAKE,
                                  64, FAKE, 2, max_seq_len, FAKE, index, nbytes, FAKE, None,
                                  None, FAKE, 1 << 30, None, None)
    assert dec(c, index=None) == 1
    assert dec(_cfg()) == 1                                    # index without tables
    assert dec(c, nbytes=size - 1) == 3
    assert dec(c, max_seq_len=(1 << 19) + 1) == 2


def test_noalloc_entry_point_rejects_before_any_launch():
    """dkv_decode_append_noalloc checks the step's workspace need against its
    static scratch before it touches the device, and validates pointers."""
    lib = dkv.load_library()
    c = _cfg()

    def call(cfg, batch, max_seq_len, q=FAKE, num_blocks=200, max_blocks=64):
        return lib.dkv_decode_append_noalloc(
            ctypes.byref(cfg) if cfg is not None else None, q, FAKE, FAKE, FAKE, FAKE,
            num_blocks, FAKE, max_blocks, FAKE, batch, max_seq_len, FAKE, FAKE, None,
            None, None)
    need = lib.dkv_decode_workspace_size(ctypes.byref(c), 16, 131072)
    assert need > dkv.NOALLOC_SCRATCH_BYTES
    assert call(c, 16, 131072, num_blocks=16 * 8192, max_blocks=8192) == 3
    assert lib.dkv_decode_workspace_size(ctypes.byref(c), 2, 1000) <= dkv.NOALLOC_SCRATCH_BYTES
    assert call(c, 2, 1000, q=None) == 1
    assert call(None, 2, 1000) == 1
    assert call(_cfg(lsh_tables=4, lsh_bits=8), 2, 1000) == 1
    assert call(_cfg(code_bits=96), 2, 1000) == 2


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define DKV_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == dkv.NOALLOC_SCRATCH_BYTES
