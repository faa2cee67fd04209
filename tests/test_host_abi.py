"""The C-ABI library on the host, without a GPU: it loads, exports every entry point that
include/gva.h (and the measurement aid in include/gva_diag.h) declares, rejects bad arguments before any launch, plans splits, and fills a RoPE
table bit-identical to the oracle's. None of these tests launches a kernel."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import gva_oracle as O
from value_only_kv_amd import binding as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gva.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "gva_diag.h")]


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gb.LIB_PATH):
        from value_only_kv_amd import _build
        _build.build()
    return gb.lib()


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(gva_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert len(declared) >= 11
    out = subprocess.run(["nm", "-D", "--defined-only", gb.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(gva_\w+)", out))
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    assert sorted(gb.EXPORTED) == declared
    for f in declared:
        assert hasattr(L, f)


def test_version_and_status_strings(L):
    assert "gfx950" in gb.gva_version()
    for s, name in enumerate(["GVA_OK", "GVA_ERR_INVALID_ARG", "GVA_ERR_UNSUPPORTED",
                              "GVA_ERR_WORKSPACE", "GVA_ERR_HIP"]):
        assert L.gva_status_string(s).decode() == name


@pytest.mark.parametrize("max_pos,d_r", [(1, 2), (300, 16), (1025, 24), (77, 64), (40, 128)])
def test_rope_table_bit_identical_to_oracle(L, max_pos, d_r):
    lib_tab = gb.gva_rope_table_fill(max_pos, d_r, 10000.0)
    ora_tab = O.rope_table(max_pos, d_r, 10000.0)
    assert lib_tab.tobytes() == ora_tab.tobytes()
    assert gb.gva_rope_table_bytes(max_pos, d_r) == ora_tab.nbytes


def test_rope_table_rejects_bad_arguments(L):
    buf = np.empty(64, dtype=np.float64)
    for args in [(0, 16, 1e4), (4, 3, 1e4), (4, 0, 1e4), (4, 514, 1e4), (4, 16, -1.0),
                 (4, 16, float("inf"))]:
        assert L.gva_rope_table_fill(buf.ctypes.data, *args) == gb.GVA_ERR_INVALID_ARG
    assert L.gva_rope_table_fill(None, 4, 16, 1e4) == gb.GVA_ERR_INVALID_ARG
    assert gb.gva_rope_table_bytes(0, 16) == 0 and gb.gva_rope_table_bytes(4, 5) == 0
    assert gb.gva_rope_table_bytes(4, 128) == 4 * 64 * 2 * 8     # a key-wide table (d_n = 128)


# ---- validation, with fake (never dereferenced) device addresses ----------------------------

A = 1 << 20  # an aligned fake address


def _dims(H=32, G=8, d_h=128, d_n=128, d_r=16):
    return gb.GvaDims(H, G, d_h, d_n, d_r)


def _cache(dtype=gb.GVA_DTYPE_BF16, bs=16, max_blocks=8, num_blocks=64, d=None, **kw):
    d = d or _dims()
    s = gb.GvaCacheStruct()
    s.dtype = dtype
    s.v, s.kr = A, A + 4096
    s.v_stride_block = d.G * bs * d.d_h
    s.v_stride_token = d.d_h
    s.v_stride_group = bs * d.d_h
    s.kr_stride_block = bs * d.d_r
    s.kr_stride_token = d.d_r
    s.num_blocks, s.block_size, s.max_blocks = num_blocks, bs, max_blocks
    s.block_table, s.rope, s.max_pos, s.err_flag = A + 8192, A + 16384, 1024, None
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def _decode(L, d, c, B=2, seq_len=A, max_len=100, q_abs=A, scale=0.1, S=0, kernel=0, ws=None,
            ws_bytes=0, out=A, lse=None):
    return L.gva_decode(ctypes.byref(d), ctypes.byref(c), B, seq_len, max_len, q_abs, scale, S,
                        kernel, ws, ws_bytes, out, lse, None)


@pytest.mark.parametrize("bad", [
    dict(H=0), dict(H=257), dict(G=0), dict(G=5), dict(H=12, G=8), dict(d_h=0), dict(d_h=7),
    dict(d_h=258), dict(d_n=0), dict(d_n=513), dict(d_r=0), dict(d_r=3), dict(d_r=66),
])
def test_decode_rejects_bad_dims(L, bad):
    kw = dict(H=32, G=8, d_h=128, d_n=128, d_r=16)
    kw.update(bad)
    d = gb.GvaDims(**kw)
    assert _decode(L, d, _cache()) == gb.GVA_ERR_INVALID_ARG
    assert L.gva_last_error().decode() != ""


@pytest.mark.parametrize("field,value", [
    ("dtype", 7), ("v", None), ("kr", None), ("v", A + 2), ("kr", A + 8), ("block_table", None),
    ("rope", None), ("rope", A + 8), ("max_pos", 0), ("num_blocks", 0), ("block_size", 12),
    ("block_size", 0), ("max_blocks", 0), ("v_stride_token", -8), ("kr_stride_token", 3),
    ("kr_stride_token", 8), ("num_blocks", 1 << 40),
])
def test_decode_rejects_bad_cache(L, field, value):
    assert _decode(L, _dims(), _cache(**{field: value})) == gb.GVA_ERR_INVALID_ARG


def test_decode_rejects_bad_call_arguments(L):
    d, c = _dims(), _cache()
    assert _decode(L, d, c, B=0) == gb.GVA_ERR_INVALID_ARG
    assert _decode(L, d, c, seq_len=None) == gb.GVA_ERR_INVALID_ARG
    assert _decode(L, d, c, q_abs=None) == gb.GVA_ERR_INVALID_ARG
    assert _decode(L, d, c, q_abs=A + 4) == gb.GVA_ERR_INVALID_ARG
    assert _decode(L, d, c, out=None) == gb.GVA_ERR_INVALID_ARG
    assert _decode(L, d, c, max_len=-1) == gb.GVA_ERR_INVALID_ARG
    assert _decode(L, d, c, max_len=8 * 16 + 1) == gb.GVA_ERR_INVALID_ARG  # beyond capacity
    assert _decode(L, d, c, scale=0.0) == gb.GVA_ERR_INVALID_ARG
    assert _decode(L, d, c, scale=float("nan")) == gb.GVA_ERR_INVALID_ARG
    assert _decode(L, d, c, S=-1) == gb.GVA_ERR_INVALID_ARG
    assert _decode(L, d, c, S=1025) == gb.GVA_ERR_INVALID_ARG
    assert _decode(L, d, c, kernel=3) == gb.GVA_ERR_INVALID_ARG


def test_decode_workspace_errors(L):
    d, c = _dims(), _cache(max_blocks=64)
    need = gb.gva_decode_workspace_bytes(d, 2, 1000, 4)
    assert need > 0
    assert _decode(L, d, c, max_len=1000, S=4) == gb.GVA_ERR_WORKSPACE
    assert _decode(L, d, c, max_len=1000, S=4, ws=A, ws_bytes=need - 1) == gb.GVA_ERR_WORKSPACE
    assert _decode(L, d, c, max_len=1000, S=4, ws=A + 16, ws_bytes=need) == gb.GVA_ERR_WORKSPACE


def test_mfma_kernel_shape_limits(L):
    # forcing the matrix-core kernel on shapes it does not cover is GVA_ERR_UNSUPPORTED
    cases = [
        (_dims(), _cache(dtype=gb.GVA_DTYPE_F32)),
        (_dims(d_h=48, d_n=48), _cache(d=_dims(d_h=48, d_n=48))),
        (_dims(d_r=20), _cache(d=_dims(d_r=20), kr_stride_token=24)),
        (_dims(d_r=40), _cache(d=_dims(d_r=40))),
        (_dims(H=64, G=2), _cache(d=_dims(H=64, G=2))),
        (_dims(H=32, G=32), _cache(d=_dims(H=32, G=32))),
        (_dims(), _cache(bs=8, max_blocks=16)),
        (_dims(), _cache(v_stride_token=132)),
    ]
    for d, c in cases:
        assert _decode(L, d, c, S=1, kernel=gb.GVA_KERNEL_MFMA) == gb.GVA_ERR_UNSUPPORTED


def test_split_planning(L):
    d = _dims()
    # automatic: a single sequence gets 128 chunks, long sequences chunks of at most 2048
    # positions (rounded up to multiples of 64), short ones chunks down to 64 positions
    S = gb.gva_decode_num_splits(d, 1, 131072, 0)
    assert S == 128
    assert gb.gva_decode_num_splits(d, 256, 32769, 0) == 17     # chunks of 1984 positions
    assert gb.gva_decode_num_splits(d, 8, 4097, 0) == 13         # 16 asked, chunks of 320
    assert gb.gva_decode_num_splits(d, 1, 1000, 0) == 16         # chunks of 64
    # explicit split counts are kept unless a chunk would start beyond max_len
    for S in (64, 128, 256):
        assert gb.gva_decode_num_splits(d, 1, 131072, S) == S
    assert gb.gva_decode_num_splits(d, 1, 100, 8) == 2        # chunks of 64 positions
    assert gb.gva_decode_num_splits(d, 1, 0, 0) == 1
    assert gb.gva_decode_workspace_bytes(d, 1, 131072, 1) == 0
    ws = gb.gva_decode_workspace_bytes(d, 4, 5000, 8)
    S = gb.gva_decode_num_splits(d, 4, 5000, 8)
    assert ws >= 4 * S * 32 * (128 + 2) * 4 and ws % 256 == 0
    assert gb.gva_decode_num_splits(d, 0, 10, 0) == 0


def test_balanced_range_planning(L):
    """The matrix-core kernel's automatic plan: equal tile ranges, one pass of work-groups over
    256 CUs, never more ranges than tiles, and none for a single sequence. With G a multiple of
    8 and at least 256 ranges of 32 tiles, a range is one 8-wave work-group (one per CU, sharing
    the positional key), so 256 ranges; otherwise three four-wave work-groups per CU, so up to
    3 * 256 / (G / 4) ranges, at least 256 / (G / 4) or ranges of 32 tiles."""
    d = _dims()
    assert gb.gva_decode_num_ranges(d, 256, 32769) == 256
    assert gb.gva_decode_num_ranges(d, 8, 32768) == 256                # 8192 tiles: shared key
    assert gb.gva_decode_num_ranges(d, 4, 8705) == 128                 # 1092 tiles: four-wave
    assert gb.gva_decode_num_ranges(d, 16, 4096) == 128                # 2048 tiles / 32 < 128
    assert gb.gva_decode_num_ranges(d, 64, 32768) == 256               # one pass
    assert gb.gva_decode_num_ranges(d, 3, 40) == 6                     # one tile per range
    assert gb.gva_decode_num_ranges(d, 1, 131072) == 0
    assert gb.gva_decode_num_ranges(d, 2, 0) == 0
    d4 = _dims(H=16, G=4, d_h=64, d_n=64)
    assert gb.gva_decode_num_ranges(d4, 256, 32769) == 768             # 3 x 256 four-wave groups
    assert gb.gva_decode_num_ranges(d4, 65, 4097) == 263               # 8385 tiles / 32 > 256
    # the workspace query covers every plan, the GQA comparator's too (two four-wave
    # work-groups per range at G = 8: up to 384 ranges)
    ws = gb.gva_decode_workspace_bytes(d, 256, 32769, 0)
    assert ws >= (384 + 256) * 32 * (128 + 2) * 4 + 257 * 4


def test_merged_decode_planning(L):
    """Small batches at d_h of 32 or 64 (B G <= 256 sequence-groups, automatic split count) take
    the merged plan: no tile ranges, and a workspace that holds the tickets and K partials per
    (sequence, group) with K = min(256 / (B G), ceil(tiles / 8), 32). d_h = 128 keeps the
    ranges."""
    d64 = _dims(H=16, G=4, d_h=64, d_n=64)
    assert gb.gva_decode_num_ranges(d64, 8, 4097) == 0
    assert gb.gva_decode_num_ranges(d64, 64, 100) == 0                 # 256 pairs, K = 1
    assert gb.gva_decode_num_ranges(d64, 65, 100) > 0                  # 260 pairs: ranges
    assert gb.gva_decode_num_ranges(_dims(), 8, 32768) == 256          # d_h = 128: ranges
    assert gb.gva_decode_num_ranges(_dims(H=8, G=4, d_h=32, d_n=32), 3, 5000) == 0
    # K = min(256 / 32, ceil(129 / 8), 32) = 8 partials of 4 heads per pair, after the tickets
    ws = gb.gva_decode_workspace_bytes(d64, 8, 4097, 0)
    assert ws >= 1024 + 8 * 32 * 4 * (64 + 2) * 4 and ws % 256 == 0
    # an explicit split count keeps the split grid
    assert gb.gva_decode_num_splits(d64, 8, 4097, 16) == 13      # chunks of 320


def test_append_and_absorb_validation(L):
    d, c = _dims(), _cache()
    app = lambda **kw: L.gva_cache_append(ctypes.byref(d), ctypes.byref(kw.get("c", c)),
                                          kw.get("B", 2), kw.get("n", 3), kw.get("seq", A),
                                          kw.get("pos", A), kw.get("v", A), kw.get("kr", A), None)
    assert app(n=0) == gb.GVA_OK                  # nothing to do, nothing launched
    assert app(B=0) == gb.GVA_ERR_INVALID_ARG
    assert app(n=-1) == gb.GVA_ERR_INVALID_ARG
    assert app(seq=None) == gb.GVA_ERR_INVALID_ARG
    assert app(v=A + 4) == gb.GVA_ERR_INVALID_ARG
    assert app(c=_cache(block_size=3)) == gb.GVA_ERR_INVALID_ARG
    ab = lambda **kw: L.gva_absorb_query(ctypes.byref(kw.get("d", d)), kw.get("n", 2),
                                         kw.get("qn", A), kw.get("qr", A), kw.get("qp", A),
                                         kw.get("M", A), kw.get("rope", A), kw.get("mp", 10),
                                         kw.get("out", A), None, None)
    assert ab(n=0) == gb.GVA_OK
    assert ab(n=-2) == gb.GVA_ERR_INVALID_ARG
    assert ab(M=None) == gb.GVA_ERR_INVALID_ARG
    assert ab(M=A + 8) == gb.GVA_ERR_INVALID_ARG
    assert ab(mp=0) == gb.GVA_ERR_INVALID_ARG
    assert ab(d=_dims(d_n=126)) == gb.GVA_ERR_UNSUPPORTED


def test_decode_step_validation(L):
    """Every call here fails validation on the host, before anything is launched."""
    d, c = _dims(), _cache()
    def st(**kw):
        return L.gva_decode_step(ctypes.byref(kw.get("d", d)), ctypes.byref(kw.get("c", c)),
                                 kw.get("B", 2), kw.get("pos", A), kw.get("v", A),
                                 kw.get("kr", A), kw.get("qn", A), kw.get("qr", A), kw.get("M", A),
                                 kw.get("sl", A), kw.get("ml", 100), kw.get("scale", 0.1),
                                 kw.get("S", 0), kw.get("kernel", 0), kw.get("qa", A),
                                 kw.get("ws", None), kw.get("wsb", 0), kw.get("out", A), None, None)
    assert st(B=0) == gb.GVA_ERR_INVALID_ARG
    assert st(pos=None) == gb.GVA_ERR_INVALID_ARG
    assert st(v=None) == gb.GVA_ERR_INVALID_ARG
    assert st(kr=A + 4) == gb.GVA_ERR_INVALID_ARG
    assert st(qn=None) == gb.GVA_ERR_INVALID_ARG
    assert st(M=A + 8) == gb.GVA_ERR_INVALID_ARG
    assert st(qa=None) == gb.GVA_ERR_INVALID_ARG
    assert st(qa=A + 8) == gb.GVA_ERR_INVALID_ARG          # the decode reads q_abs 16-aligned
    assert st(sl=None) == gb.GVA_ERR_INVALID_ARG
    assert st(out=None) == gb.GVA_ERR_INVALID_ARG
    assert st(scale=0.0) == gb.GVA_ERR_INVALID_ARG
    assert st(ml=8 * 16 + 1) == gb.GVA_ERR_INVALID_ARG      # beyond the table's capacity
    assert st(S=1025) == gb.GVA_ERR_INVALID_ARG
    assert st(d=_dims(d_n=126)) == gb.GVA_ERR_UNSUPPORTED   # the absorption's float4 rows
    assert st(c=_cache(rope=None)) == gb.GVA_ERR_INVALID_ARG
    assert st(c=_cache(max_pos=0)) == gb.GVA_ERR_INVALID_ARG
    # the automatic plan of a bf16 batch needs a workspace
    assert st() == gb.GVA_ERR_WORKSPACE
    assert st(ws=A + 64, wsb=1 << 30) == gb.GVA_ERR_WORKSPACE   # not 256-byte aligned
    assert b"workspace" in L.gva_last_error()


def test_prefill_validation(L):
    d, c = _dims(), _cache(max_blocks=64)
    pf = lambda **kw: L.gva_prefill_chunk(ctypes.byref(kw.get("d", d)), ctypes.byref(kw.get("c", c)),
                                          2, A, kw.get("ms", 100), kw.get("C", 64), A, A, A,
                                          kw.get("scale", 0.1), A, None, None)
    assert pf(C=0) == gb.GVA_OK
    assert pf(C=-1) == gb.GVA_ERR_INVALID_ARG
    assert pf(ms=1000) == gb.GVA_ERR_INVALID_ARG           # beyond the table's capacity
    assert pf(scale=-1.0) == gb.GVA_ERR_INVALID_ARG
    assert pf(c=_cache(dtype=gb.GVA_DTYPE_F32, max_blocks=64)) == gb.GVA_ERR_UNSUPPORTED


def test_recon_validation(L):
    """The non-absorbable comparator's argument checks, all on the host before any launch."""
    d, c = _dims(), _cache()

    def rc(**kw):
        return L.gva_recon_decode(ctypes.byref(kw.get("d", d)), ctypes.byref(kw.get("c", c)),
                                  kw.get("B", 2), kw.get("sl", A), kw.get("ml", 100),
                                  kw.get("q", A), kw.get("qp", A), kw.get("Mt", A),
                                  kw.get("rope", A + 16384), kw.get("mp", 1024),
                                  kw.get("scale", 0.1), kw.get("S", 0), kw.get("ws", None),
                                  kw.get("wsb", 0), kw.get("out", A), None, None)
    assert rc(B=0) == gb.GVA_ERR_INVALID_ARG
    for k in ("sl", "q", "qp", "Mt", "rope", "out"):
        assert rc(**{k: None}) == gb.GVA_ERR_INVALID_ARG, k
    for k in ("q", "Mt", "rope", "out"):
        assert rc(**{k: A + 8}) == gb.GVA_ERR_INVALID_ARG, k      # 16-byte alignment
    assert rc(mp=31) == gb.GVA_ERR_INVALID_ARG                     # the in-tile angles need 32 rows
    assert rc(ml=8 * 16 + 1) == gb.GVA_ERR_INVALID_ARG              # beyond the table's capacity
    assert rc(ml=-1) == gb.GVA_ERR_INVALID_ARG
    assert rc(scale=0.0) == gb.GVA_ERR_INVALID_ARG
    assert rc(S=1025) == gb.GVA_ERR_INVALID_ARG
    assert rc(d=_dims(d_h=96)) == gb.GVA_ERR_UNSUPPORTED
    assert rc(d=_dims(d_n=96)) == gb.GVA_ERR_UNSUPPORTED
    assert rc(d=_dims(H=32, G=4)) == gb.GVA_ERR_UNSUPPORTED         # eight heads per group
    assert rc(d=_dims(H=12, G=8)) == gb.GVA_ERR_INVALID_ARG
    assert rc(c=_cache(dtype=gb.GVA_DTYPE_F32)) == gb.GVA_ERR_UNSUPPORTED
    assert rc(c=_cache(v_stride_token=132)) == gb.GVA_ERR_INVALID_ARG
    assert rc(c=_cache(block_size=24)) == gb.GVA_ERR_INVALID_ARG
    # d_r is not used: dims with d_r = 0 pass the shape checks (and then need a workspace)
    assert rc(d=_dims(d_r=0)) == gb.GVA_ERR_WORKSPACE
    # two sequences of up to 100 positions are split in two chunks of 64: a workspace is needed
    wsb = gb.gva_recon_decode_workspace_bytes(d, 2, 100, 0)
    assert wsb > 0
    assert rc() == gb.GVA_ERR_WORKSPACE
    assert rc(ws=A + 64, wsb=wsb) == gb.GVA_ERR_WORKSPACE          # not 256-byte aligned
    assert rc(ws=A, wsb=wsb - 1) == gb.GVA_ERR_WORKSPACE
    # a large batch runs one chunk per sequence and needs none
    assert gb.gva_recon_decode_workspace_bytes(d, 256, 100, 0) == 0
    assert gb.gva_recon_decode_workspace_bytes(d, 2, 100, 1) == 0


def test_mla_validation(L):
    """The MLA-style latent comparator's argument checks, all on the host before any launch."""
    d = _dims(H=32, G=1, d_h=256, d_n=256, d_r=64)
    c = _cache(d=_dims(H=32, G=1, d_h=256, d_n=256, d_r=64))

    def ml(**kw):
        return L.gva_mla_decode(ctypes.byref(kw.get("d", d)), ctypes.byref(kw.get("c", c)),
                                kw.get("B", 2), kw.get("sl", A), kw.get("ml", 100),
                                kw.get("q", A), kw.get("scale", 0.1), kw.get("S", 0),
                                kw.get("ws", None), kw.get("wsb", 0), kw.get("out", A), None, None)
    assert ml(d=_dims(H=32, G=2, d_h=256, d_r=64)) == gb.GVA_ERR_INVALID_ARG     # one latent
    assert ml(d=_dims(H=24, G=1, d_h=256, d_r=64)) == gb.GVA_ERR_UNSUPPORTED
    assert ml(d=_dims(H=32, G=1, d_h=384, d_r=64)) == gb.GVA_ERR_UNSUPPORTED
    assert ml(d=_dims(H=32, G=1, d_h=256, d_r=12)) == gb.GVA_ERR_UNSUPPORTED
    assert ml(d=_dims(H=32, G=1, d_h=256, d_r=72)) == gb.GVA_ERR_UNSUPPORTED
    assert ml(c=_cache(dtype=gb.GVA_DTYPE_F32)) == gb.GVA_ERR_UNSUPPORTED
    assert ml(c=_cache(d=d, v_stride_token=260)) == gb.GVA_ERR_INVALID_ARG       # not 8-aligned
    assert ml(c=_cache(d=d, bs=8, max_blocks=16)) == gb.GVA_ERR_UNSUPPORTED     # blocks < 16
    assert ml(B=0) == gb.GVA_ERR_INVALID_ARG
    for k in ("sl", "q", "out"):
        assert ml(**{k: None}) == gb.GVA_ERR_INVALID_ARG, k
    assert ml(q=A + 8) == gb.GVA_ERR_INVALID_ARG
    assert ml(ml=8 * 16 + 1) == gb.GVA_ERR_INVALID_ARG
    assert ml(scale=0.0) == gb.GVA_ERR_INVALID_ARG
    assert ml(S=1025) == gb.GVA_ERR_INVALID_ARG
    # d_c = 512 is accepted (and a split plan then needs a workspace)
    d512 = _dims(H=32, G=1, d_h=256, d_n=256, d_r=64)
    d512.d_h = 512
    wsb = gb.gva_mla_decode_workspace_bytes(d512, 2, 100, 0)
    assert wsb > 0
    assert ml(d=d512, c=_cache(d=d, v_stride_token=512, v_stride_block=16 * 512)) == gb.GVA_ERR_WORKSPACE
    assert ml(d=d512, c=_cache(d=d, v_stride_token=512, v_stride_block=16 * 512),
              ws=A + 64, wsb=wsb) == gb.GVA_ERR_WORKSPACE
    # one chunk per sequence: no partials, only the work queue's counter
    assert gb.gva_mla_decode_workspace_bytes(d512, 256, 100, 0) == 256
    assert ml(d=d512, c=_cache(d=d, v_stride_token=512, v_stride_block=16 * 512),
              B=256, ml=100) == gb.GVA_ERR_WORKSPACE


# ---- the head -> group map (gva_dims.g_of_h) ----------------------------------------------------


def _absorb_empty(L, d):
    """gva_absorb_query with no tokens: validates the dims and launches nothing."""
    return L.gva_absorb_query(ctypes.byref(d), 0, A, A, A, A, A, 16, A, None, None)


@pytest.mark.parametrize("gmap,ok", [
    (None, True),
    ([0, 0, 1, 1, 2, 2, 3, 3], True),                 # the contiguous map written out
    ([3, 1, 0, 2, 1, 3, 2, 0], True),                 # a balanced permutation
    ([0, 0, 1, 1, 2, 2, 3, 4], False),                # a group outside [0, G)
    ([0, 0, 1, 1, 2, 2, 3, -1], False),               # a negative group
    ([0, 0, 0, 1, 2, 2, 3, 3], False),                # group 0 holds 3 heads, group 1 one
])
def test_group_map_validation(L, gmap, ok):
    d = gb.dims_struct(8, 4, 64, 64, 16, gmap)
    st = _absorb_empty(L, d)
    assert st == (gb.GVA_OK if ok else gb.GVA_ERR_INVALID_ARG), L.gva_last_error().decode()
    # every entry point that takes dims rejects the same map before any launch
    ws = gb.gva_decode_workspace_bytes(d, 2, 100, 0)
    assert (ws > 0) == ok
    if not ok:
        assert _decode(L, d, _cache(d=d)) == gb.GVA_ERR_INVALID_ARG
        assert "g_of_h" in L.gva_last_error().decode()


# ---- the allocation-free decode -----------------------------------------------------------


def test_noalloc_rejects_a_plan_above_the_static_scratch(L):
    """A plan whose partials exceed GVA_NOALLOC_SCRATCH_BYTES (32 MiB) is refused before any HIP
    call, with the need and the limit in the message; bad arguments are refused as gva_decode
    refuses them."""
    d = _dims(H=256, G=1, d_h=256, d_n=256, d_r=16)
    c = _cache(d=d, bs=16, max_blocks=4096, num_blocks=1 << 16)
    need = gb.gva_decode_workspace_bytes(d, 64, 60000, 1024)
    assert need > 32 << 20
    st = L.gva_decode_noalloc(ctypes.byref(d), ctypes.byref(c), 64, A, 60000, A, 0.1, 1024,
                              gb.GVA_KERNEL_GENERIC, A, None, None)
    assert st == gb.GVA_ERR_WORKSPACE
    msg = L.gva_last_error().decode()
    assert "static scratch" in msg and str(32 << 20) in msg
    bad = gb.GvaDims(32, 5, 128, 128, 16)
    assert L.gva_decode_noalloc(ctypes.byref(bad), ctypes.byref(_cache()), 2, A, 100, A, 0.1, 0,
                                0, A, None, None) == gb.GVA_ERR_INVALID_ARG
    assert L.gva_decode_noalloc(ctypes.byref(_dims()), ctypes.byref(_cache()), 2, A, 100, A + 4,
                                0.1, 0, 0, A, None, None) == gb.GVA_ERR_INVALID_ARG


def test_stream_read_rejects_bad_arguments(L):
    P = ctypes.c_void_p
    assert L.gva_diag_stream_read(A + 8, 1024, 16, 4, A, None) == gb.GVA_ERR_INVALID_ARG
    assert L.gva_diag_stream_read(A, 1000, 16, 4, A, None) == gb.GVA_ERR_INVALID_ARG
    assert L.gva_diag_stream_read(A, 1024, 0, 4, A, None) == gb.GVA_ERR_INVALID_ARG
    assert L.gva_diag_stream_read(A, 1024, 16, 3, A, None) == gb.GVA_ERR_INVALID_ARG
    assert L.gva_diag_stream_read(None, 1024, 16, 4, A, None) == gb.GVA_ERR_INVALID_ARG


def test_absorb_requires_aligned_query_rows(L):
    """q_nope and M are read 16 bytes at a time: a q_nope only 4- or 8-byte aligned is refused
    before any launch (as are M, q_rope and q_abs off their alignment)."""
    d = _dims()
    for qn, qr, m, qa in ((A + 4, A, A, A), (A + 8, A, A, A), (A, A + 4, A, A), (A, A, A + 8, A),
                          (A, A, A, A + 4)):
        st = L.gva_absorb_query(ctypes.byref(d), 1, qn, qr, A, m, A, 16, qa, None, None)
        assert st == gb.GVA_ERR_INVALID_ARG, (qn, qr, m, qa)
        assert "misaligned" in L.gva_last_error().decode()


def test_decode_step_launches_plan(L):
    """The one-launch step serves small batches: on the matrix cores the shapes with d_h of 32
    or 64, the automatic split count and sequences of at most 4 MiB of values per group; on the
    vector ALU (float32 caches, or the generic kernel) sequences of at most 1024 positions whose
    group's rows of M fit the LDS region."""
    d = _dims(H=16, G=4, d_h=64, d_n=64)             # the 350M-class layer
    c = _cache(d=d, max_blocks=4096)
    n = lambda *a: L.gva_decode_step_launches(ctypes.byref(d), ctypes.byref(c), *a)
    assert n(8, 4097, 0, 0) == 1                     # B = 8, T = 4096 + 1
    assert n(64, 4097, 0, 0) == 1                    # 256 sequence-groups
    assert n(65, 4097, 0, 0) == 3                    # 260: the balanced plan and its combine
    assert n(8, 4097, 3, 0) == 3                     # an explicit split count
    assert n(8, 32769, 0, 0) == 2                    # more than 4 MiB of values per group:
    #                                                  append + absorb, then the merged decode
    assert n(8, 4097, 0, gb.GVA_KERNEL_GENERIC) == 3
    assert n(0, 100, 0, 0) == 0 and n(4, 100, 0, 9) == 0
    d128 = _dims()                                   # d_h = 128: two launches
    assert L.gva_decode_step_launches(ctypes.byref(d128), ctypes.byref(_cache(max_blocks=2048)),
                                      4, 8705, 0, 0) == 3
    c32 = _cache(dtype=gb.GVA_DTYPE_F32, max_blocks=2048)
    n32 = lambda *a: L.gva_decode_step_launches(ctypes.byref(d), ctypes.byref(c32), *a)
    assert n32(1, 256, 1, 0) == 2                    # an explicit split count
    assert n32(1, 257, 0, 0) == 1                    # the vector-ALU step in one launch
    assert n32(64, 1024, 0, 0) == 1                  # 256 sequence-groups, 1024 positions
    assert n32(64, 1025, 0, 0) == 3                  # longer: append + absorb, decode, combine
    assert n32(65, 100, 0, 0) == 3                   # 260 sequence-groups: split and combine
    assert n(8, 1000, 0, gb.GVA_KERNEL_GENERIC) == 1 # the generic kernel asked for, short
    d8 = _dims(H=16, G=2, d_h=128, d_n=128)          # 8 heads x 128 x 128 of M: above the region
    c8 = _cache(d=d8, dtype=gb.GVA_DTYPE_F32, max_blocks=2048)
    assert L.gva_decode_step_launches(ctypes.byref(d8), ctypes.byref(c8), 2, 300, 0, 0) == 3
    d256 = _dims(H=8, G=2, d_h=256, d_n=256)
    assert L.gva_decode_step_launches(ctypes.byref(d256), ctypes.byref(_cache(d=d256)), 2, 100, 0, 0) == 3
