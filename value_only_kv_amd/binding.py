"""Thin Python binding of the GVA C ABI (include/gva.h): argument marshalling only.

Every function here has the name of the C entry point it calls and only turns tensors into
pointers and a stream handle; all of the work runs in the HIP kernels of libgva.so. There is
no fallback: if the library is missing, loading raises.

PyTorch supplies device memory and streams. `GvaCache` helps allocate one layer's cache as
torch tensors with the strides the library reads.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p
from dataclasses import dataclass
from typing import Optional

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgva.so")

GVA_OK, GVA_ERR_INVALID_ARG, GVA_ERR_UNSUPPORTED, GVA_ERR_WORKSPACE, GVA_ERR_HIP = range(5)
GVA_DTYPE_F32, GVA_DTYPE_BF16 = 0, 1
GVA_KERNEL_AUTO, GVA_KERNEL_GENERIC, GVA_KERNEL_MFMA = 0, 1, 2
DEVERR_BLOCK, DEVERR_CAPACITY, DEVERR_ROPE, DEVERR_SEQ, DEVERR_LENGTH = 1, 2, 4, 8, 16

EXPORTED = [
    "gva_rope_table_bytes", "gva_rope_table_fill", "gva_cache_append", "gva_absorb_query",
    "gva_decode_workspace_bytes", "gva_decode_num_splits", "gva_decode_num_ranges", "gva_decode",
    "gva_decode_step", "gva_decode_step_launches", "gva_prefill_chunk", "gva_gqa_decode", "gva_decode_noalloc",
    "gva_recon_decode_workspace_bytes", "gva_recon_decode",
    "gva_mla_decode_workspace_bytes", "gva_mla_decode",
    "gva_status_string", "gva_last_error", "gva_version", "gva_diag_stream_read",
]


class GvaDims(ctypes.Structure):
    _fields_ = [("H", c_int32), ("G", c_int32), ("d_h", c_int32), ("d_n", c_int32),
                ("d_r", c_int32), ("g_of_h", c_void_p)]


class GvaCacheStruct(ctypes.Structure):
    _fields_ = [
        ("dtype", c_int32), ("v", c_void_p), ("kr", c_void_p),
        ("v_stride_block", c_int64), ("v_stride_token", c_int64), ("v_stride_group", c_int64),
        ("kr_stride_block", c_int64), ("kr_stride_token", c_int64),
        ("num_blocks", c_int64), ("block_size", c_int32), ("max_blocks", c_int32),
        ("block_table", c_void_p), ("rope", c_void_p), ("max_pos", c_int32),
        ("err_flag", c_void_p),
    ]


class GVAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_status_name(status)}: {detail}")
        self.status = status
        self.detail = detail


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Loads libgva.so (built in-tree); raises ImportError when it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m value_only_kv_amd._build` "
                          "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    L.gva_rope_table_bytes.argtypes = [c_int32, c_int32]
    L.gva_rope_table_bytes.restype = c_size_t
    L.gva_rope_table_fill.argtypes = [P, c_int32, c_int32, c_double]
    L.gva_rope_table_fill.restype = c_int32
    L.gva_cache_append.argtypes = [POINTER(GvaDims), POINTER(GvaCacheStruct), c_int32, c_int32,
                                   P, P, P, P, P]
    L.gva_cache_append.restype = c_int32
    L.gva_absorb_query.argtypes = [POINTER(GvaDims), c_int32, P, P, P, P, P, c_int32, P, P, P]
    L.gva_absorb_query.restype = c_int32
    L.gva_decode_workspace_bytes.argtypes = [POINTER(GvaDims), c_int32, c_int32, c_int32]
    L.gva_decode_workspace_bytes.restype = c_size_t
    L.gva_decode_num_splits.argtypes = [POINTER(GvaDims), c_int32, c_int32, c_int32]
    L.gva_decode_num_splits.restype = c_int32
    L.gva_decode_num_ranges.argtypes = [POINTER(GvaDims), c_int32, c_int32]
    L.gva_decode_num_ranges.restype = c_int32
    L.gva_decode.argtypes = [POINTER(GvaDims), POINTER(GvaCacheStruct), c_int32, P, c_int32, P,
                             c_float, c_int32, c_int32, P, c_size_t, P, P, P]
    L.gva_decode.restype = c_int32
    L.gva_decode_noalloc.argtypes = [POINTER(GvaDims), POINTER(GvaCacheStruct), c_int32, P,
                                     c_int32, P, c_float, c_int32, c_int32, P, P, P]
    L.gva_decode_noalloc.restype = c_int32
    L.gva_decode_step_launches.argtypes = [POINTER(GvaDims), POINTER(GvaCacheStruct), c_int32,
                                           c_int32, c_int32, c_int32]
    L.gva_decode_step_launches.restype = c_int32
    L.gva_decode_step.argtypes = [POINTER(GvaDims), POINTER(GvaCacheStruct), c_int32, P, P, P, P,
                                  P, P, P, c_int32, c_float, c_int32, c_int32, P, P, c_size_t, P,
                                  P, P]
    L.gva_decode_step.restype = c_int32
    L.gva_prefill_chunk.argtypes = [POINTER(GvaDims), POINTER(GvaCacheStruct), c_int32, P, c_int32,
                                    c_int32, P, P, P, c_float, P, P, P]
    L.gva_prefill_chunk.restype = c_int32
    L.gva_gqa_decode.argtypes = [POINTER(GvaDims), POINTER(GvaCacheStruct), P, c_int32, P, c_int32,
                                 P, c_float, P, c_size_t, P, P, P]
    L.gva_gqa_decode.restype = c_int32
    L.gva_recon_decode_workspace_bytes.argtypes = [POINTER(GvaDims), c_int32, c_int32, c_int32]
    L.gva_recon_decode_workspace_bytes.restype = c_size_t
    L.gva_recon_decode.argtypes = [POINTER(GvaDims), POINTER(GvaCacheStruct), c_int32, P, c_int32,
                                   P, P, P, P, c_int32, c_float, c_int32, P, c_size_t, P, P, P]
    L.gva_recon_decode.restype = c_int32
    L.gva_mla_decode_workspace_bytes.argtypes = [POINTER(GvaDims), c_int32, c_int32, c_int32]
    L.gva_mla_decode_workspace_bytes.restype = c_size_t
    L.gva_mla_decode.argtypes = [POINTER(GvaDims), POINTER(GvaCacheStruct), c_int32, P, c_int32,
                                 P, c_float, c_int32, P, c_size_t, P, P, P]
    L.gva_mla_decode.restype = c_int32
    L.gva_diag_stream_read.argtypes = [P, c_size_t, c_int32, c_int32, P, P]
    L.gva_diag_stream_read.restype = c_int32
    L.gva_status_string.argtypes = [c_int32]
    L.gva_status_string.restype = c_char_p
    L.gva_last_error.argtypes = []
    L.gva_last_error.restype = c_char_p
    L.gva_version.argtypes = []
    L.gva_version.restype = c_char_p
    _LIB = L
    return L


def _status_name(status: int) -> str:
    try:
        return lib().gva_status_string(status).decode()
    except Exception:
        return f"status {status}"


def _check(status: int) -> None:
    if status != GVA_OK:
        raise GVAError(status, lib().gva_last_error().decode())


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (None passes NULL); ints pass through as raw addresses."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dims_struct(H: int, G: int, d_h: int, d_n: int, d_r: int, g_of_h=None) -> GvaDims:
    """The C struct; g_of_h (a sequence of H group indices, or None for the contiguous map) is
    kept alive as a host int32 array referenced by the struct."""
    d = GvaDims(H, G, d_h, d_n, d_r, None)
    if g_of_h is not None:
        arr = np.ascontiguousarray(np.asarray(g_of_h, dtype=np.int32))
        d._g_of_h_keep = arr
        d.g_of_h = arr.ctypes.data
    return d


# ---- entry points (same names as the C ABI) -------------------------------------------------


def gva_rope_table_bytes(max_pos: int, d_r: int) -> int:
    return int(lib().gva_rope_table_bytes(max_pos, d_r))


def gva_rope_table_fill(max_pos: int, d_r: int, base: float = 10000.0) -> np.ndarray:
    """Returns the host float64 table [max_pos, d_r/2, 2] filled by the library."""
    out = np.empty((max_pos, d_r // 2, 2), dtype=np.float64)
    _check(lib().gva_rope_table_fill(out.ctypes.data, max_pos, d_r, base))
    return out


def gva_cache_append(dims: GvaDims, cache: "GvaCache", B: int, seq, pos, v_new, kr_raw,
                     stream=None) -> None:
    n_tok = int(seq.numel())
    _check(lib().gva_cache_append(ctypes.byref(dims), ctypes.byref(cache.struct), B, n_tok,
                                  _ptr(seq), _ptr(pos), _ptr(v_new), _ptr(kr_raw),
                                  _stream(stream)))


def gva_absorb_query(dims: GvaDims, q_nope, q_rope, q_pos, M, rope, max_pos: int, q_abs,
                     err_flag=None, stream=None) -> None:
    n_q = int(q_pos.numel())
    _check(lib().gva_absorb_query(ctypes.byref(dims), n_q, _ptr(q_nope), _ptr(q_rope), _ptr(q_pos),
                                  _ptr(M), _ptr(rope), max_pos, _ptr(q_abs), _ptr(err_flag),
                                  _stream(stream)))


def gva_decode_workspace_bytes(dims: GvaDims, B: int, max_len: int, num_splits: int = 0) -> int:
    return int(lib().gva_decode_workspace_bytes(ctypes.byref(dims), B, max_len, num_splits))


def gva_decode_num_splits(dims: GvaDims, B: int, max_len: int, num_splits: int = 0) -> int:
    return int(lib().gva_decode_num_splits(ctypes.byref(dims), B, max_len, num_splits))


def gva_decode_num_ranges(dims: GvaDims, B: int, max_len: int) -> int:
    return int(lib().gva_decode_num_ranges(ctypes.byref(dims), B, max_len))


def gva_decode(dims: GvaDims, cache: "GvaCache", B: int, seq_len, max_len: int, q_abs,
               scale: float, out, lse=None, num_splits: int = 0, kernel: int = GVA_KERNEL_AUTO,
               workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gva_decode(ctypes.byref(dims), ctypes.byref(cache.struct), B, _ptr(seq_len),
                            max_len, _ptr(q_abs), scale, num_splits, kernel, _ptr(workspace),
                            ws_bytes, _ptr(out), _ptr(lse), _stream(stream)))


def gva_decode_noalloc(dims: GvaDims, cache: "GvaCache", B: int, seq_len, max_len: int, q_abs,
                       scale: float, out, lse=None, num_splits: int = 0,
                       kernel: int = GVA_KERNEL_AUTO, stream=None) -> None:
    """gva_decode with its partials in the library's static device scratch (no workspace)."""
    _check(lib().gva_decode_noalloc(ctypes.byref(dims), ctypes.byref(cache.struct), B,
                                    _ptr(seq_len), max_len, _ptr(q_abs), scale, num_splits,
                                    kernel, _ptr(out), _ptr(lse), _stream(stream)))


def gva_decode_step(dims: GvaDims, cache: "GvaCache", B: int, pos, v_new, kr_raw, q_nope, q_rope,
                    M, seq_len, max_len: int, scale: float, q_abs, out, lse=None,
                    num_splits: int = 0, kernel: int = GVA_KERNEL_AUTO, workspace=None,
                    stream=None) -> None:
    """Append + absorb (one launch) + decode for one new token per sequence."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gva_decode_step(ctypes.byref(dims), ctypes.byref(cache.struct), B, _ptr(pos),
                                 _ptr(v_new), _ptr(kr_raw), _ptr(q_nope), _ptr(q_rope), _ptr(M),
                                 _ptr(seq_len), max_len, scale, num_splits, kernel, _ptr(q_abs),
                                 _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse),
                                 _stream(stream)))


def gva_decode_step_launches(dims: GvaDims, cache: "GvaCache", B: int, max_len: int,
                             num_splits: int = 0, kernel: int = GVA_KERNEL_AUTO) -> int:
    return int(lib().gva_decode_step_launches(ctypes.byref(dims), ctypes.byref(cache.struct), B,
                                              max_len, num_splits, kernel))


def gva_prefill_chunk(dims: GvaDims, cache: "GvaCache", B: int, start, max_start: int,
                      chunk_len: int, q_abs, v_new, kr_raw, scale: float, out, lse=None,
                      stream=None) -> None:
    _check(lib().gva_prefill_chunk(ctypes.byref(dims), ctypes.byref(cache.struct), B, _ptr(start),
                                   max_start, chunk_len, _ptr(q_abs), _ptr(v_new), _ptr(kr_raw),
                                   scale, _ptr(out), _ptr(lse), _stream(stream)))


def gva_gqa_decode(dims: GvaDims, values: "GvaCache", keys, B: int, seq_len, max_len: int, q,
                   scale: float, out, lse=None, workspace=None, stream=None) -> None:
    """The GQA comparator: keys is a tensor laid out exactly like values.v."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gva_gqa_decode(ctypes.byref(dims), ctypes.byref(values.struct), _ptr(keys), B,
                                _ptr(seq_len), max_len, _ptr(q), scale, _ptr(workspace), ws_bytes,
                                _ptr(out), _ptr(lse), _stream(stream)))


def gva_recon_decode_workspace_bytes(dims: GvaDims, B: int, max_len: int, num_splits: int = 0) -> int:
    return int(lib().gva_recon_decode_workspace_bytes(ctypes.byref(dims), B, max_len, num_splits))


def gva_recon_decode(dims: GvaDims, values: "GvaCache", B: int, seq_len, max_len: int, q, q_pos,
                     Mt, rope, max_pos: int, scale: float, out, lse=None, num_splits: int = 0,
                     workspace=None, stream=None) -> None:
    """The non-absorbable comparator: Mt is bf16 bits [H][d_n][d_h] (an int16 tensor), rope a
    float64 table of width d_n."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gva_recon_decode(ctypes.byref(dims), ctypes.byref(values.struct), B,
                                  _ptr(seq_len), max_len, _ptr(q), _ptr(q_pos), _ptr(Mt),
                                  _ptr(rope), max_pos, scale, num_splits, _ptr(workspace),
                                  ws_bytes, _ptr(out), _ptr(lse), _stream(stream)))


def gva_mla_decode_workspace_bytes(dims: GvaDims, B: int, max_len: int, num_splits: int = 0) -> int:
    return int(lib().gva_mla_decode_workspace_bytes(ctypes.byref(dims), B, max_len, num_splits))


def gva_mla_decode(dims: GvaDims, latent: "GvaCache", B: int, seq_len, max_len: int, q_abs,
                   scale: float, out, lse=None, num_splits: int = 0, workspace=None,
                   stream=None) -> None:
    """The MLA-style latent comparator: dims with G = 1 and d_h = d_c; latent.v holds the
    latents, latent.kr the rotated positional keys."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gva_mla_decode(ctypes.byref(dims), ctypes.byref(latent.struct), B, _ptr(seq_len),
                                max_len, _ptr(q_abs), scale, num_splits, _ptr(workspace),
                                ws_bytes, _ptr(out), _ptr(lse), _stream(stream)))


def gva_diag_stream_read(src, nbytes: int, work_groups: int, in_flight: int, sink,
                         stream=None) -> None:
    """The read-only streaming kernel of gva_diag.h (a measurement aid): reads nbytes at src."""
    _check(lib().gva_diag_stream_read(_ptr(src), nbytes, work_groups, in_flight, _ptr(sink),
                                      _stream(stream)))


def gva_version() -> str:
    return lib().gva_version().decode()


# ---- one layer's cache as torch tensors ------------------------------------------------------


@dataclass
class GvaCache:
    """Owns the torch tensors of one cache and the C struct that describes them."""
    v: "object"
    kr: "object"
    block_table: "object"
    rope: "object"
    err_flag: "object"
    struct: GvaCacheStruct

    @staticmethod
    def allocate(dims: GvaDims, dtype: str, num_blocks: int, block_size: int, block_table,
                 rope, strides, device="cuda", fill_bits: Optional[int] = None) -> "GvaCache":
        """Allocates V and kr pools of num_blocks blocks with element strides
        (v_sb, v_st, v_sg, kr_sb, kr_st); fill_bits (optional) fills every element with that
        raw bit pattern (a sentinel)."""
        import torch
        v_sb, v_st, v_sg, kr_sb, kr_st = strides
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        idt = torch.int16 if dtype == "bf16" else torch.int32
        v = torch.empty(num_blocks * v_sb, dtype=tdt, device=device)
        kr = torch.empty(num_blocks * kr_sb, dtype=tdt, device=device)
        if fill_bits is not None:
            fb = int(np.array(fill_bits, dtype=np.uint16 if dtype == "bf16" else np.uint32)
                     .view(np.int16 if dtype == "bf16" else np.int32))
            v.view(idt).fill_(fb)
            kr.view(idt).fill_(fb)
        err = torch.zeros(1, dtype=torch.int32, device=device)
        return GvaCache.wrap(dims, dtype, v, kr, block_size, block_table, rope, strides,
                             num_blocks, err)

    @staticmethod
    def wrap(dims: GvaDims, dtype: str, v, kr, block_size: int, block_table, rope, strides,
             num_blocks: int, err_flag=None) -> "GvaCache":
        v_sb, v_st, v_sg, kr_sb, kr_st = strides
        s = GvaCacheStruct()
        s.dtype = GVA_DTYPE_BF16 if dtype == "bf16" else GVA_DTYPE_F32
        s.v = v.data_ptr()
        s.kr = kr.data_ptr()
        s.v_stride_block, s.v_stride_token, s.v_stride_group = v_sb, v_st, v_sg
        s.kr_stride_block, s.kr_stride_token = kr_sb, kr_st
        s.num_blocks = num_blocks
        s.block_size = block_size
        s.max_blocks = int(block_table.shape[1])
        s.block_table = block_table.data_ptr()
        s.rope = rope.data_ptr()
        s.max_pos = int(rope.shape[0])
        s.err_flag = None if err_flag is None else err_flag.data_ptr()
        return GvaCache(v, kr, block_table, rope, err_flag, s)
