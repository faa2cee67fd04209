"""Shared set-up for the GPU parity tests: one workload's cache built twice from the same seeded
inputs, on the device through gva_cache_append and on the host by the oracle's own append."""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import gva_oracle as O
from value_only_kv_amd import binding as gb
from value_only_kv_amd import synth

SENTINEL = {"bf16": 0x7FC1, "f32": 0x7FC00001}   # NaN patterns no append can produce from finite data

# Tolerances for outputs: bf16 cache with fp32 accumulation -> max-abs 1e-2
# and relative L2 3e-3 over the whole output; fp32 cache -> max-abs 1e-5.
TOL_BF16_MAXABS, TOL_BF16_RELL2 = 1e-2, 3e-3
TOL_F32_MAXABS = 1e-5

# (what, max-abs error, relative L2) of every output check in this process; conftest writes it
# to a file at the end of the session when GVA_PARITY_LOG names one.
ERRORS = []


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_output(got, ref, dtype, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    r = rel_l2(got, ref) if got.size else 0.0
    ERRORS.append((what, dtype, err, r))
    if dtype == "f32":
        assert err <= TOL_F32_MAXABS, (what, err)
    else:
        assert err <= TOL_BF16_MAXABS and r <= TOL_BF16_RELL2, (what, err, r)
    return err


class Case:
    """One workload: device cache + oracle pool built from the same synthetic inputs."""

    def __init__(self, w: synth.Workload, lens=None, group_major=True, device="cuda",
                 max_pos=None, sentinel=True, g_of_h=None):
        self.w = w
        self.lens = np.asarray(lens if lens is not None else synth.lengths(w), dtype=np.int64)
        self.lay = synth.layout(w, self.lens, group_major)
        gmap = None if g_of_h is None else tuple(int(g) for g in g_of_h)
        self.dims = O.Dims(w.H, w.G, w.d_h, w.d_n, w.d_r, gmap)
        self.cdims = gb.dims_struct(w.H, w.G, w.d_h, w.d_n, w.d_r, gmap)
        cap = synth.capacity(w, self.lens)
        self.max_pos = int(max_pos if max_pos is not None else int(cap.max()) + 1)
        self.device = device
        self.tab_lib = torch.from_numpy(gb.gva_rope_table_fill(self.max_pos, w.d_r, w.base)).to(device)
        self._tab_ora = None
        lay = self.lay
        strides = (lay.v_sb, lay.v_st, lay.v_sg, lay.kr_sb, lay.kr_st)
        self.block_table = torch.from_numpy(lay.block_table).to(device)
        sent = SENTINEL[w.dtype] if sentinel else None
        self.cache = gb.GvaCache.allocate(self.cdims, w.dtype, lay.num_blocks, lay.block_size,
                                          self.block_table, self.tab_lib, strides, device,
                                          fill_bits=sent)
        self.pool = O.Pool.empty(w.dtype, lay.v_elems, lay.kr_elems, strides, lay.num_blocks,
                                 lay.block_size, lay.block_table, sentinel=sent)

    @property
    def tab_ora(self):
        if self._tab_ora is None:
            self._tab_ora = O.rope_table(self.max_pos, self.w.d_r, self.w.base)
        return self._tab_ora

    def append_prefix(self, n_per_seq=None, oracle=True, seqs=None):
        """Appends positions 0..n_b-1 of each sequence (n_b = lens[b] by default)."""
        n_per_seq = self.lens if n_per_seq is None else np.asarray(n_per_seq)
        seqs = range(self.w.B) if seqs is None else seqs
        for b in seqs:
            n = int(n_per_seq[b])
            if n == 0:
                continue
            v, kr = synth.sequence_tokens(self.w, b, n)
            self.append_tokens(np.full(n, b), np.arange(n), v, kr, oracle=oracle)

    def append_tokens(self, seq, pos, v, kr, oracle=True):
        d = self.device
        seq_t = torch.from_numpy(np.asarray(seq, np.int32)).to(d)
        pos_t = torch.from_numpy(np.asarray(pos, np.int32)).to(d)
        v_t = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(d)
        k_t = torch.from_numpy(np.ascontiguousarray(kr, np.float32)).to(d)
        gb.gva_cache_append(self.cdims, self.cache, self.w.B, seq_t, pos_t, v_t, k_t)
        if oracle:
            return O.append(self.pool, self.dims, seq, pos, v, kr, self.tab_ora)
        return 0

    def device_bits(self):
        torch.cuda.synchronize()
        it = torch.int16 if self.w.dtype == "bf16" else torch.int32
        nt = np.uint16 if self.w.dtype == "bf16" else np.uint32
        v = self.cache.v.view(it).cpu().numpy().view(nt)
        kr = self.cache.kr.view(it).cpu().numpy().view(nt)
        return v, kr

    def err_flag(self) -> int:
        return int(self.cache.err_flag.item())

    def decode(self, seq_len, q_abs, num_splits=0, kernel=gb.GVA_KERNEL_AUTO, max_len=None,
               with_lse=True, ws_fill=None):
        """Runs gva_decode; returns (out, lse) on the host as float32 arrays. ws_fill: a value
        the workspace holds past its first 1024 bytes (the tickets stay zero) before the call."""
        d = self.device
        B, H = self.w.B, self.w.H
        seq_len = np.asarray(seq_len, np.int32)
        max_len = int(seq_len.max()) if max_len is None else int(max_len)
        sl = torch.from_numpy(seq_len).to(d)
        q = torch.from_numpy(np.ascontiguousarray(q_abs, np.float32)).to(d)
        out = torch.full((B, H, self.w.d_h), float("nan"), device=d)
        lse = torch.full((B, H), float("nan"), device=d) if with_lse else None
        wsb = gb.gva_decode_workspace_bytes(self.cdims, B, max_len, num_splits)
        ws = torch.zeros(max(wsb, 256) // 4, dtype=torch.float32, device=d) if wsb else None
        if ws is not None and ws_fill is not None:
            ws[256:] = ws_fill
        gb.gva_decode(self.cdims, self.cache, B, sl, max_len, q, self.w.scale, out, lse,
                      num_splits=num_splits, kernel=kernel, workspace=ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), (lse.cpu().numpy() if with_lse else None)

    def oracle_decode(self, seq_len, q_abs, seqs=None):
        """Oracle output for the given sequences (all by default): out [B,H,d_h], lse [B,H]."""
        B, H = self.w.B, self.w.H
        out = np.zeros((B, H, self.w.d_h))
        lse = np.full((B, H), -np.inf)
        seqs = range(B) if seqs is None else seqs
        for b in seqs:
            n = int(seq_len[b])
            V, kr = O.gather(self.pool, self.dims, b, n)
            out[b], lse[b] = O.decode_sequence(V, kr, self.dims, q_abs[b], self.w.scale)
        return out, lse


def absorbed_queries(w, n_q, q_pos, tab_ora, q_scale=1.0):
    """Oracle q_abs (float64) for the workload's synthetic queries at positions q_pos."""
    M = synth.weights(w)
    q_nope, q_rope = synth.queries(w, n_q, q_scale)
    qt, r = O.absorb(q_nope, q_rope, q_pos, M, tab_ora)
    return O.q_abs_of(qt, r), (M, q_nope, q_rope)


def lse_ok(got, ref, tol):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):
        d = np.abs(np.where(both_inf, 0.0, got - ref))
    return bool(np.all(d <= tol)), float(np.max(d)) if d.size else 0.0
