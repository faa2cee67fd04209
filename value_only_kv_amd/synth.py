"""Seeded synthetic workloads for Grouped Value Attention (GVA) decode and prefill.

This module only draws random numbers and lays out integer bookkeeping (lengths,
positions, block tables). It holds none of the method's arithmetic: no rotation,
no rounding to the cache type, no attention. The device path and the CPU oracle
both take their inputs from here, so the two see identical data.

Shapes follow the notation of the GVA pages: T cached tokens, H query heads,
G value groups, d_h value width, d_n content-query width, d_r positional width
("Grouped Value Attention: Efficient KV Caching via On-Demand Key
Reconstruction", summary on agihunt.info; review on shibing624.github.io,
section 问题 and section 缓存账本).

Streams (numpy PCG64 through SeedSequence):
  * [1000 + k, 1 << 20]  weights and queries of config k: M, then q_nope, q_rope
  * [1000 + k, b]        sequence b of config k: V rows, then raw positional keys
  * [1000 + k, 99999]    config k's lengths, then its block permutation
  * [1000 + k, 1 << 22 | s] the non-absorbable comparator's maps and queries
  * [1000 + k, 1 << 23 | s] the latent comparator's absorbed queries
All values are drawn in float64 from N(0, 1) and cast to float32 once.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

WEIGHT_STREAM = 1 << 20
LAYOUT_STREAM = 99999


@dataclass(frozen=True)
class Workload:
    """One benchmark or parity configuration.

    lengths: cached tokens per sequence before the step (None: all equal T).
    append_one: the step appends one token at position len_b before decoding
      (the decode then reads len_b + 1 entries).
    chunk: number of new causal query tokens for a prefill workload (0: decode).
    """
    name: str
    index: int
    B: int
    T: int
    H: int
    G: int
    d_h: int
    d_n: int
    d_r: int
    dtype: str                 # "f32" or "bf16": element type of the cache
    block_size: int            # power of two; >= capacity means one block per sequence
    paged: bool                # True: seeded permutation of a shared block pool
    lengths_uniform: Optional[tuple] = None   # (lo, hi) inclusive, drawn per sequence
    append_one: bool = False
    chunk: int = 0
    base: float = 10000.0
    num_splits: tuple = ()     # split counts exercised for this workload
    note: str = ""

    @property
    def heads_per_group(self) -> int:
        return self.H // self.G

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_n + self.d_r))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def m_sigma(self) -> float:
        # Scale-matched initialisation with unit query and value variance: sigma_M^2 = 1 / d_in,
        # where d_in = d_h is the width of the value that M maps.
        return 1.0 / float(np.sqrt(self.d_h))


WORKLOADS = {
    "C1": Workload("C1", 0, B=1, T=256, H=8, G=4, d_h=64, d_n=64, d_r=16, dtype="f32",
                   block_size=256, paged=False, num_splits=(1, 2, 3, 4),
                   note="single decode step, fp32 cache, query at position T"),
    "C2": Workload("C2", 1, B=8, T=4096, H=16, G=4, d_h=64, d_n=64, d_r=16, dtype="bf16",
                   block_size=4096, paged=False, num_splits=(1, 8, 16),
                   note="350M-class layer, contiguous bf16 cache"),
    "C3": Workload("C3", 2, B=1, T=131072, H=32, G=8, d_h=128, d_n=128, d_r=16, dtype="bf16",
                   block_size=131072, paged=False, num_splits=(64, 128, 256),
                   note="long-context split-K decode, d_r=16"),
    "C3r24": Workload("C3r24", 2, B=1, T=131072, H=32, G=8, d_h=128, d_n=128, d_r=24,
                      dtype="bf16", block_size=131072, paged=False, num_splits=(64, 128, 256),
                      note="long-context split-K decode, d_r=24"),
    "C4": Workload("C4", 3, B=256, T=0, H=32, G=8, d_h=128, d_n=128, d_r=24, dtype="bf16",
                   block_size=16, paged=True, lengths_uniform=(512, 32768), append_one=True,
                   note="ragged paged batch: append one token, then decode over len+1"),
    "C5": Workload("C5", 4, B=4, T=8192, H=32, G=8, d_h=128, d_n=128, d_r=16, dtype="bf16",
                   block_size=16, paged=True, chunk=512, append_one=True,
                   note="chunked prefill of 512 causal queries over 8192 cached tokens, "
                        "then one decode step that appends one token"),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def _rng(w: Workload, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([1000 + w.index, stream]))


def _normal_f32(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float64)
    if sigma != 1.0:
        x = x * sigma
    return x.astype(np.float32)


def lengths(w: Workload) -> np.ndarray:
    """Cached tokens per sequence before the step (int64 [B])."""
    return _lengths_and_layout_rng(w)[0]


def _lengths_and_layout_rng(w: Workload):
    rng = _rng(w, LAYOUT_STREAM)
    if w.lengths_uniform is None:
        return np.full(w.B, w.T, dtype=np.int64), rng
    lo, hi = w.lengths_uniform
    return rng.integers(lo, hi + 1, size=w.B, dtype=np.int64), rng


def capacity(w: Workload, lens: np.ndarray) -> np.ndarray:
    """Tokens each sequence must hold after the step."""
    extra = w.chunk + (1 if w.append_one else 0)
    return lens + extra


@dataclass
class Layout:
    """Where each sequence's tokens live: a block table over a pool of blocks.

    V element (blk, tok, g, i) sits at v_offset = blk*v_sb + tok*v_st + g*v_sg + i and
    kr element (blk, tok, i) at blk*kr_sb + tok*kr_st + i (element offsets).
    """
    block_size: int
    num_blocks: int
    max_blocks: int
    block_table: np.ndarray        # int32 [B, max_blocks]; -1 marks an unused slot
    v_sb: int
    v_st: int
    v_sg: int
    kr_sb: int
    kr_st: int
    v_elems: int = field(default=0)
    kr_elems: int = field(default=0)


def layout(w: Workload, lens: np.ndarray, group_major: bool = True) -> Layout:
    """Block table and strides for workload w.

    Contiguous workloads use one block per sequence, laid out [B][T][G][d_h] with
    kr [B][T][d_r] (token-major). Paged workloads use blocks of block_size tokens laid
    out [blk][G][BS][d_h] (group_major=True) or [blk][BS][G][d_h], with kr [blk][BS][d_r],
    and a seeded permutation of the pool dealt to the sequences in order.
    """
    cap = capacity(w, lens)
    bs = w.block_size
    G, d_h, d_r = w.G, w.d_h, w.d_r
    if not w.paged:
        cap_max = int(cap.max())
        if bs < cap_max:
            raise ValueError("contiguous workload needs block_size >= capacity")
        table = np.arange(w.B, dtype=np.int32).reshape(w.B, 1)
        lay = Layout(bs, w.B, 1, table, v_sb=bs * G * d_h, v_st=G * d_h, v_sg=d_h,
                     kr_sb=bs * d_r, kr_st=d_r)
    else:
        nblk = (cap + bs - 1) // bs
        total = int(nblk.sum())
        rng = _lengths_and_layout_rng(w)[1]  # the permutation follows the lengths draw
        perm = rng.permutation(total).astype(np.int32)
        max_blocks = int(nblk.max())
        table = np.full((w.B, max_blocks), -1, dtype=np.int32)
        o = 0
        for b in range(w.B):
            n = int(nblk[b])
            table[b, :n] = perm[o:o + n]
            o += n
        if group_major:
            lay = Layout(bs, total, max_blocks, table, v_sb=G * bs * d_h, v_st=d_h,
                         v_sg=bs * d_h, kr_sb=bs * d_r, kr_st=d_r)
        else:
            lay = Layout(bs, total, max_blocks, table, v_sb=bs * G * d_h, v_st=G * d_h,
                         v_sg=d_h, kr_sb=bs * d_r, kr_st=d_r)
    lay.v_elems = lay.num_blocks * lay.v_sb
    lay.kr_elems = lay.num_blocks * lay.kr_sb
    return lay


def weights(w: Workload) -> np.ndarray:
    """Reconstruction maps M [H, d_h, d_n] float32, M ~ N(0, 1/d_h)."""
    rng = _rng(w, WEIGHT_STREAM)
    return _normal_f32(rng, (w.H, w.d_h, w.d_n), w.m_sigma)


def queries(w: Workload, n_q: int, q_scale: float = 1.0):
    """Raw query slices for n_q query tokens: q_nope [n_q, H, d_n], q_rope [n_q, H, d_r].

    q_scale multiplies both slices (a value > 1 makes the softmax peaky).
    """
    rng = _rng(w, WEIGHT_STREAM)
    rng.standard_normal(size=(w.H, w.d_h, w.d_n))  # M comes first on this stream
    q_nope = _normal_f32(rng, (n_q, w.H, w.d_n), q_scale)
    q_rope = _normal_f32(rng, (n_q, w.H, w.d_r), q_scale)
    return q_nope, q_rope


def sequence_tokens(w: Workload, b: int, n_tok: int):
    """Per-token inputs of sequence b for positions 0..n_tok-1.

    Returns v [n_tok, G, d_h] float32 and kr_raw [n_tok, d_r] float32 (not yet rotated).
    Rows are drawn position by position, so a prefix of a longer draw is identical.
    """
    rng = _rng(w, b)
    row = w.G * w.d_h + w.d_r
    x = rng.standard_normal(size=(n_tok, row), dtype=np.float64).astype(np.float32)
    v = np.ascontiguousarray(x[:, : w.G * w.d_h].reshape(n_tok, w.G, w.d_h))
    kr = np.ascontiguousarray(x[:, w.G * w.d_h:])
    return v, kr


def comparator_keys(w: Workload, b: int, n_tok: int) -> np.ndarray:
    """Keys of sequence b for a matched GQA cache (the comparator): [n_tok, G, d_h] float32 drawn
    from N(0, 1) on a stream of their own, [1000 + k, b, 2], position by position."""
    rng = np.random.default_rng(np.random.SeedSequence([1000 + w.index, b, 2]))
    x = rng.standard_normal(size=(n_tok, w.G * w.d_h), dtype=np.float64).astype(np.float32)
    return np.ascontiguousarray(x.reshape(n_tok, w.G, w.d_h))


def recon_inputs(w: Workload, stream: int = 3):
    """Inputs of the non-absorbable comparator on a stream of their own, [1000 + k, 1 << 22 |
    stream]: maps M ~ N(0, 1/d_h) held in bf16 (the model's weight type) and queries
    q ~ N(0, 1) [B, H, d_n] float32.

    Returns (q, M, Mt_bits): M [H, d_h, d_n] float64 holding exactly the bf16 values, and
    Mt_bits [H, d_n, d_h] uint16, the same values' bits transposed as the library takes them.
    The rounding to bf16 is torch's (float32 to bfloat16, nearest-even)."""
    import torch
    rng = _rng(w, (1 << 22) | stream)
    M32 = _normal_f32(rng, (w.H, w.d_h, w.d_n), 1.0 / float(np.sqrt(w.d_h)))
    q = _normal_f32(rng, (w.B, w.H, w.d_n))
    Mb = torch.from_numpy(M32).to(torch.bfloat16)
    M = Mb.to(torch.float64).numpy()
    Mt_bits = Mb.transpose(1, 2).contiguous().view(torch.int16).numpy().view(np.uint16)
    return q, M, Mt_bits


def mla_queries(w: Workload, H: int, d_c: int, d_r: int, stream: int = 1) -> np.ndarray:
    """Absorbed queries of the MLA-style latent comparator, [B, H, d_c + d_r] float32 N(0, 1), on
    a stream of their own, [1000 + k, 1 << 23 | stream]."""
    rng = _rng(w, (1 << 23) | stream)
    return _normal_f32(rng, (w.B, H, d_c + d_r))


def decode_query_positions(w: Workload, lens: np.ndarray) -> np.ndarray:
    """Position of each sequence's query token: the next position after the cached ones."""
    return lens.astype(np.int32)


def direct_q_abs(w: Workload, n_q: int, stream: int = 7) -> np.ndarray:
    """A random absorbed query [n_q, H, d_h + d_r] for decode-only tests (float32)."""
    rng = _rng(w, (1 << 21) + stream)
    return _normal_f32(rng, (n_q, w.H, w.d_h + w.d_r))
