"""Plain, slow, obviously correct CPU oracle for Grouped Value Attention (GVA) decode.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or executes this
module: only the tests, the smoke() check and bench.py's cpu_baseline leg do. It
shares no code with the HIP library and imports nothing from it; it computes in float64
with numpy (and Python's libm-backed math module for the RoPE angles).

Sources (web pages about arXiv:2609.13285, "Grouped Value Attention: Efficient KV
Caching via On-Demand Key Reconstruction"):
  [review]   shibing624.github.io review, "GVA：KV 缓存里的 Key 其实可以不存"
  [summary]  agihunt.info summary of the paper
  [abstract] hotpaper.ai page holding the paper's abstract
  [kvcache]  liumengxuan04.github.io, "KV Cache 优化（一）：从 MHA 到 MQA 与 GQA"

What the method computes (restated):
  * The cache keeps, per token, the G grouped values v_g (width d_h) and one positional
    key kr (width d_r) shared by every head, stored after its rotation
    ([review] section 关键技巧二; [summary]; [review] section 缓存账本, the N_GVA equation).
  * Head h has a map M_h of shape d_h x d_n; its content key would be K_h = V_{g(h)} M_h
    ([review] section 第二次尝试, the K_h equation).
  * Because M_h is fixed at inference, q_nope_h . (v M_h) = (q_nope_h M_h^T) . v exactly;
    q~_h = q_nope_h M_h^T is formed once per query token ([review] section 关键技巧一,
    the absorption identity; [summary] "absorption").
  * The score adds a content term and a positional term
    ([review] section 关键技巧二, the two-term score equation), then a softmax over the
    cached positions weights a sum over the same cached values ([summary]; [kvcache] §1,
    the decode-step attention equation).

Readings where the pages are silent:
  * RoPE pairs are interleaved (x_{2i}, x_{2i+1}); theta_i = base^(-2i/d_r), base 10000.
  * Rotation is done in float64 with each product and sum rounded separately, and the
    cache stores one round-to-nearest-even of that float64 value.
  * g(h) = h // (H/G) unless a map is given (Dims.g_of_h).
  * Decode attends to every cached entry j < len_b; prefill query i at position
    start_b + i attends to positions 0..start_b + i inclusive.
  * len_b = 0 gives output 0 and lse = -inf.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

# --------------------------------------------------------------------------------------
# O1: RoPE angle table.  Readings: interleaved pairs, theta_i = base^(-2i/d_r).
# [review] section 关键技巧二 only fixes that a d_r-wide slice is rotated by position; the
# frequencies are the conventional RoPE ones.
# --------------------------------------------------------------------------------------


def rope_theta(d_r: int, base: float) -> list:
    """Per-pair frequencies theta_i = base ** (-2 i / d_r), i in [0, d_r/2)."""
    return [base ** (-2 * i / d_r) for i in range(d_r // 2)]


def rope_table(max_pos: int, d_r: int, base: float = 10000.0) -> np.ndarray:
    """float64 [max_pos, d_r/2, 2]: (cos, sin) of p * theta_i, each from libm (math)."""
    th = rope_theta(d_r, base)
    out = np.empty((max_pos, d_r // 2, 2), dtype=np.float64)
    cos, sin = math.cos, math.sin
    for i, t in enumerate(th):
        col_c = out[:, i, 0]
        col_s = out[:, i, 1]
        for p in range(max_pos):
            a = p * t
            col_c[p] = cos(a)
            col_s[p] = sin(a)
    return out


def rope_rows(positions: np.ndarray, d_r: int, base: float = 10000.0) -> np.ndarray:
    """Only the table rows at the given positions: float64 [n, d_r/2, 2]."""
    th = rope_theta(d_r, base)
    pos = np.asarray(positions).reshape(-1)
    out = np.empty((pos.size, d_r // 2, 2), dtype=np.float64)
    for k, p in enumerate(pos.tolist()):
        for i, t in enumerate(th):
            a = p * t
            out[k, i, 0] = math.cos(a)
            out[k, i, 1] = math.sin(a)
    return out


# --------------------------------------------------------------------------------------
# O2: rotation of interleaved pairs at one position, float64, no fused multiply-add.
# --------------------------------------------------------------------------------------


def rotate(x: np.ndarray, cs: np.ndarray) -> np.ndarray:
    """Rotate pairs (x_{2i}, x_{2i+1}) by the angle whose (cos, sin) is cs[..., i, :].

    x: [..., d_r] (any float type, promoted exactly to float64); cs: [..., d_r/2, 2]
    broadcastable against x's leading axes. y_{2i} = x_{2i} c - x_{2i+1} s and
    y_{2i+1} = x_{2i} s + x_{2i+1} c, each product and each sum rounded to float64.
    """
    x = np.asarray(x, dtype=np.float64)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    c = cs[..., 0]
    s = cs[..., 1]
    a = x0 * c
    b = x1 * s
    y0 = a - b
    a = x0 * s
    b = x1 * c
    y1 = a + b
    y = np.empty(np.broadcast(x0, c).shape[:-1] + (x.shape[-1],), dtype=np.float64)
    y[..., 0::2] = y0
    y[..., 1::2] = y1
    return y


# --------------------------------------------------------------------------------------
# O3: cast to the cache element type with one round-to-nearest-even.
# bfloat16: 8 significant bits and float32's exponent range. The rounding is done on
# the value with frexp / rint / ldexp, never through float32 (that would round twice).
# --------------------------------------------------------------------------------------

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                     # |x| in [2^(e-1), 2^e)
    q = np.maximum(e - 8, -133)            # quantum exponent: 8 bits, or subnormal 2^-133
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)   # np.rint rounds half to even, exactly
    y = np.where(np.abs(y) > BF16_MAX, np.copysign(np.inf, x), y)
    return np.where(np.isfinite(x), y, x)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns (uint16), via round_bf16 (exact in float32)."""
    y = round_bf16(x).astype(np.float32)   # exact: every bfloat16 value is a float32 value
    return (y.view(np.uint32) >> 16).astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 values (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f32_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 bit patterns with one round-to-nearest-even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)


def f32_value(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def to_cache_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else f32_bits(x)


def from_cache_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_value(bits) if dtype == "bf16" else f32_value(bits)


# --------------------------------------------------------------------------------------
# O4: the cache and its append.  One layer's cache holds G value streams plus one shared
# positional-key stream ([review] section 缓存账本, N_GVA = T G d_h + T d_r; [summary]).
# Paging (a block table over a pool of fixed-size blocks) changes where entries live,
# not what attention computes ([kvcache] §7, the PagedAttention remark).
# --------------------------------------------------------------------------------------

ERR_BLOCK = 1       # a block-table entry outside [0, num_blocks)
ERR_CAPACITY = 2    # a position beyond the block table's capacity (max_blocks * block_size)
ERR_ROPE = 4        # a position at or beyond the RoPE table (max_pos)
ERR_SEQ = 8         # a sequence index outside [0, B)
ERR_LENGTH = 16     # a length or position that is negative, or a length above max_len


@dataclass
class Dims:
    H: int
    G: int
    d_h: int
    d_n: int
    d_r: int
    # g(h) for every head h, or None for the contiguous map h // (H/G). Heads are partitioned into
    # groups that share one cached value stream ([kvcache] section 4; [review] section 第二次尝试);
    # the pages draw the groups contiguous but nothing in the method depends on it.
    g_of_h: Optional[tuple] = None

    def group_of(self, h: int) -> int:
        if self.g_of_h is not None:
            return int(self.g_of_h[h])
        return h // (self.H // self.G)


@dataclass
class Pool:
    """The oracle's own copy of a cache: raw element bits at the same offsets as the device.

    V(blk, tok, g, i) is v[blk*v_sb + tok*v_st + g*v_sg + i]; kr(blk, tok, i) is
    kr[blk*kr_sb + tok*kr_st + i]. block_table[b][k] names the block holding positions
    k*block_size .. (k+1)*block_size - 1 of sequence b.
    """
    dtype: str
    v: np.ndarray
    kr: np.ndarray
    v_sb: int
    v_st: int
    v_sg: int
    kr_sb: int
    kr_st: int
    num_blocks: int
    block_size: int
    block_table: np.ndarray

    @staticmethod
    def empty(dtype, v_elems, kr_elems, strides, num_blocks, block_size, block_table,
              sentinel=None):
        bits = np.uint16 if dtype == "bf16" else np.uint32
        fill = sentinel if sentinel is not None else 0
        v = np.full(v_elems, fill, dtype=bits)
        kr = np.full(kr_elems, fill, dtype=bits)
        v_sb, v_st, v_sg, kr_sb, kr_st = strides
        return Pool(dtype, v, kr, v_sb, v_st, v_sg, kr_sb, kr_st, num_blocks, block_size,
                    np.asarray(block_table, dtype=np.int64))

    def slot(self, b: int, p: int):
        """(block, offset) of position p of sequence b."""
        return int(self.block_table[b][p // self.block_size]), p % self.block_size


def append(pool: Pool, dims: Dims, seq, pos, v_new, kr_raw, table: np.ndarray) -> int:
    """Write n new tokens into the pool; returns the error bits that a bad token raises.

    Token k belongs to sequence seq[k] at position pos[k]. Its G values are stored
    after one rounding to the cache type; its positional key is rotated to pos[k] in
    float64 and stored after one rounding ([review] section 关键技巧二: the shared
    positional key is cached already rotated; [kvcache] §1: the new token's state is
    appended before the query reads the history). A token with a bad index is skipped.
    """
    seq = np.asarray(seq, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    v_new = np.asarray(v_new)
    kr_raw = np.asarray(kr_raw)
    B = pool.block_table.shape[0]
    cap = pool.block_table.shape[1] * pool.block_size
    err = 0
    ok = np.ones(seq.size, dtype=bool)
    for k in range(seq.size):
        b, p = int(seq[k]), int(pos[k])
        if b < 0 or b >= B:
            err |= ERR_SEQ
            ok[k] = False
            continue
        if p < 0:
            err |= ERR_LENGTH
            ok[k] = False
            continue
        if p >= cap:
            err |= ERR_CAPACITY
            ok[k] = False
            continue
        if p >= table.shape[0]:
            err |= ERR_ROPE
            ok[k] = False
            continue
        blk = int(pool.block_table[b][p // pool.block_size])
        if blk < 0 or blk >= pool.num_blocks:
            err |= ERR_BLOCK
            ok[k] = False
    idx = np.nonzero(ok)[0]
    if idx.size == 0:
        return err
    b = seq[idx]
    p = pos[idx]
    blk = pool.block_table[b, p // pool.block_size]
    off = p % pool.block_size
    # values: one rounding each
    g = np.arange(dims.G)
    i = np.arange(dims.d_h)
    vo = (blk[:, None, None] * pool.v_sb + off[:, None, None] * pool.v_st
          + g[None, :, None] * pool.v_sg + i[None, None, :])
    pool.v[vo] = to_cache_bits(np.asarray(v_new[idx], dtype=np.float64), pool.dtype)
    # positional key: rotate at its own position in float64, then one rounding
    rot = rotate(kr_raw[idx], table[p])
    j = np.arange(dims.d_r)
    ko = blk[:, None] * pool.kr_sb + off[:, None] * pool.kr_st + j[None, :]
    pool.kr[ko] = to_cache_bits(rot, pool.dtype)
    return err


def gather(pool: Pool, dims: Dims, b: int, n: int):
    """Positions 0..n-1 of sequence b as exact float64: V [n, G, d_h], kr [n, d_r]."""
    p = np.arange(n, dtype=np.int64)
    blk = pool.block_table[b, p // pool.block_size]
    off = p % pool.block_size
    g = np.arange(dims.G)
    i = np.arange(dims.d_h)
    vo = (blk[:, None, None] * pool.v_sb + off[:, None, None] * pool.v_st
          + g[None, :, None] * pool.v_sg + i[None, None, :])
    j = np.arange(dims.d_r)
    ko = blk[:, None] * pool.kr_sb + off[:, None] * pool.kr_st + j[None, :]
    return from_cache_bits(pool.v[vo], pool.dtype), from_cache_bits(pool.kr[ko], pool.dtype)


# --------------------------------------------------------------------------------------
# O5: query absorption.  q~_h = q_nope_h M_h^T (so q~_h[i] = sum_k M_h[i, k] q_nope_h[k]),
# once per query token ([review] section 关键技巧一); the positional slice of the query is
# rotated at the query's position ([review] section 关键技巧二).
# --------------------------------------------------------------------------------------


def absorb(q_nope, q_rope, q_pos, M, table: np.ndarray):
    """Returns (q~ [n, H, d_h], r [n, H, d_r]) in float64."""
    qn = np.asarray(q_nope, dtype=np.float64)
    Mh = np.asarray(M, dtype=np.float64)
    qt = np.einsum("hik,nhk->nhi", Mh, qn)
    cs = table[np.asarray(q_pos, dtype=np.int64)]          # [n, d_r/2, 2]
    r = rotate(q_rope, cs[:, None, :, :])
    return qt, r


def q_abs_of(qt: np.ndarray, r: np.ndarray) -> np.ndarray:
    """The absorbed query laid out as the library expects: [n, H, d_h + d_r]."""
    return np.concatenate([qt, r], axis=-1)


# --------------------------------------------------------------------------------------
# O6: decode, absorbed form.  s_j = scale (q~_h . v_{j,g(h)} + r_h . kr_j); softmax over
# the cached positions; output = sum_j w_j v_{j,g(h)}; lse = m + ln sum_j e^(s_j - m).
# ([review] 关键技巧一 and 关键技巧二; [kvcache] §1 decode-step attention.)
# --------------------------------------------------------------------------------------


def softmax_attend(s: np.ndarray, V: np.ndarray):
    """Softmax of scores s [n] followed by the weighted sum of rows V [n, d]."""
    if s.size == 0:
        return np.zeros(V.shape[1]), -np.inf, np.zeros(0)
    m = np.max(s)
    e = np.exp(s - m)
    z = np.sum(e)
    w = e / z
    return w @ V, m + math.log(z), w


def decode(pool: Pool, dims: Dims, seq_len, q_abs, scale: float):
    """Decode every (b, h): returns out [B, H, d_h] and lse [B, H] in float64.

    q_abs [B, H, d_h + d_r]: q~_h followed by the rotated positional query r_h.
    """
    q_abs = np.asarray(q_abs, dtype=np.float64)
    B = len(seq_len)
    out = np.zeros((B, dims.H, dims.d_h))
    lse = np.full((B, dims.H), -np.inf)
    for b in range(B):
        n = int(seq_len[b])
        if n == 0:
            continue
        V, kr = gather(pool, dims, b, n)
        for h in range(dims.H):
            g = dims.group_of(h)
            qt = q_abs[b, h, :dims.d_h]
            r = q_abs[b, h, dims.d_h:]
            s = scale * (V[:, g, :] @ qt + kr @ r)
            out[b, h], lse[b, h], _ = softmax_attend(s, V[:, g, :])
    return out, lse


def decode_sequence(V: np.ndarray, kr: np.ndarray, dims: Dims, q_abs_b, scale: float):
    """Decode one sequence from already gathered V [n, G, d_h] and kr [n, d_r]."""
    q_abs_b = np.asarray(q_abs_b, dtype=np.float64)
    out = np.zeros((dims.H, dims.d_h))
    lse = np.full(dims.H, -np.inf)
    if V.shape[0] == 0:
        return out, lse
    S = kr @ q_abs_b[:, dims.d_h:].T                       # positional term [n, H]
    for g in range(dims.G):
        hs = [h for h in range(dims.H) if dims.group_of(h) == g]
        Sg = V[:, g, :] @ q_abs_b[hs, :dims.d_h].T          # content term [n, |hs|]
        for k, h in enumerate(hs):
            s = scale * (Sg[:, k] + S[:, h])
            out[h], lse[h], _ = softmax_attend(s, V[:, g, :])
    return out, lse


# --------------------------------------------------------------------------------------
# O6': decode with the content keys written out: K_h = V_{g(h)} M_h and the score
# q_nope_h . K_h[j] + r_h . kr_j ([review] section 第二次尝试 and section 关键技巧二).
# Used only to check the absorbed form.
# --------------------------------------------------------------------------------------


def decode_materialized(V: np.ndarray, kr: np.ndarray, dims: Dims, q_nope_b, r_b, M,
                        scale: float):
    """One sequence; V [n, G, d_h], kr [n, d_r], q_nope_b [H, d_n], r_b [H, d_r]."""
    q_nope_b = np.asarray(q_nope_b, dtype=np.float64)
    r_b = np.asarray(r_b, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    out = np.zeros((dims.H, dims.d_h))
    lse = np.full(dims.H, -np.inf)
    for h in range(dims.H):
        g = dims.group_of(h)
        K = V[:, g, :] @ M[h]                                # [n, d_n]
        s = scale * (K @ q_nope_b[h] + kr @ r_b[h])
        out[h], lse[h], _ = softmax_attend(s, V[:, g, :])
    return out, lse


# --------------------------------------------------------------------------------------
# GQA comparator: what a matched grouped-query model caches and reads per step, G keys and
# G values per token ([kvcache] section 4: the query heads of a group share one key head and
# one value head), decoded with the textbook step ([kvcache] section 1). Keys are cached as
# the model produced them (any rotation already applied), so the score of head h at cached
# position j is scale * q_h . k_{j, g(h)}.
# --------------------------------------------------------------------------------------


def gqa_decode_sequence(K: np.ndarray, V: np.ndarray, dims: Dims, q_b, scale: float):
    """One sequence; K, V [n, G, d_h] (the cached values in float64), q_b [H, d_h]."""
    q_b = np.asarray(q_b, dtype=np.float64)
    out = np.zeros((dims.H, dims.d_h))
    lse = np.full(dims.H, -np.inf)
    if V.shape[0] == 0:
        return out, lse
    for h in range(dims.H):
        g = dims.group_of(h)
        s = scale * (K[:, g, :] @ q_b[h])
        out[h], lse[h], _ = softmax_attend(s, V[:, g, :])
    return out, lse


# --------------------------------------------------------------------------------------
# Non-absorbable variant (comparator).  The scale-matched row applies ordinary RoPE to the
# reconstructed content key, which is why its map cannot be absorbed into the query
# ([summary], the scale-matched + query RMSNorm row; [review] section 第二次尝试 for
# K_h = V_g M_h). Its cache holds the G value streams only: position enters through the key.
# Head h's key at position j is k_{h,j} = R_j (M_h^T v_{j,g(h)}) (width d_n), its query at
# position p is R_p q_h, and s_j = scale (R_p q_h) . k_{h,j}; the softmax and the weighted sum
# over the cached values are O6's.
# Readings: RoPE over all d_n dims of the key, interleaved pairs, theta_i = base^(-2i/d_n)
# (O1's convention at width d_n); the query arrives already normalised (the row's query
# RMSNorm acts before attention, on the query projection).
# --------------------------------------------------------------------------------------


def recon_decode_sequence(V: np.ndarray, dims: Dims, q_b, p: int, M, scale: float,
                          base: float = 10000.0, key_pos=None):
    """One sequence; V [n, G, d_h] (cached values, float64), q_b [H, d_n], M [H, d_h, d_n].

    The query sits at position p; key j sits at key_pos[j] (default j).
    Returns out [H, d_h] and lse [H] (float64).
    """
    q_b = np.asarray(q_b, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    n = V.shape[0]
    out = np.zeros((dims.H, dims.d_h))
    lse = np.full(dims.H, -np.inf)
    if n == 0:
        return out, lse
    kp = np.arange(n) if key_pos is None else np.asarray(key_pos)
    cs_k = rope_rows(kp, dims.d_n, base)                   # [n, d_n/2, 2]
    cs_q = rope_rows(np.array([p]), dims.d_n, base)[0]     # [d_n/2, 2]
    for h in range(dims.H):
        g = dims.group_of(h)
        K = rotate(V[:, g, :] @ M[h], cs_k)                # k_{h,j} = R_j (M_h^T v_j), [n, d_n]
        s = scale * (K @ rotate(q_b[h], cs_q))
        out[h], lse[h], _ = softmax_attend(s, V[:, g, :])
    return out, lse


def recon_decode_flops(len_b: int, H: int, d_h: int, d_n: int) -> int:
    """Multiply-adds x 2 of one step of one sequence: key rebuild, score and weighted sum."""
    return H * len_b * (2 * d_h * d_n + 2 * d_n + 2 * d_h)


# --------------------------------------------------------------------------------------
# MLA-style latent comparator. MLA caches one joint latent of width d_c plus a shared RoPE
# channel, T (d_c + d_r) scalars, and projects keys and values back up from the latent at
# decode ([review] section 问题; [mla] section 3.1 for the up-projections W^UK and W^UV).
# With the key up-projection folded into the query, q~_h = W^UK_h q_nope_h, its decode is the
# absorbed decode above with one group whose cached "value" is the latent: decode_sequence
# with G = 1 and d_h = d_c; the value up-projection multiplies the latent output afterwards.
# mla_decode_materialized writes the textbook form out (every head's keys and values projected
# up from the latents) to check that identity.
# --------------------------------------------------------------------------------------


def mla_cache_scalars(T: int, d_c: int, d_r: int) -> int:
    """Scalars one layer's MLA cache holds: T (d_c + d_r)."""
    return T * (d_c + d_r)


def mla_decode_materialized(C: np.ndarray, kr: np.ndarray, q_nope_b, r_b, W_uk, W_uv,
                            scale: float):
    """One sequence; C [n, d_c] cached latents, kr [n, d_r] cached (rotated) positional keys,
    q_nope_b [H, d_k], r_b [H, d_r] rotated positional queries, W_uk [H, d_c, d_k],
    W_uv [H, d_c, d_v]. Keys K_h = C W_uk[h], values V_h = C W_uv[h]; returns out [H, d_v]
    and lse [H] (float64)."""
    C = np.asarray(C, dtype=np.float64)
    kr = np.asarray(kr, dtype=np.float64)
    q_nope_b = np.asarray(q_nope_b, dtype=np.float64)
    r_b = np.asarray(r_b, dtype=np.float64)
    H = q_nope_b.shape[0]
    out = np.zeros((H, W_uv.shape[2]))
    lse = np.full(H, -np.inf)
    for h in range(H):
        K = C @ np.asarray(W_uk[h], dtype=np.float64)
        V = C @ np.asarray(W_uv[h], dtype=np.float64)
        s = scale * (K @ q_nope_b[h] + kr @ r_b[h])
        out[h], lse[h], _ = softmax_attend(s, V)
    return out, lse


# --------------------------------------------------------------------------------------
# O7: chunked prefill.  The chunk's tokens are appended first (O4); query i of sequence b
# sits at position start_b + i and attends to positions 0..start_b + i (inclusive), over
# the cache-rounded values ([summary]: prefill is a dense, matrix-heavy pass).
# --------------------------------------------------------------------------------------


def prefill(pool: Pool, dims: Dims, start, chunk_len: int, q_abs, v_new, kr_raw,
            scale: float, table: np.ndarray):
    """q_abs [B, C, H, d_h + d_r], v_new [B, C, G, d_h], kr_raw [B, C, d_r].

    Returns out [B, C, H, d_h], lse [B, C, H] (float64) and the append error bits.
    """
    B = len(start)
    C = chunk_len
    q_abs = np.asarray(q_abs, dtype=np.float64)
    seq = np.repeat(np.arange(B), C)
    pos = (np.asarray(start, dtype=np.int64)[:, None] + np.arange(C)[None, :]).reshape(-1)
    err = append(pool, dims, seq, pos, np.asarray(v_new).reshape(B * C, dims.G, dims.d_h),
                 np.asarray(kr_raw).reshape(B * C, dims.d_r), table)
    out = np.zeros((B, C, dims.H, dims.d_h))
    lse = np.full((B, C, dims.H), -np.inf)
    for b in range(B):
        P0 = int(start[b])
        V, kr = gather(pool, dims, b, P0 + C)
        S_pos = kr @ q_abs[b, :, :, dims.d_h:].reshape(C * dims.H, dims.d_r).T  # [n, C*H]
        S_pos = S_pos.reshape(P0 + C, C, dims.H)
        for g in range(dims.G):
            hs = [h for h in range(dims.H) if dims.group_of(h) == g]
            for h in hs:
                Sc = V[:, g, :] @ q_abs[b, :, h, :dims.d_h].T               # [n, C]
                for i in range(C):
                    n = P0 + i + 1
                    s = scale * (Sc[:n, i] + S_pos[:n, i, h])
                    out[b, i, h], lse[b, i, h], _ = softmax_attend(s, V[:n, g, :])
    return out, lse, err


# --------------------------------------------------------------------------------------
# O8: the same decode taken over contiguous chunks of positions and merged through the
# log-sum-exp of each chunk (a re-association of the softmax sums, not in the pages).
# --------------------------------------------------------------------------------------


def decode_partials(s: np.ndarray, V: np.ndarray, chunk: int, num_splits: int):
    """Per-chunk (m, l, o) with o unnormalised; empty chunks give (-inf, 0, 0)."""
    parts = []
    for c in range(num_splits):
        lo, hi = c * chunk, min((c + 1) * chunk, s.size)
        if lo >= hi:
            parts.append((-np.inf, 0.0, np.zeros(V.shape[1])))
            continue
        m = np.max(s[lo:hi])
        e = np.exp(s[lo:hi] - m)
        parts.append((m, float(np.sum(e)), e @ V[lo:hi]))
    return parts


def combine(parts):
    """Merge chunk partials: m* = max m_c, L = sum l_c e^(m_c - m*), o = sum o_c e^(m_c - m*) / L."""
    ms = np.array([p[0] for p in parts])
    if ms.size == 0 or np.all(np.isneginf(ms)):
        return np.zeros_like(parts[0][2]) if parts else None, -np.inf
    mx = np.max(ms)
    L = 0.0
    o = np.zeros_like(parts[0][2])
    for m, l, oc in parts:
        if np.isneginf(m):
            continue
        f = math.exp(m - mx)
        L += l * f
        o = o + oc * f
    return o / L, mx + math.log(L)


# --------------------------------------------------------------------------------------
# O9: cache accounting ([review] section 问题 and section 缓存账本; [kvcache] §2-§5).
# --------------------------------------------------------------------------------------


def gva_cache_scalars(T: int, G: int, d_h: int, d_r: int) -> int:
    """Scalars one layer's GVA cache holds for T tokens: T (G d_h + d_r)."""
    return T * (G * d_h + d_r)


def gqa_cache_scalars(T: int, G: int, d_h: int) -> int:
    """Scalars a matched GQA cache holds: 2 T G d_h (a key and a value per group)."""
    return 2 * T * G * d_h


def mha_cache_scalars(T: int, H: int, d_h: int) -> int:
    return 2 * T * H * d_h


def kv_cache_bytes(layers: int, batch: int, T: int, kv_heads: int, d_h: int,
                   elem_bytes: int) -> int:
    """Bytes of a key/value cache with kv_heads key heads and as many value heads."""
    return 2 * layers * batch * T * kv_heads * d_h * elem_bytes


def gqa_decode_bytes(len_b: int, G: int, d_h: int, elem_bytes: int) -> int:
    """Cache bytes one GQA decode step of a sequence reads: every key and value, once."""
    return len_b * gqa_cache_scalars(1, G, d_h) * elem_bytes


def gva_decode_bytes(len_b: int, G: int, d_h: int, d_r: int, elem_bytes: int) -> int:
    """Cache bytes one decode step of one sequence must read once: len (G d_h + d_r) s."""
    return len_b * (G * d_h + d_r) * elem_bytes


def gva_decode_flops(len_b: int, H: int, d_h: int, d_r: int) -> int:
    """Multiply-adds x 2 of one decode step of one sequence, all heads."""
    return H * len_b * (2 * (d_h + d_r) + 2 * d_h)
