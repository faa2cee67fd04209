"""GPU parity at the full sizes the benchmark runs, in its launch configuration (automatic split
count), on outputs the oracle computes one sequence at a time.

* One sequence of T = 131072 cached positions (H=32, G=8, d_h=d_n=128, d_r=16 and 24), decoded
  with 64, 128 and 256 splits and the automatic count: every head against the oracle.
* The ragged paged batch (B=256, lengths U[512, 32768], d_r=24, 16-token blocks in a seeded
  permutation of the pool): append one token per sequence, absorb the queries, decode over
  len_b + 1 positions. Six sampled sequences (the longest, the shortest and four drawn at random)
  carry the seeded synthetic tokens and are checked against the oracle; the other sequences are
  filled with device random values, which only they read. The non-absorbable comparator runs on
  the same cache and is checked on three of the sampled sequences.
"""
import numpy as np
import pytest
import torch

from oracle import gva_oracle as O
from value_only_kv_amd import binding as gb
from value_only_kv_amd import synth
from tests.gpu_cases import SENTINEL, Case, absorbed_queries, check_output, lse_ok

pytestmark = pytest.mark.gpu


def _device_absorb(cdims, w, q_nope, q_rope, q_pos, M, tab, max_pos):
    n = q_nope.shape[0]
    out = torch.empty((n, w.H, w.d_h + w.d_r), device="cuda")
    gb.gva_absorb_query(cdims, torch.from_numpy(q_nope).cuda(), torch.from_numpy(q_rope).cuda(),
                        torch.from_numpy(np.asarray(q_pos, np.int32)).cuda(),
                        torch.from_numpy(M).cuda(), tab, max_pos, out)
    return out.cpu().numpy()


@pytest.mark.parametrize("name", ["C3", "C3r24"])
def test_long_context_full_size(name):
    w = synth.workload(name)
    c = Case(w, sentinel=False)
    c.append_prefix()
    T = int(c.lens[0])
    q_ref, (M, q_nope, q_rope) = absorbed_queries(w, 1, [T], c.tab_ora)
    q_dev = _device_absorb(c.cdims, w, q_nope, q_rope, [T], M, c.tab_lib, c.max_pos)
    ref, ref_lse = c.oracle_decode([T], q_ref)
    for S in (64, 128, 256, 0):
        out, lse = c.decode([T], q_dev, num_splits=S)
        check_output(out, ref, "bf16", f"{name} T={T} S={S}")
        ok, e = lse_ok(lse, ref_lse, 1e-3)
        assert ok, (S, e)
    assert c.err_flag() == 0


@pytest.fixture(scope="module")
def ragged():
    """The full ragged batch, built once for the tests below: sampled sequences carry their
    seeded synthetic tokens (the appended step token included), the others device random values."""
    w = synth.workload("C4")
    lens = synth.lengths(w)
    lay = synth.layout(w, lens)
    B, G, d_h, d_r, H = w.B, w.G, w.d_h, w.d_r, w.H
    cdims = gb.GvaDims(H, G, d_h, w.d_n, d_r)
    max_pos = int(synth.capacity(w, lens).max()) + 1
    tab_lib = torch.from_numpy(gb.gva_rope_table_fill(max_pos, d_r, w.base)).cuda()
    # every element starts as a NaN sentinel that no append of finite data can produce
    cache = gb.GvaCache.allocate(cdims, w.dtype, lay.num_blocks, lay.block_size,
                                 torch.from_numpy(lay.block_table).cuda(), tab_lib,
                                 (lay.v_sb, lay.v_st, lay.v_sg, lay.kr_sb, lay.kr_st),
                                 fill_bits=SENTINEL["bf16"])
    rng = np.random.default_rng(17)
    sampled = sorted({int(np.argmax(lens)), int(np.argmin(lens)),
                      *(int(x) for x in rng.choice(B, 4, replace=False))})
    print(f"sampled sequences {sampled}, lengths {[int(lens[b]) for b in sampled]}", flush=True)

    # filler: positions 0 .. len_b - 1 of the other sequences, device random values
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    others = [b for b in range(B) if b not in sampled]
    seqs = np.repeat(np.asarray(others, np.int32), lens[others])
    poss = np.concatenate([np.arange(lens[b], dtype=np.int32) for b in others])
    for o in range(0, seqs.size, 1 << 16):
        n = min(1 << 16, seqs.size - o)
        gb.gva_cache_append(cdims, cache, B, torch.from_numpy(seqs[o:o + n]).cuda(),
                            torch.from_numpy(poss[o:o + n]).cuda(),
                            torch.randn((n, G, d_h), generator=gen, device="cuda"),
                            torch.randn((n, d_r), generator=gen, device="cuda"))
    # sampled sequences: their seeded tokens; position len_b is appended as the step's token
    toks = {}
    for b in sampled:
        n = int(lens[b])
        v, kr = synth.sequence_tokens(w, b, n + 1)
        toks[b] = (v, kr)
        gb.gva_cache_append(cdims, cache, B, torch.full((n,), b, dtype=torch.int32).cuda(),
                            torch.arange(n, dtype=torch.int32).cuda(),
                            torch.from_numpy(v[:n]).cuda(), torch.from_numpy(kr[:n]).cuda())
    # the step: append one token per sequence at position len_b
    v_step = torch.randn((B, G, d_h), generator=gen, device="cuda")
    k_step = torch.randn((B, d_r), generator=gen, device="cuda")
    for b in sampled:
        v_step[b] = torch.from_numpy(toks[b][0][-1]).cuda()
        k_step[b] = torch.from_numpy(toks[b][1][-1]).cuda()
    pos = lens.astype(np.int32)
    gb.gva_cache_append(cdims, cache, B, torch.arange(B, dtype=torch.int32).cuda(),
                        torch.from_numpy(pos).cuda(), v_step, k_step)
    torch.cuda.synchronize()
    return dict(w=w, lens=lens, lay=lay, cdims=cdims, dims=O.Dims(H, G, d_h, w.d_n, d_r),
                cache=cache, tab_lib=tab_lib, max_pos=max_pos, sampled=sampled, toks=toks,
                pos=pos, v_step=v_step.cpu().numpy(), k_step=k_step.cpu().numpy())


def _sequence_values(r, b):
    """The oracle's own contiguous pool for sampled sequence b: V [n, G, d_h] and kr [n, d_r]."""
    w, dims = r["w"], r["dims"]
    G, d_h, d_r = w.G, w.d_h, w.d_r
    n = int(r["lens"][b]) + 1
    v, kr = r["toks"][b]
    tab_ora = O.rope_rows(np.arange(n), d_r, w.base)
    pool = O.Pool.empty("bf16", n * G * d_h, n * d_r, (n * G * d_h, G * d_h, d_h, n * d_r, d_r),
                        1, 1 << int(np.ceil(np.log2(n))), np.zeros((1, 1)))
    O.append(pool, dims, np.zeros(n, np.int64), np.arange(n), v, kr, tab_ora)
    return O.gather(pool, dims, 0, n)


def _device_blocks(cache, lay, ids):
    """Raw bits (uint16) of whole blocks `ids` of the device pool: V [n, v_sb], kr [n, kr_sb]."""
    idx = torch.from_numpy(np.asarray(ids, np.int64)).cuda()
    v = cache.v.view(torch.int16).view(lay.num_blocks, lay.v_sb)[idx]
    kr = cache.kr.view(torch.int16).view(lay.num_blocks, lay.kr_sb)[idx]
    torch.cuda.synchronize()
    return v.cpu().numpy().view(np.uint16), kr.cpu().numpy().view(np.uint16)


def test_ragged_batch_full_size_cache_bits(ragged):
    """The cache append at full size, bit for bit. (1) Every block a sampled sequence owns
    (its whole history and its step token, and the sentinel in the slots past its end) equals the
    block the oracle's own append writes from the same tokens into a pool of the same layout.
    (2) The step token of every one of the 256 sequences, at position len_b in the seeded
    permutation of the pool, equals the oracle's rounding of that token (rotated at len_b)."""
    r = ragged
    w, lay, dims, cache, lens, pos = r["w"], r["lay"], r["dims"], r["cache"], r["lens"], r["pos"]
    strides = (lay.v_sb, lay.v_st, lay.v_sg, lay.kr_sb, lay.kr_st)
    tab = O.rope_table(r["max_pos"], w.d_r, w.base)
    for b in r["sampled"]:
        n = int(lens[b]) + 1
        nblk = -(-n // lay.block_size)
        ids = lay.block_table[b, :nblk]
        pool = O.Pool.empty("bf16", nblk * lay.v_sb, nblk * lay.kr_sb, strides, nblk,
                            lay.block_size, np.arange(nblk)[None, :], sentinel=SENTINEL["bf16"])
        v, kr = r["toks"][b]
        assert O.append(pool, dims, np.zeros(n, np.int64), np.arange(n), v, kr, tab) == 0
        dv, dk = _device_blocks(cache, lay, ids)
        assert np.array_equal(dv.reshape(-1), pool.v), f"value blocks of sequence {b}"
        assert np.array_equal(dk.reshape(-1), pool.kr), f"positional-key blocks of sequence {b}"
    # the step tokens of all sequences: one block per sequence in the oracle's pool
    B = w.B
    table = np.full((B, lay.max_blocks), -1, np.int64)
    table[np.arange(B), pos // lay.block_size] = np.arange(B)
    pool = O.Pool.empty("bf16", B * lay.v_sb, B * lay.kr_sb, strides, B, lay.block_size, table,
                        sentinel=SENTINEL["bf16"])
    assert O.append(pool, dims, np.arange(B), pos, r["v_step"], r["k_step"], tab) == 0
    ids = lay.block_table[np.arange(B), pos // lay.block_size]
    dv, dk = _device_blocks(cache, lay, ids)
    off = pos % lay.block_size
    g = np.arange(w.G)[None, :, None]
    i = np.arange(w.d_h)[None, None, :]
    vo = g * lay.v_sg + off[:, None, None] * lay.v_st + i                       # [B, G, d_h]
    ko = off[:, None] * lay.kr_st + np.arange(w.d_r)[None, :]                   # [B, d_r]
    bsel = np.arange(B)
    got_v = dv[bsel[:, None, None], vo]
    want_v = pool.v.reshape(B, lay.v_sb)[bsel[:, None, None], vo]
    got_k = dk[bsel[:, None], ko]
    want_k = pool.kr.reshape(B, lay.kr_sb)[bsel[:, None], ko]
    assert np.array_equal(got_v, want_v) and np.array_equal(got_k, want_k)
    assert int(cache.err_flag.item()) == 0


def test_ragged_batch_full_size_sampled_sequences(ragged):
    """Absorb the queries and decode over len_b + 1 positions, as the bench does."""
    r = ragged
    w, cdims, dims, cache, pos = r["w"], r["cdims"], r["dims"], r["cache"], r["pos"]
    B, H, d_h = w.B, w.H, w.d_h
    M = synth.weights(w)
    q_nope, q_rope = synth.queries(w, B)
    q_dev = _device_absorb(cdims, w, q_nope, q_rope, pos, M, r["tab_lib"], r["max_pos"])
    seq_len = torch.from_numpy(pos + 1).cuda()
    max_len = int(pos.max()) + 1
    out = torch.full((B, H, d_h), float("nan"), device="cuda")
    lse = torch.full((B, H), float("nan"), device="cuda")
    wsb = gb.gva_decode_workspace_bytes(cdims, B, max_len, 0)
    ws = torch.zeros(max(wsb, 256) // 4, dtype=torch.float32, device="cuda")
    gb.gva_decode(cdims, cache, B, seq_len, max_len, torch.from_numpy(q_dev).cuda(), w.scale,
                  out, lse, workspace=ws)
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(out))

    tab_ora = O.rope_rows(np.arange(r["max_pos"]), w.d_r, w.base)
    for b in r["sampled"]:
        n = int(r["lens"][b]) + 1
        V, krc = _sequence_values(r, b)
        qt, rr = O.absorb(q_nope[b:b + 1], q_rope[b:b + 1], pos[b:b + 1], M, tab_ora)
        q_ref = O.q_abs_of(qt, rr)[0]
        ref, ref_lse = O.decode_sequence(V, krc, dims, q_ref, w.scale)
        check_output(out[b], ref, "bf16", f"ragged batch seq {b} len {n}")
        ok, e = lse_ok(lse[b], ref_lse, 1e-3)
        assert ok, (b, e)


def test_recon_comparator_full_size(ragged):
    """The non-absorbable comparator on the same batch, in the bench's configuration (automatic
    split count, the query at the appended position, a key-wide RoPE table): the longest, the
    shortest and one more sampled sequence against the oracle."""
    r = ragged
    w, cdims, dims, cache, pos = r["w"], r["cdims"], r["dims"], r["cache"], r["pos"]
    B, H, d_h = w.B, w.H, w.d_h
    max_len = int(pos.max()) + 1
    max_pos = max_len + 1
    rope = torch.from_numpy(gb.gva_rope_table_fill(max_pos, w.d_n, w.base)).cuda()
    q, Mv, mt_bits = synth.recon_inputs(w)
    out = torch.full((B, H, d_h), float("nan"), device="cuda")
    lse = torch.full((B, H), float("nan"), device="cuda")
    wsb = gb.gva_recon_decode_workspace_bytes(cdims, B, max_len, 0)
    ws = torch.zeros(max(wsb, 256) // 4, dtype=torch.float32, device="cuda")
    scale = 1.0 / float(np.sqrt(w.d_n))
    gb.gva_recon_decode(cdims, cache, B, torch.from_numpy(pos + 1).cuda(), max_len,
                        torch.from_numpy(q).cuda(), torch.from_numpy(pos).cuda(),
                        torch.from_numpy(mt_bits.view(np.int16)).cuda(), rope, max_pos, scale,
                        out, lse, workspace=ws)
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(out))
    s = r["sampled"]
    for b in sorted({s[0], s[-1], s[len(s) // 2]}):
        V, _ = _sequence_values(r, b)
        ref, ref_lse = O.recon_decode_sequence(V, dims, q[b], int(pos[b]), Mv, scale, w.base)
        check_output(out[b], ref, "bf16", f"comparator ragged batch seq {b} len {V.shape[0]}")
        ok, e = lse_ok(lse[b], ref_lse, 1e-3)
        assert ok, (b, e)


@pytest.fixture(scope="module")
def ragged_latent():
    """The ragged batch's lengths (len_b + 1 tokens, as the bench decodes) in an MLA-style latent
    pool: d_c = 512 described as two token-major groups of 256, a 64-wide positional key, 32
    heads. Sampled sequences carry their seeded tokens, the others device random values."""
    w = synth.workload("C4", G=2, d_h=256, d_n=256, d_r=64)
    lens = synth.lengths(w) + 1
    lay = synth.layout(w, lens, group_major=False)
    B, G, d_h, d_r, H = w.B, w.G, w.d_h, w.d_r, w.H
    cdims = gb.GvaDims(H, G, d_h, w.d_n, d_r)
    max_pos = int(synth.capacity(w, lens).max()) + 1
    tab_lib = torch.from_numpy(gb.gva_rope_table_fill(max_pos, d_r, w.base)).cuda()
    # every element starts as a NaN sentinel that no append of finite data can produce
    cache = gb.GvaCache.allocate(cdims, w.dtype, lay.num_blocks, lay.block_size,
                                 torch.from_numpy(lay.block_table).cuda(), tab_lib,
                                 (lay.v_sb, lay.v_st, lay.v_sg, lay.kr_sb, lay.kr_st),
                                 fill_bits=SENTINEL["bf16"])
    rng = np.random.default_rng(29)
    sampled = sorted({int(np.argmax(lens)), int(np.argmin(lens)),
                      int(rng.choice(B))})
    print(f"latent pool: sampled sequences {sampled}, lengths {[int(lens[b]) for b in sampled]}",
          flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    others = [b for b in range(B) if b not in sampled]
    seqs = np.repeat(np.asarray(others, np.int32), lens[others])
    poss = np.concatenate([np.arange(lens[b], dtype=np.int32) for b in others])
    for o in range(0, seqs.size, 1 << 16):
        n = min(1 << 16, seqs.size - o)
        gb.gva_cache_append(cdims, cache, B, torch.from_numpy(seqs[o:o + n]).cuda(),
                            torch.from_numpy(poss[o:o + n]).cuda(),
                            torch.randn((n, G, d_h), generator=gen, device="cuda"),
                            torch.randn((n, d_r), generator=gen, device="cuda"))
    toks = {}
    for b in sampled:
        n = int(lens[b])
        v, kr = synth.sequence_tokens(w, b, n)
        toks[b] = (v, kr)
        gb.gva_cache_append(cdims, cache, B, torch.full((n,), b, dtype=torch.int32).cuda(),
                            torch.arange(n, dtype=torch.int32).cuda(),
                            torch.from_numpy(v).cuda(), torch.from_numpy(kr).cuda())
    torch.cuda.synchronize()
    return dict(w=w, lens=lens, cdims=cdims, dims=O.Dims(H, G, d_h, w.d_n, d_r), cache=cache,
                sampled=sampled, toks=toks)


def test_mla_comparator_full_size(ragged_latent):
    """The MLA-style latent comparator in the bench's configuration (the ragged batch's lengths,
    d_c = 512, d_r = 64, 32 heads, automatic split count): the longest, the shortest and one more
    sampled sequence against the oracle's absorbed one-group decode."""
    r = ragged_latent
    w, cache, lens, dims = r["w"], r["cache"], r["lens"], r["dims"]
    B, H, d_c, d_r = w.B, w.H, w.G * w.d_h, w.d_r
    mdims = gb.GvaDims(H, 1, d_c, d_c, d_r)
    odims = O.Dims(H, 1, d_c, d_c, d_r)
    q = synth.mla_queries(w, H, d_c, d_r)
    scale = 1.0 / float(np.sqrt(d_c + d_r))
    max_len = int(lens.max())
    out = torch.full((B, H, d_c), float("nan"), device="cuda")
    lse = torch.full((B, H), float("nan"), device="cuda")
    wsb = gb.gva_mla_decode_workspace_bytes(mdims, B, max_len, 0)
    ws = torch.zeros(max(wsb, 256) // 4, dtype=torch.float32, device="cuda")
    gb.gva_mla_decode(mdims, cache, B, torch.from_numpy(lens.astype(np.int32)).cuda(), max_len,
                      torch.from_numpy(q).cuda(), scale, out, lse, workspace=ws)
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(out))
    for b in r["sampled"]:
        n = int(lens[b])
        v, kr = r["toks"][b]
        tab_ora = O.rope_rows(np.arange(n), d_r, w.base)
        pool = O.Pool.empty("bf16", n * w.G * w.d_h, n * d_r,
                            (n * w.G * w.d_h, w.G * w.d_h, w.d_h, n * d_r, d_r),
                            1, 1 << int(np.ceil(np.log2(n))), np.zeros((1, 1)))
        O.append(pool, dims, np.zeros(n, np.int64), np.arange(n), v, kr, tab_ora)
        V, K = O.gather(pool, dims, 0, n)
        ref, ref_lse = O.decode_sequence(V.reshape(n, 1, d_c), K, odims, q[b], scale)
        check_output(out[b], ref, "bf16", f"latent comparator ragged batch seq {b} len {n}")
        ok, e = lse_ok(lse[b], ref_lse, 1e-3)
        assert ok, (b, e)
