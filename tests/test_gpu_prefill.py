"""GPU parity of gva_prefill_chunk (chunk append + causal attention on matrix cores) against the
oracle: the appended chunk is bit-exact in the pool, and outputs are within the bf16 tolerance."""
import numpy as np
import pytest
import torch

from oracle import gva_oracle as O
from value_only_kv_amd import binding as gb
from value_only_kv_amd import synth
from tests.gpu_cases import ERRORS, Case, check_output, lse_ok

pytestmark = pytest.mark.gpu

# The lse of a row depends on its scores only, and moves by at most max_j |error of s_j| (the
# log-sum-exp is 1-Lipschitz in the largest score error). The scores use the absorbed query as a
# bf16 hi + lo pair (relative error 2^-16 per element) against exact bf16 keys with float32
# accumulation, so |error of s_j| <= scale sum_i |q_i| |k_i| (2^-16 + (d_h + d_r) 2^-24): about
# 2e-4 for unit-normal queries and keys at these widths. The probabilities' bf16 rounding enters
# only the weighted sum, not the sum of exponentials. The bar is that of the decode, 1e-3.
LSE_TOL = 1e-3


def _lse_check(got, ref, what):
    ok, e = lse_ok(got, ref, LSE_TOL)
    ERRORS.append((what + " lse", "bf16", e, 0.0))
    assert ok, (what, e)


def _run_prefill(c, start, C, q_abs, v_new, kr_new):
    w = c.w
    B = w.B
    st = torch.from_numpy(np.asarray(start, np.int32)).cuda()
    out = torch.full((B, C, w.H, w.d_h), float("nan"), device="cuda")
    lse = torch.full((B, C, w.H), float("nan"), device="cuda")
    gb.gva_prefill_chunk(c.cdims, c.cache, B, st, int(max(start)), C,
                         torch.from_numpy(np.ascontiguousarray(q_abs, np.float32)).cuda(),
                         torch.from_numpy(np.ascontiguousarray(v_new, np.float32)).cuda(),
                         torch.from_numpy(np.ascontiguousarray(kr_new, np.float32)).cuda(),
                         w.scale, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _chunk_inputs(w, starts, C):
    v_new = np.zeros((w.B, C, w.G, w.d_h), np.float32)
    kr_new = np.zeros((w.B, C, w.d_r), np.float32)
    for b in range(w.B):
        v, kr = synth.sequence_tokens(w, b, int(starts[b]) + C)
        v_new[b], kr_new[b] = v[starts[b]:], kr[starts[b]:]
    rng = np.random.default_rng(5)
    q_abs = rng.standard_normal((w.B, C, w.H, w.d_h + w.d_r)).astype(np.float32)
    return q_abs, v_new, kr_new


@pytest.mark.parametrize("shape", [
    dict(H=8, G=2, d_h=64, d_n=64, d_r=16),        # 4 heads per group
    dict(H=32, G=8, d_h=128, d_n=128, d_r=24),     # the long-context shape
    dict(H=6, G=3, d_h=96, d_n=96, d_r=8),         # 2 heads per group, d_h = 3 x 32
    dict(H=4, G=2, d_h=256, d_n=256, d_r=32),      # one row tile per wave
])
@pytest.mark.parametrize("starts,C", [((100, 37, 0), 70), ((0, 5, 300), 1), ((64, 0, 16), 257)])
def test_prefill_small_against_oracle(shape, starts, C):
    w = synth.workload("C5", B=len(starts), T=0, chunk=C, append_one=False,
                       lengths_uniform=None, **shape)
    lens = np.asarray(starts, np.int64)
    c = Case(w, lens=lens)
    c.append_prefix()                                   # positions 0 .. start_b - 1
    q_abs, v_new, kr_new = _chunk_inputs(w, starts, C)
    out, lse = _run_prefill(c, starts, C, q_abs, v_new, kr_new)
    ref, ref_lse, err = O.prefill(c.pool, c.dims, starts, C, q_abs.astype(np.float64), v_new,
                                  kr_new, w.scale, c.tab_ora)
    assert err == 0 and c.err_flag() == 0
    # the chunk append wrote exactly what the oracle wrote (whole pools, sentinels included)
    v_bits, kr_bits = c.device_bits()
    assert np.array_equal(v_bits, c.pool.v) and np.array_equal(kr_bits, c.pool.kr)
    check_output(out, ref, "bf16", f"prefill {shape} starts={starts} C={C}")
    _lse_check(lse, ref_lse, f"prefill {shape} starts={starts} C={C}")


def test_prefill_end_to_end_through_absorb():
    """Queries absorbed on the device at positions start_b + i; the oracle absorbs its own."""
    w = synth.workload("C5", B=2, T=0, chunk=96, append_one=False, H=16, G=4, d_h=64, d_n=64)
    starts = np.array([200, 77])
    c = Case(w, lens=starts)
    c.append_prefix()
    C = w.chunk
    _, v_new, kr_new = _chunk_inputs(w, starts, C)
    M = synth.weights(w)
    q_nope, q_rope = synth.queries(w, w.B * C)
    q_pos = (starts[:, None] + np.arange(C)[None, :]).reshape(-1).astype(np.int32)
    q_dev = torch.empty((w.B * C, w.H, w.d_h + w.d_r), device="cuda")
    gb.gva_absorb_query(c.cdims, torch.from_numpy(q_nope).cuda(), torch.from_numpy(q_rope).cuda(),
                        torch.from_numpy(q_pos).cuda(), torch.from_numpy(M).cuda(), c.tab_lib,
                        c.max_pos, q_dev)
    qt, r = O.absorb(q_nope, q_rope, q_pos, M, c.tab_ora)
    q_ref = O.q_abs_of(qt, r).reshape(w.B, C, w.H, -1)
    out, _ = _run_prefill(c, starts, C, q_dev.cpu().numpy().reshape(w.B, C, w.H, -1), v_new, kr_new)
    ref, _, _ = O.prefill(c.pool, c.dims, starts, C, q_ref, v_new, kr_new, w.scale, c.tab_ora)
    check_output(out, ref, "bf16", "prefill end to end")


def test_prefill_c5_full_size_sampled_rows():
    """B=4 sequences, 8192 cached positions + a 512-token causal chunk, H=32, G=8, d_h=128,
    d_r=16, 16-token blocks; the oracle checks sampled (sequence, query, head) rows."""
    w = synth.workload("C5", append_one=False)
    lens = synth.lengths(w)
    c = Case(w, lens=lens)
    c.append_prefix(oracle=False)
    C = w.chunk
    starts = lens.astype(np.int64)
    q_abs, v_new, kr_new = _chunk_inputs(w, starts, C)
    out, lse = _run_prefill(c, starts, C, q_abs, v_new, kr_new)
    assert c.err_flag() == 0
    rng = np.random.default_rng(11)
    for b in range(w.B):
        n = int(starts[b]) + C
        # the oracle's pool for this sequence only: its own append of all n positions
        v, kr = synth.sequence_tokens(w, b, n)
        O.append(c.pool, c.dims, np.full(n, b), np.arange(n), v, kr, c.tab_ora)
        V, krc = O.gather(c.pool, c.dims, b, n)
        queries = sorted(set([0, 1, C - 1] + list(rng.integers(0, C, size=13))))
        got, ref = [], []
        for i in queries:
            L = int(starts[b]) + i + 1
            o, l = O.decode_sequence(V[:L], krc[:L], c.dims, q_abs[b, i].astype(np.float64), w.scale)
            got.append(out[b, i])
            ref.append(o)
            _lse_check(lse[b, i], l, f"C5 seq {b} query {i}")
        check_output(np.array(got), np.array(ref), "bf16", f"C5 seq {b}")
    v_bits, kr_bits = c.device_bits()
    assert np.array_equal(v_bits, c.pool.v) and np.array_equal(kr_bits, c.pool.kr)


def test_prefill_bad_start_poisons_rows():
    w = synth.workload("C5", B=2, T=0, chunk=40, append_one=False, H=8, G=2, d_h=64, d_n=64)
    starts = np.array([50, 20])
    c = Case(w, lens=starts)
    c.append_prefix()
    q_abs, v_new, kr_new = _chunk_inputs(w, starts, 40)
    bad = np.array([50, -3])
    out, lse = _run_prefill(c, bad, 40, q_abs, v_new, kr_new)
    assert np.all(np.isfinite(out[0])) and np.all(np.isnan(out[1]))
    assert c.err_flag() & gb.DEVERR_LENGTH


def _oracle_rows(c, b, start, C, q_abs, upto):
    """Oracle outputs of sequence b's queries i with start + i < upto (their windows end before
    position upto), from the oracle's pool: out [n, H, d_h], lse [n, H]."""
    w = c.w
    n = max(0, min(C, upto - start))
    V, kr = O.gather(c.pool, c.dims, b, start + n)
    out = np.zeros((n, w.H, w.d_h))
    lse = np.zeros((n, w.H))
    for i in range(n):
        L = start + i + 1
        out[i], lse[i] = O.decode_sequence(V[:L], kr[:L], c.dims, q_abs[b, i].astype(np.float64),
                                           w.scale)
    return out, lse


def _error_case(starts, C=40, max_pos=None):
    w = synth.workload("C5", B=len(starts), T=0, chunk=C, append_one=False, lengths_uniform=None,
                       H=8, G=2, d_h=64, d_n=64, d_r=16)
    starts = np.asarray(starts, np.int64)
    c = Case(w, lens=starts, max_pos=max_pos)
    c.append_prefix()
    return c, starts


def test_prefill_corrupt_prefix_block_poisons_the_sequence():
    """A block-table entry outside the pool in the cached prefix of sequence 0: every query of
    that sequence sees it, so all its rows are NaN and the BLOCK bit is raised; sequence 1 is
    untouched and matches the oracle. The kernel reads block 0 in its place and exits normally."""
    c, starts = _error_case([100, 64])
    C = c.w.chunk
    q_abs, v_new, kr_new = _chunk_inputs(c.w, starts, C)
    c.block_table[0, 3] = c.lay.num_blocks + 7          # positions 48 .. 63 of sequence 0
    out, lse = _run_prefill(c, starts, C, q_abs, v_new, kr_new)
    assert c.err_flag() & gb.DEVERR_BLOCK
    assert np.all(np.isnan(out[0])) and np.all(np.isnan(lse[0]))
    # the chunk itself was appended (its blocks are valid): the pools agree bit for bit
    O.append(c.pool, c.dims, np.repeat(np.arange(2), C),
             (starts[:, None] + np.arange(C)[None, :]).reshape(-1),
             v_new.reshape(-1, c.w.G, c.w.d_h), kr_new.reshape(-1, c.w.d_r), c.tab_ora)
    v_bits, kr_bits = c.device_bits()
    assert np.array_equal(v_bits, c.pool.v) and np.array_equal(kr_bits, c.pool.kr)
    ref, ref_lse = _oracle_rows(c, 1, int(starts[1]), C, q_abs, 1 << 30)
    check_output(out[1], ref, "bf16", "prefill, other sequence beside a corrupt block")
    _lse_check(lse[1], ref_lse, "prefill beside a corrupt block")


def test_prefill_corrupt_block_inside_the_chunk_poisons_later_rows_only():
    """The entry of the block holding chunk positions 112 .. 127 of sequence 0 is corrupt: the
    chunk append skips those tokens (BLOCK), queries at positions below 112 never see them and
    match the oracle, and every query at 112 or later is NaN."""
    c, starts = _error_case([100, 64])
    C = c.w.chunk
    q_abs, v_new, kr_new = _chunk_inputs(c.w, starts, C)
    bad = c.lay.num_blocks + 3
    c.block_table[0, 7] = bad
    c.pool.block_table[0, 7] = bad                      # the oracle's append skips them too
    out, lse = _run_prefill(c, starts, C, q_abs, v_new, kr_new)
    assert c.err_flag() & gb.DEVERR_BLOCK
    err = O.append(c.pool, c.dims, np.repeat(np.arange(2), C),
                   (starts[:, None] + np.arange(C)[None, :]).reshape(-1),
                   v_new.reshape(-1, c.w.G, c.w.d_h), kr_new.reshape(-1, c.w.d_r), c.tab_ora)
    assert err & O.ERR_BLOCK
    v_bits, kr_bits = c.device_bits()
    assert np.array_equal(v_bits, c.pool.v) and np.array_equal(kr_bits, c.pool.kr)
    n_ok = 112 - int(starts[0])
    assert np.all(np.isnan(out[0, n_ok:])) and np.all(np.isnan(lse[0, n_ok:]))
    ref, ref_lse = _oracle_rows(c, 0, int(starts[0]), C, q_abs, 112)
    check_output(out[0, :n_ok], ref, "bf16", "prefill rows before a corrupt chunk block")
    _lse_check(lse[0, :n_ok], ref_lse, "prefill before a corrupt chunk block")
    assert np.all(np.isfinite(out[1]))


def test_prefill_chunk_past_the_rope_table():
    """The RoPE table has 120 rows: sequence 0's chunk (positions 100 .. 139) does not fit, so its
    tokens from 120 on are not appended, the ROPE bit is raised and all its rows are NaN;
    sequence 1 (positions 20 .. 59) is unaffected."""
    c, starts = _error_case([100, 20], max_pos=120)
    C = c.w.chunk
    q_abs, v_new, kr_new = _chunk_inputs(c.w, starts, C)
    out, lse = _run_prefill(c, starts, C, q_abs, v_new, kr_new)
    assert c.err_flag() & gb.DEVERR_ROPE
    assert np.all(np.isnan(out[0])) and np.all(np.isnan(lse[0]))
    err = O.append(c.pool, c.dims, np.repeat(np.arange(2), C),
                   (starts[:, None] + np.arange(C)[None, :]).reshape(-1),
                   v_new.reshape(-1, c.w.G, c.w.d_h), kr_new.reshape(-1, c.w.d_r), c.tab_ora)
    assert err & O.ERR_ROPE
    v_bits, kr_bits = c.device_bits()
    assert np.array_equal(v_bits, c.pool.v) and np.array_equal(kr_bits, c.pool.kr)
    ref, ref_lse = _oracle_rows(c, 1, int(starts[1]), C, q_abs, 1 << 30)
    check_output(out[1], ref, "bf16", "prefill, other sequence beside a short RoPE table")
