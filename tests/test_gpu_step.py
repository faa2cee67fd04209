"""GPU parity of gva_decode_step against the three separate calls and the oracle. Small batches
run the whole step as one launch (one work-group per sequence and group); the others run the
append and the absorption as one launch, then the decode. Either way the cache bytes and the
absorbed queries are bit-identical to the three calls; the outputs are bit-identical on the
multi-launch path and within rounding of them on the one-launch path (it splits the positions
differently), and within the bf16/fp32 bars of the oracle's float64 append, absorption and
decode."""
import numpy as np
import pytest
import torch

from oracle import gva_oracle as O
from value_only_kv_amd import binding as gb
from value_only_kv_amd import synth
from tests.gpu_cases import Case, absorbed_queries, check_output, lse_ok

pytestmark = pytest.mark.gpu


def _case(name, **kw):
    w = synth.workload(name, **kw)
    c = Case(w)
    c.append_prefix()
    return c


def _step_inputs(c, seed):
    """New tokens (one per sequence, at position lens[b]) and their queries."""
    w = c.w
    rng = np.random.default_rng(np.random.SeedSequence([4242, seed]))
    v_new = rng.standard_normal((w.B, w.G, w.d_h)).astype(np.float32)
    kr_raw = rng.standard_normal((w.B, w.d_r)).astype(np.float32)
    pos = c.lens.astype(np.int64)
    q_ref, (M, q_nope, q_rope) = absorbed_queries(w, w.B, pos, c.tab_ora)
    return pos, v_new, kr_raw, M, q_nope, q_rope, q_ref


def _t(x, dtype=None):
    a = np.ascontiguousarray(x if dtype is None else np.asarray(x, dtype))
    return torch.from_numpy(a).cuda()


def _run_step(c, pos, v_new, kr_raw, M, q_nope, q_rope, num_splits, fused, kernel=gb.GVA_KERNEL_AUTO):
    w = c.w
    B, H = w.B, w.H
    sl = pos + 1
    ml = int(sl.max())
    pos_t, sl_t = _t(pos, np.int32), _t(sl, np.int32)
    qa = torch.full((B, H, w.d_h + w.d_r), float("nan"), device="cuda")
    out = torch.full((B, H, w.d_h), float("nan"), device="cuda")
    lse = torch.full((B, H), float("nan"), device="cuda")
    wsb = gb.gva_decode_workspace_bytes(c.cdims, B, ml, num_splits)
    ws = torch.zeros(max(wsb, 256) // 4, device="cuda") if wsb else None
    args = tuple(_t(x, np.float32) for x in (v_new, kr_raw, q_nope, q_rope, M))
    if fused:
        gb.gva_decode_step(c.cdims, c.cache, B, pos_t, *args[:2], *args[2:], sl_t, ml, w.scale, qa,
                           out, lse, num_splits=num_splits, kernel=kernel, workspace=ws)
    else:
        seq = _t(np.arange(B), np.int32)
        gb.gva_cache_append(c.cdims, c.cache, B, seq, pos_t, args[0], args[1])
        gb.gva_absorb_query(c.cdims, args[2], args[3], pos_t, args[4], c.tab_lib, c.max_pos, qa,
                            err_flag=c.cache.err_flag)
        gb.gva_decode(c.cdims, c.cache, B, sl_t, ml, qa, w.scale, out, lse,
                      num_splits=num_splits, kernel=kernel, workspace=ws)
    torch.cuda.synchronize()
    return qa.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()


# (name, workload overrides, num_splits, launches the step takes)
SHAPES = [
    pytest.param("C1", dict(append_one=True, block_size=512), 1, 2, id="C1-fp32"),
    pytest.param("C4", dict(B=3, lengths_uniform=(200, 400), d_h=256, d_n=256, H=8, G=2, d_r=16),
                 0, 3, id="d_h-256"),
    pytest.param("C4", dict(B=5, lengths_uniform=(100, 900), H=32, G=4), 0, 3,
                 id="eight-heads-per-group"),
    pytest.param("C4", dict(B=5, lengths_uniform=(100, 900), H=32, G=4, d_h=64, d_n=64), 0, 1,
                 id="eight-heads-per-group-d_h-64"),
    pytest.param("C4", dict(B=40, lengths_uniform=(0, 300)), 0, 3, id="forty-sequences"),
    pytest.param("C2", dict(append_one=True, block_size=8192), 0, 1, id="C2-bf16-auto"),
    pytest.param("C2", dict(append_one=True, block_size=8192), 3, 3, id="C2-bf16-S3"),
    pytest.param("C4", dict(B=9, lengths_uniform=(0, 700)), 0, 3, id="ragged-paged-balanced"),
    pytest.param("C4", dict(B=9, lengths_uniform=(0, 700), d_h=64, d_n=64), 0, 1,
                 id="ragged-paged-one-launch"),
    pytest.param("C4", dict(B=9, lengths_uniform=(0, 700)), 2, 3, id="ragged-paged-S2"),
    pytest.param("C4", dict(B=6, lengths_uniform=(0, 2000), H=16, G=8, d_h=32, d_n=32, d_r=16), 0, 1,
                 id="d_h-32-two-heads-per-group"),
    pytest.param("C4", dict(B=2, lengths_uniform=(9000, 12000), H=8, G=8, d_h=64, d_n=64, d_r=8),
                 0, 1, id="one-head-per-group-long"),
    # the vector-ALU path in one launch: float32 caches and shapes the matrix cores do not take
    pytest.param("C1", dict(append_one=True, block_size=512), 0, 1, id="C1-fp32-auto"),
    pytest.param("C4", dict(B=4, lengths_uniform=(0, 600), H=8, G=4, d_h=64, d_n=64, d_r=12), 0, 1,
                 id="valu-d_r-12-one-launch"),
    pytest.param("C4", dict(B=3, lengths_uniform=(100, 1000), H=4, G=4, d_h=128, d_n=128,
                            dtype="f32"), 0, 1, id="valu-fp32-d_h-128-one-launch"),
    pytest.param("C4", dict(B=5, lengths_uniform=(0, 900), H=16, G=2, d_h=32, d_n=32, d_r=8,
                            dtype="f32"), 0, 1, id="valu-fp32-eight-heads-per-group"),
    pytest.param("C4", dict(B=2, lengths_uniform=(1500, 2000), H=8, G=4, d_h=64, d_n=64,
                            dtype="f32"), 0, 3, id="valu-fp32-long-three-launches"),
]


@pytest.mark.parametrize("name,kw,num_splits,launches", SHAPES)
def test_step_matches_separate_calls(name, kw, num_splits, launches):
    """Same cache bytes and absorbed queries, bit for bit; the same outputs, bit for bit on the
    multi-launch path and to rounding on the one-launch path."""
    a, b = _case(name, **kw), _case(name, **kw)
    pos, v_new, kr_raw, M, q_nope, q_rope, _ = _step_inputs(a, 1)
    assert gb.gva_decode_step_launches(a.cdims, a.cache, a.w.B, int(pos.max()) + 1,
                                       num_splits) == launches
    qa1, o1, l1 = _run_step(a, pos, v_new, kr_raw, M, q_nope, q_rope, num_splits, fused=False)
    qa2, o2, l2 = _run_step(b, pos, v_new, kr_raw, M, q_nope, q_rope, num_splits, fused=True)
    va, ka = a.device_bits()
    vb, kb = b.device_bits()
    assert np.array_equal(va, vb) and np.array_equal(ka, kb)
    assert qa1.tobytes() == qa2.tobytes()
    if launches > 1:
        assert o1.tobytes() == o2.tobytes() and l1.tobytes() == l2.tobytes()
    else:
        assert np.max(np.abs(o1 - o2)) <= 5e-5 and np.max(np.abs(l1 - l2)) <= 5e-5
    assert a.err_flag() == 0 and b.err_flag() == 0


@pytest.mark.parametrize("name,kw,num_splits,launches", SHAPES)
def test_step_against_oracle(name, kw, num_splits, launches):
    c = _case(name, **kw)
    pos, v_new, kr_raw, M, q_nope, q_rope, q_ref = _step_inputs(c, 2)
    qa, out, lse = _run_step(c, pos, v_new, kr_raw, M, q_nope, q_rope, num_splits, fused=True)
    # the oracle appends the same tokens into its own pool; the cache bytes must agree exactly
    O.append(c.pool, c.dims, np.arange(c.w.B), pos, v_new, kr_raw, c.tab_ora)
    v_dev, k_dev = c.device_bits()
    assert np.array_equal(v_dev, c.pool.v) and np.array_equal(k_dev, c.pool.kr)
    # the absorbed queries: float32 accumulation against float64
    assert np.max(np.abs(qa - q_ref)) <= 1e-4 * max(1.0, float(np.max(np.abs(q_ref))))
    ref, ref_lse = c.oracle_decode(pos + 1, q_ref)
    dtype = "f32" if c.w.dtype == "f32" else "bf16"
    check_output(out, ref, dtype, f"step {name} S={num_splits}")
    ok, e = lse_ok(lse, ref_lse, 1e-5 if dtype == "f32" else 1e-3)
    assert ok, e


def test_step_flags_a_position_outside_the_rope_table():
    """A new token beyond the RoPE table: its append is skipped, its query row is NaN, the
    other sequences are unaffected and the ROPE bit is raised."""
    c = _case("C4", B=4, lengths_uniform=(100, 300))
    pos, v_new, kr_raw, M, q_nope, q_rope, q_ref = _step_inputs(c, 3)
    bad = pos.copy()
    bad[2] = c.max_pos + 3
    w = c.w
    B, H = w.B, w.H
    sl = pos + 1
    ml = int(sl.max())
    qa = torch.full((B, H, w.d_h + w.d_r), 0.0, device="cuda")
    out = torch.empty((B, H, w.d_h), device="cuda")
    wsb = gb.gva_decode_workspace_bytes(c.cdims, B, ml, 0)
    ws = torch.zeros(max(wsb, 256) // 4, device="cuda")
    gb.gva_decode_step(c.cdims, c.cache, B, _t(bad, np.int32),
                       *(_t(x, np.float32) for x in (v_new, kr_raw, q_nope, q_rope, M)),
                       _t(sl, np.int32), ml, w.scale, qa, out, workspace=ws)
    torch.cuda.synchronize()
    assert c.err_flag() & gb.DEVERR_ROPE
    qa = qa.cpu().numpy()
    out = out.cpu().numpy()
    assert np.all(np.isnan(qa[2])) and np.all(np.isnan(out[2]))
    good = [0, 1, 3]
    O.append(c.pool, c.dims, np.array(good), pos[good], v_new[good], kr_raw[good], c.tab_ora)
    ref, _ = c.oracle_decode(sl, q_ref, seqs=good)
    check_output(out[good], ref[good], "bf16", "healthy sequences")


def test_step_with_empty_histories():
    """Sequences whose new token is their first (pos = 0): the step appends it and the decode
    reads that one position, so the output is the token's own values."""
    w = synth.workload("C4", B=12, lengths_uniform=(0, 300))
    lens = synth.lengths(w).copy()
    lens[[0, 3, 7]] = 0
    c = Case(w, lens=lens)
    c.append_prefix()
    pos, v_new, kr_raw, M, q_nope, q_rope, q_ref = _step_inputs(c, 4)
    qa, out, lse = _run_step(c, pos, v_new, kr_raw, M, q_nope, q_rope, 0, fused=True)
    O.append(c.pool, c.dims, np.arange(w.B), pos, v_new, kr_raw, c.tab_ora)
    ref, ref_lse = c.oracle_decode(pos + 1, q_ref)
    check_output(out, ref, "bf16", "empty histories")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
    V, _ = O.gather(c.pool, c.dims, 3, 1)
    for h in range(w.H):
        assert np.allclose(out[3, h], V[0, c.dims.group_of(h)], rtol=0, atol=1e-6)


# the two one-launch kernels: matrix cores (bf16, d_h <= 64) and vector ALU (here d_r = 12, which
# the matrix-core kernel does not take, and a float32 cache)
ONE_LAUNCH = [pytest.param({}, "bf16", id="mfma"),
              pytest.param(dict(d_r=12), "bf16", id="valu-bf16"),
              pytest.param(dict(dtype="f32"), "f32", id="valu-fp32")]


def _one_launch_case(B=6, lo=100, hi=900, **kw):
    kw = dict(dict(d_h=64, d_n=64), **kw)
    c = _case("C4", B=B, lengths_uniform=(lo, hi), **kw)
    assert gb.gva_decode_step_launches(c.cdims, c.cache, B, int(c.lens.max()) + 1, 0) == 1
    return c


@pytest.mark.parametrize("kw,dtype", ONE_LAUNCH)
def test_one_launch_step_not_reading_its_token(kw, dtype):
    """seq_len = pos: the token is appended (bit-exact) but the decode reads only the history."""
    c = _one_launch_case(**kw)
    w = c.w
    pos, v_new, kr_raw, M, q_nope, q_rope, q_ref = _step_inputs(c, 6)
    sl = pos.copy()
    qa = torch.full((w.B, w.H, w.d_h + w.d_r), float("nan"), device="cuda")
    out = torch.full((w.B, w.H, w.d_h), float("nan"), device="cuda")
    lse = torch.full((w.B, w.H), float("nan"), device="cuda")
    ml = int(pos.max()) + 1
    ws = torch.zeros(max(gb.gva_decode_workspace_bytes(c.cdims, w.B, ml, 0), 256) // 4, device="cuda")
    gb.gva_decode_step(c.cdims, c.cache, w.B, _t(pos, np.int32),
                       *(_t(x, np.float32) for x in (v_new, kr_raw, q_nope, q_rope, M)),
                       _t(sl, np.int32), ml, w.scale, qa, out, lse, workspace=ws)
    torch.cuda.synchronize()
    O.append(c.pool, c.dims, np.arange(w.B), pos, v_new, kr_raw, c.tab_ora)
    v_dev, k_dev = c.device_bits()
    assert np.array_equal(v_dev, c.pool.v) and np.array_equal(k_dev, c.pool.kr)
    ref, ref_lse = c.oracle_decode(sl, q_ref)
    check_output(out.cpu().numpy(), ref, dtype, f"one-launch step, token not read, {kw}")
    ok, e = lse_ok(lse.cpu().numpy(), ref_lse, 1e-5 if dtype == "f32" else 1e-3)
    assert ok, e
    assert c.err_flag() == 0


@pytest.mark.parametrize("kw,dtype", ONE_LAUNCH)
def test_one_launch_step_device_errors(kw, dtype):
    """A bad block-table entry in sequence 1's history and a length above max_len for sequence
    4: their rows are NaN and the BLOCK and LENGTH bits are raised; the token of sequence 4 is
    still appended; the other sequences match the oracle. Every work-group exits normally."""
    c = _one_launch_case(**kw)
    w = c.w
    pos, v_new, kr_raw, M, q_nope, q_rope, q_ref = _step_inputs(c, 7)
    c.block_table[1, 2] = c.lay.num_blocks + 11          # positions 32 .. 47 of sequence 1
    sl = pos + 1
    ml = int(sl.max())
    bad_sl = sl.copy()
    bad_sl[4] = ml + 5
    qa = torch.full((w.B, w.H, w.d_h + w.d_r), float("nan"), device="cuda")
    out = torch.full((w.B, w.H, w.d_h), float("nan"), device="cuda")
    lse = torch.full((w.B, w.H), float("nan"), device="cuda")
    ws = torch.zeros(max(gb.gva_decode_workspace_bytes(c.cdims, w.B, ml, 0), 256) // 4, device="cuda")
    gb.gva_decode_step(c.cdims, c.cache, w.B, _t(pos, np.int32),
                       *(_t(x, np.float32) for x in (v_new, kr_raw, q_nope, q_rope, M)),
                       _t(bad_sl, np.int32), ml, w.scale, qa, out, lse, workspace=ws)
    torch.cuda.synchronize()
    f = c.err_flag()
    assert f & gb.DEVERR_BLOCK and f & gb.DEVERR_LENGTH
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isnan(out[[1, 4]])) and np.all(np.isnan(lse[[1, 4]]))
    good = [0, 2, 3, 5]
    O.append(c.pool, c.dims, np.arange(w.B), pos, v_new, kr_raw, c.tab_ora)
    v_dev, k_dev = c.device_bits()
    assert np.array_equal(v_dev, c.pool.v) and np.array_equal(k_dev, c.pool.kr)
    ref, ref_lse = c.oracle_decode(sl, q_ref, seqs=good)
    check_output(out[good], ref[good], dtype, f"one-launch step beside device errors, {kw}")
