"""GPU parity of gva_decode (split decode + combine) against the oracle, for both kernels: the
vector-ALU kernel (any shape, fp32 or bf16 cache) and the matrix-core kernel (bf16 cache)."""
import numpy as np
import pytest
import torch

from oracle import gva_oracle as O
from value_only_kv_amd import binding as gb
from value_only_kv_amd import synth
from tests.gpu_cases import Case, absorbed_queries, check_output, lse_ok, rel_l2

pytestmark = pytest.mark.gpu

GENERIC, MFMA = gb.GVA_KERNEL_GENERIC, gb.GVA_KERNEL_MFMA
KERNELS = [pytest.param(GENERIC, id="generic"), pytest.param(MFMA, id="mfma")]


def _device_absorb(case, q_nope, q_rope, q_pos, M):
    w = case.w
    n = q_nope.shape[0]
    out = torch.empty((n, w.H, w.d_h + w.d_r), device="cuda")
    gb.gva_absorb_query(case.cdims, torch.from_numpy(q_nope).cuda(),
                        torch.from_numpy(q_rope).cuda(),
                        torch.from_numpy(np.asarray(q_pos, np.int32)).cuda(),
                        torch.from_numpy(M).cuda(), case.tab_lib, case.max_pos, out)
    return out.cpu().numpy()


@pytest.fixture(scope="module")
def c1():
    c = Case(synth.workload("C1"))
    c.append_prefix()
    return c


@pytest.fixture(scope="module")
def c2():
    c = Case(synth.workload("C2"))
    c.append_prefix()
    return c


@pytest.mark.parametrize("num_splits", [1, 2, 3, 4])
def test_c1_fp32_end_to_end(c1, num_splits):
    """Absorb on the device, decode on the device; the oracle does both in float64."""
    w = c1.w
    q_pos = [w.T]
    q_ref, (M, q_nope, q_rope) = absorbed_queries(w, 1, q_pos, c1.tab_ora)
    q_dev = _device_absorb(c1, q_nope, q_rope, q_pos, M)
    out, lse = c1.decode([w.T], q_dev, num_splits=num_splits, kernel=GENERIC)
    ref, ref_lse = c1.oracle_decode([w.T], q_ref)
    check_output(out, ref, "f32", f"C1 S={num_splits}")
    ok, e = lse_ok(lse, ref_lse, 1e-5)
    assert ok, e


def test_c1_mfma_refuses_fp32(c1):
    with pytest.raises(gb.GVAError) as ei:
        c1.decode([c1.w.T], np.zeros((1, c1.w.H, c1.w.d_h + c1.w.d_r)), kernel=MFMA)
    assert ei.value.status == gb.GVA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("num_splits", [1, 8, 16, 0])
def test_c2_bf16_end_to_end(c2, kernel, num_splits):
    w = c2.w
    q_pos = [w.T] * w.B
    q_ref, (M, q_nope, q_rope) = absorbed_queries(w, w.B, q_pos, c2.tab_ora)
    q_dev = _device_absorb(c2, q_nope, q_rope, q_pos, M)
    out, lse = c2.decode([w.T] * w.B, q_dev, num_splits=num_splits, kernel=kernel)
    ref, ref_lse = c2.oracle_decode([w.T] * w.B, q_ref)
    check_output(out, ref, "bf16", f"C2 S={num_splits}")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e


def _ragged_case(B=9, lo=0, hi=700, d_r=24, group_major=True, **kw):
    w = synth.workload("C4", B=B, lengths_uniform=(lo, hi), d_r=d_r, **kw)
    c = Case(w, group_major=group_major)
    c.append_prefix()
    return c


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("group_major", [True, False])
@pytest.mark.parametrize("num_splits", [1, 3, 7, 0])
def test_ragged_paged_with_empty_splits(kernel, group_major, num_splits):
    c = _ragged_case(group_major=group_major)
    lens = c.lens.copy()
    lens[0], lens[1], lens[2] = 0, 1, 17     # empty, single-entry and sub-tile sequences
    q = synth.direct_q_abs(c.w, c.w.B)
    out, lse = c.decode(lens, q, num_splits=num_splits, kernel=kernel, max_len=int(c.lens.max()))
    ref, ref_lse = c.oracle_decode(lens, q.astype(np.float64))
    check_output(out, ref, "bf16", f"ragged S={num_splits}")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
    # an empty history gives 0 and -inf; a single entry gives that entry's value
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    V, _ = O.gather(c.pool, c.dims, 1, 1)
    for h in range(c.w.H):
        assert np.allclose(out[1, h], V[0, c.dims.group_of(h)], rtol=0, atol=1e-6)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("d_r,heads", [(8, (8, 8)), (16, (16, 4)), (32, (8, 1)), (24, (32, 2))])
def test_other_shapes(kernel, d_r, heads):
    H, G = heads
    c = _ragged_case(B=3, lo=100, hi=500, d_r=d_r, H=H, G=G)
    q = synth.direct_q_abs(c.w, c.w.B)
    out, lse = c.decode(c.lens, q, num_splits=0, kernel=kernel)
    ref, _ = c.oracle_decode(c.lens, q.astype(np.float64))
    check_output(out, ref, "bf16", f"H={H} G={G} d_r={d_r}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_d_h_64_and_256(kernel):
    for d_h in (64, 256):
        c = _ragged_case(B=2, lo=200, hi=400, d_h=d_h, d_n=d_h, H=8, G=2, d_r=16)
        q = synth.direct_q_abs(c.w, c.w.B)
        out, _ = c.decode(c.lens, q, num_splits=2, kernel=kernel)
        ref, _ = c.oracle_decode(c.lens, q.astype(np.float64))
        check_output(out, ref, "bf16", f"d_h={d_h}")


@pytest.mark.parametrize("d_h,heads", [(96, (6, 3)), (160, (8, 4)), (32, (16, 2)), (256, (4, 2))])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_value_widths_both_load_layouts(d_h, heads, num_splits):
    """The matrix-core kernel loads value rows whole-line (d_h = 32 KS with KS a power of two,
    staged through LDS for the score operand) or in the operand layout (other KS): widths of
    both kinds, token- and group-major, against the oracle."""
    H, G = heads
    for group_major in (True, False):
        c = _ragged_case(B=5, lo=40, hi=900, d_h=d_h, d_n=d_h, H=H, G=G, d_r=16,
                         group_major=group_major)
        lens = c.lens.copy()
        lens[0], lens[1] = 1, 17
        q = synth.direct_q_abs(c.w, c.w.B)
        out, lse = c.decode(lens, q, num_splits=num_splits, kernel=MFMA)
        ref, ref_lse = c.oracle_decode(lens, q.astype(np.float64))
        check_output(out, ref, "bf16", f"d_h={d_h} H={H} G={G} gm={group_major}")
        ok, e = lse_ok(lse, ref_lse, 1e-3)
        assert ok, e


@pytest.mark.parametrize("kernel", KERNELS)
def test_peaky_and_flat_scores(kernel):
    c = _ragged_case(B=4, lo=300, hi=900)
    q = synth.direct_q_abs(c.w, c.w.B) * 8.0      # near one-hot softmax
    out, _ = c.decode(c.lens, q, kernel=kernel)
    ref, _ = c.oracle_decode(c.lens, q.astype(np.float64))
    check_output(out, ref, "bf16", "peaky")
    q0 = np.zeros_like(q)                          # all scores equal: the mean of the values
    out, lse = c.decode(c.lens, q0, kernel=kernel)
    ref, _ = c.oracle_decode(c.lens, q0.astype(np.float64))
    check_output(out, ref, "bf16", "flat")
    assert np.allclose(lse, np.log(c.lens)[:, None], atol=1e-5)


@pytest.mark.parametrize("kernel", KERNELS)
def test_deterministic(kernel):
    c = _ragged_case(B=5, lo=500, hi=3000)
    q = synth.direct_q_abs(c.w, c.w.B)
    a, la = c.decode(c.lens, q, kernel=kernel, num_splits=5)
    b, lb = c.decode(c.lens, q, kernel=kernel, num_splits=5)
    assert a.tobytes() == b.tobytes() and la.tobytes() == lb.tobytes()


@pytest.mark.parametrize("kernel", KERNELS)
def test_bad_block_and_length_poison_rows(kernel):
    c = _ragged_case(B=4, lo=200, hi=400)
    q = synth.direct_q_abs(c.w, c.w.B)
    lens = c.lens.copy()
    # sequence 1: corrupt one of its table entries (a block id beyond the pool)
    saved = c.block_table[1, 2].item()
    c.block_table[1, 2] = c.lay.num_blocks + 5
    # sequence 2: a length above max_len
    max_len = int(lens.max())
    lens[2] = max_len + 1
    try:
        out, lse = c.decode(lens, q, kernel=kernel, max_len=max_len, num_splits=2)
    finally:
        c.block_table[1, 2] = saved
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[2]))
    assert np.all(np.isnan(lse[1])) and np.all(np.isnan(lse[2]))
    assert np.all(np.isfinite(out[0])) and np.all(np.isfinite(out[3]))
    assert c.err_flag() & gb.DEVERR_BLOCK and c.err_flag() & gb.DEVERR_LENGTH
    ref, _ = c.oracle_decode(c.lens, q.astype(np.float64), seqs=[0, 3])
    check_output(out[[0, 3]], ref[[0, 3]], "bf16", "healthy rows")


@pytest.mark.parametrize("kernel", KERNELS)
def test_split_counts_one_to_many(kernel):
    c = _ragged_case(B=2, lo=4000, hi=4100)
    q = synth.direct_q_abs(c.w, c.w.B)
    ref, _ = c.oracle_decode(c.lens, q.astype(np.float64))
    for S in (1, 2, 5, 16, 33, 64, 1024):
        out, _ = c.decode(c.lens, q, num_splits=S, kernel=kernel)
        check_output(out, ref, "bf16", f"S={S}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("num_splits", [17, 40, 64, 200, 256])
@pytest.mark.parametrize("B", [1, 4])
def test_split_combine_ignores_unwritten_rows(kernel, num_splits, B):
    """Partial rows at or past a sequence's chunk count are never written by the decode and here
    hold NaN: the outputs must not see them. Both combines load rows before they know the
    length: the one-sequence combine every row (the sequence is shorter than max_len here, so
    some rows are unused), the batch combine its first rows per wave."""
    c = _ragged_case(B=B, lo=4000, hi=4100)
    lens = np.array([int(c.lens[0]), 900, 33, 0])[:B] if B > 1 else np.array([900])
    q = synth.direct_q_abs(c.w, c.w.B)
    out, lse = c.decode(lens, q, num_splits=num_splits, kernel=kernel, max_len=int(c.lens.max()),
                        ws_fill=float("nan"))
    ref, ref_lse = c.oracle_decode(lens, q.astype(np.float64))
    check_output(out, ref, "bf16", f"B={B} S={num_splits}, NaN in unwritten partial rows")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
    if B > 1:
        assert np.all(out[3] == 0) and np.all(np.isneginf(lse[3]))


def test_combine_many_rows_for_one_sequence():
    """A batch whose plan has few partial rows per sequence on average (so the combine takes one
    wave per (sequence, head)) but one long sequence among short ones, which spans more than 64
    ranges: the combine walks its rows 64 at a time."""
    c = _ragged_case(B=32, lo=4096, hi=4100)
    lens = np.array([4096] + [1 + 3 * i for i in range(31)])
    ml = int(lens.max())
    R = gb.gva_decode_num_ranges(c.cdims, c.w.B, ml)
    assert R // c.w.B + 1 <= 16
    tiles = (lens + 31) // 32
    P = np.concatenate([[0], np.cumsum(tiles)])
    T = int(P[-1])
    Re = min(R, T)
    rows_long = (int(P[1]) * Re - 1) // T - ((int(P[0]) + 1) * Re - 1) // T + 1
    assert rows_long > 64
    q = synth.direct_q_abs(c.w, c.w.B)
    out, lse = c.decode(lens, q, num_splits=0, kernel=MFMA, max_len=ml)
    ref, ref_lse = c.oracle_decode(lens, q.astype(np.float64))
    check_output(out, ref, "bf16", "one long sequence among short ones")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e


def test_balanced_ranges_edge_lengths():
    """The matrix-core kernel's automatic plan cuts the tiles of all sequences into equal ranges:
    empty sequences, single positions and tile-boundary lengths, and a plan with more ranges than
    the sequences have tiles (max_len far above the actual lengths)."""
    c = _ragged_case(B=40, lo=0, hi=2000)
    lens = c.lens.copy()
    lens[:12] = [0, 1, 31, 32, 33, 0, 0, 64, 65, 0, 1, 2]
    ml = int(c.lens.max())
    assert gb.gva_decode_num_ranges(c.cdims, c.w.B, ml) > 1
    q = synth.direct_q_abs(c.w, c.w.B)
    out, lse = c.decode(lens, q, num_splits=0, kernel=MFMA, max_len=ml)
    ref, ref_lse = c.oracle_decode(lens, q.astype(np.float64))
    check_output(out, ref, "bf16", "balanced edge lengths")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))

    # a cache sized for ~4000 positions, decoded over a few positions per sequence
    big = _ragged_case(B=3, lo=4000, hi=4100)
    lens = np.array([1, 5, 40])
    ml = int(big.lens.min())
    q = synth.direct_q_abs(big.w, big.w.B)
    R = gb.gva_decode_num_ranges(big.cdims, big.w.B, ml)
    assert R > int(np.sum((lens + 31) // 32))
    out, lse = big.decode(lens, q, num_splits=0, kernel=MFMA, max_len=ml)
    ref, ref_lse = big.oracle_decode(lens, q.astype(np.float64))
    check_output(out, ref, "bf16", "more ranges than tiles")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
