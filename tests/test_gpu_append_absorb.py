"""GPU parity of gva_cache_append (bit-exact, whole sentinel-filled pools) and gva_absorb_query
(the rotated slice bit-exact; q~ within the float32 summation bound) against the oracle."""
import numpy as np
import pytest
import torch

from oracle import gva_oracle as O
from value_only_kv_amd import binding as gb
from value_only_kv_amd import synth
from tests.gpu_cases import Case, SENTINEL

pytestmark = pytest.mark.gpu


def _assert_pools_equal(case):
    v, kr = case.device_bits()
    assert v.shape == case.pool.v.shape and kr.shape == case.pool.kr.shape
    bad_v = np.nonzero(v != case.pool.v)[0]
    bad_k = np.nonzero(kr != case.pool.kr)[0]
    assert bad_v.size == 0, f"{bad_v.size} V elements differ, first at {bad_v[:5]}"
    assert bad_k.size == 0, f"{bad_k.size} kr elements differ, first at {bad_k[:5]}"


def test_append_c1_fp32_contiguous_bit_exact():
    c = Case(synth.workload("C1"))
    c.append_prefix()
    _assert_pools_equal(c)
    assert c.err_flag() == 0
    # the untouched tail of the contiguous block still holds the sentinel
    v, _ = c.device_bits()
    assert np.count_nonzero(v == SENTINEL["f32"]) == (c.lay.block_size - c.w.T) * c.w.G * c.w.d_h


@pytest.mark.parametrize("group_major", [True, False])
def test_append_paged_ragged_bit_exact(group_major):
    w = synth.workload("C4", B=12, lengths_uniform=(1, 300))
    c = Case(w, group_major=group_major)
    c.append_prefix()
    _assert_pools_equal(c)
    assert c.err_flag() == 0


def test_append_interleaved_token_order_bit_exact():
    """Tokens of several sequences in one call, in a shuffled order."""
    w = synth.workload("C4", B=6, lengths_uniform=(20, 90), d_r=16)
    c = Case(w)
    seq, pos, vs, ks = [], [], [], []
    for b in range(w.B):
        n = int(c.lens[b])
        v, kr = synth.sequence_tokens(w, b, n)
        seq += [b] * n
        pos += list(range(n))
        vs.append(v)
        ks.append(kr)
    seq, pos = np.array(seq), np.array(pos)
    v, kr = np.concatenate(vs), np.concatenate(ks)
    perm = np.random.default_rng(0).permutation(seq.size)
    c.append_tokens(seq[perm], pos[perm], v[perm], kr[perm])
    _assert_pools_equal(c)


def test_append_c2_full_size_bit_exact():
    c = Case(synth.workload("C2"))
    c.append_prefix()
    _assert_pools_equal(c)


def test_append_extreme_values_bit_exact():
    """Values that exercise rounding corners: ties, bf16 subnormals, overflow, signed zeros."""
    w = synth.workload("C4", B=2, lengths_uniform=(64, 64))
    c = Case(w)
    rng = np.random.default_rng(5)
    n = 64
    v = rng.standard_normal((n, w.G, w.d_h)).astype(np.float32)
    flat = v.reshape(-1)
    specials = np.array([0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1e-39, -3e-40, 3.4e38,
                         -3.39e38, 1.5e-45, 2.0 ** -126, 65504.0, 1.0 / 3.0], dtype=np.float32)
    flat[: specials.size * 50] = np.tile(specials, 50)
    kr = (rng.standard_normal((n, w.d_r)) * np.logspace(-40, 37, n)[:, None]).astype(np.float32)
    kr[0, :4] = [0.0, -0.0, 1e-39, 3e38]
    c.append_tokens(np.zeros(n), np.arange(n), v, kr)
    _assert_pools_equal(c)


def test_append_device_errors_skip_the_token():
    w = synth.workload("C4", B=3, lengths_uniform=(10, 40))
    c = Case(w, max_pos=64)
    one_v = np.ones((1, w.G, w.d_h), np.float32)
    one_k = np.ones((1, w.d_r), np.float32)
    cap = c.lay.max_blocks * c.lay.block_size
    for seq, pos, bit in [(w.B, 0, gb.DEVERR_SEQ), (0, -1, gb.DEVERR_LENGTH),
                          (0, cap, gb.DEVERR_CAPACITY)]:
        c.cache.err_flag.zero_()
        c.append_tokens([seq], [pos], one_v, one_k, oracle=False)
        assert c.err_flag() == bit
    # a table slot that names no block (-1)
    b = int(np.argmin((c.lay.block_table >= 0).sum(axis=1)))
    p = int((c.lay.block_table[b] >= 0).sum()) * c.lay.block_size
    if p < cap and p < c.max_pos:
        c.cache.err_flag.zero_()
        c.append_tokens([b], [p], one_v, one_k, oracle=False)
        assert c.err_flag() == gb.DEVERR_BLOCK
    # beyond the RoPE table
    c2 = Case(w, max_pos=8)
    b0 = int(np.argmax((c2.lay.block_table >= 0).sum(axis=1)))
    c2.append_tokens([b0], [9], one_v, one_k, oracle=False)
    assert c2.err_flag() == gb.DEVERR_ROPE
    # nothing was written anywhere
    _assert_pools_equal(c)
    _assert_pools_equal(c2)


@pytest.mark.parametrize("name,n_q", [("C1", 5), ("C4", 37), ("C2", 8)])
def test_absorb_against_oracle(name, n_q):
    w = synth.workload(name)
    max_pos = 40000
    tab_lib = torch.from_numpy(gb.gva_rope_table_fill(max_pos, w.d_r, w.base)).cuda()
    rng = np.random.default_rng(11)
    q_pos = rng.integers(0, max_pos, size=n_q).astype(np.int32)
    q_pos[0] = 0
    M = synth.weights(w)
    q_nope, q_rope = synth.queries(w, n_q)
    out = torch.full((n_q, w.H, w.d_h + w.d_r), float("nan"), device="cuda")
    dims = gb.GvaDims(w.H, w.G, w.d_h, w.d_n, w.d_r)
    gb.gva_absorb_query(dims, torch.from_numpy(q_nope).cuda(), torch.from_numpy(q_rope).cuda(),
                        torch.from_numpy(q_pos).cuda(), torch.from_numpy(M).cuda(), tab_lib,
                        max_pos, out)
    got = out.cpu().numpy()
    tab = O.rope_rows(q_pos, w.d_r, w.base)
    qt, r = O.absorb(q_nope, q_rope, np.arange(n_q), M, tab)
    # rotated slice: one rounding of the float64 rotation, bit for bit
    assert np.array_equal(got[..., w.d_h:].view(np.uint32), O.f32_bits(r))
    assert np.array_equal(got[0, :, w.d_h:], q_rope[0])       # position 0 is the identity
    # content slice: float32 accumulation over d_n products, |err| <= gamma_{d_n} sum |M_ij q_j|
    u = 2.0 ** -24
    gamma = w.d_n * u / (1 - w.d_n * u)
    bound = gamma * np.einsum("hik,nhk->nhi", np.abs(M.astype(np.float64)),
                              np.abs(q_nope.astype(np.float64))) + 1e-30
    err = np.abs(got[..., : w.d_h] - qt)
    assert np.all(err <= bound), float(np.max(err / bound))


def test_absorb_bad_position_gives_nan_and_flag():
    w = synth.workload("C1")
    max_pos = 16
    tab_lib = torch.from_numpy(gb.gva_rope_table_fill(max_pos, w.d_r)).cuda()
    q_nope, q_rope = synth.queries(w, 3)
    q_pos = torch.tensor([3, 16, -1], dtype=torch.int32, device="cuda")
    out = torch.zeros((3, w.H, w.d_h + w.d_r), device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    dims = gb.GvaDims(w.H, w.G, w.d_h, w.d_n, w.d_r)
    gb.gva_absorb_query(dims, torch.from_numpy(q_nope).cuda(), torch.from_numpy(q_rope).cuda(),
                        q_pos, torch.from_numpy(synth.weights(w)).cuda(), tab_lib, max_pos, out,
                        err_flag=flag)
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o[0])) and np.all(np.isnan(o[1])) and np.all(np.isnan(o[2]))
    assert int(flag.item()) == gb.DEVERR_ROPE
