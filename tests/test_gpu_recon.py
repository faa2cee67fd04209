"""GPU parity of the non-absorbable comparator (gva_recon_decode): every step rebuilds each head's
content keys from the cached values and rotates them at their positions, against the oracle's
recon_decode_sequence (keys rotated at j and the query at p, in float64)."""
import numpy as np
import pytest
import torch

from oracle import gva_oracle as O
from value_only_kv_amd import binding as gb
from value_only_kv_amd import synth
from tests.gpu_cases import Case, check_output, lse_ok

pytestmark = pytest.mark.gpu


def _run(c, q, q_pos, Mt_bits, max_pos, max_len=None, num_splits=0, lens=None):
    w = c.w
    lens = c.lens if lens is None else np.asarray(lens)
    max_len = int(np.max(lens)) if max_len is None else max_len
    rope = torch.from_numpy(gb.gva_rope_table_fill(max_pos, w.d_n, w.base)).cuda()
    out = torch.full((w.B, w.H, w.d_h), float("nan"), device="cuda")
    lse = torch.full((w.B, w.H), float("nan"), device="cuda")
    wsb = gb.gva_recon_decode_workspace_bytes(c.cdims, w.B, max_len, num_splits)
    ws = torch.zeros(max(wsb, 256) // 4, dtype=torch.float32, device="cuda")
    gb.gva_recon_decode(c.cdims, c.cache, w.B,
                        torch.from_numpy(np.asarray(lens, np.int32)).cuda(), max_len,
                        torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda(),
                        torch.from_numpy(np.asarray(q_pos, np.int32)).cuda(),
                        torch.from_numpy(np.ascontiguousarray(Mt_bits).view(np.int16)).cuda(),
                        rope, max_pos, 1.0 / float(np.sqrt(w.d_n)), out, lse,
                        num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _oracle(c, q, q_pos, M, seqs=None):
    w = c.w
    out = np.zeros((w.B, w.H, w.d_h))
    lse = np.full((w.B, w.H), -np.inf)
    for b in (range(w.B) if seqs is None else seqs):
        V, _ = O.gather(c.pool, c.dims, b, int(c.lens[b]))
        out[b], lse[b] = O.recon_decode_sequence(V, c.dims, q[b], int(q_pos[b]), M,
                                                 1.0 / float(np.sqrt(w.d_n)), w.base)
    return out, lse


SHAPES = [
    dict(H=32, G=8, d_h=128, d_n=128, d_r=24),      # the ragged-batch shape, four heads per group
    dict(H=8, G=2, d_h=64, d_n=64, d_r=16),
    dict(H=16, G=8, d_h=128, d_n=64, d_r=16),       # two heads per group, d_n < d_h
    dict(H=6, G=2, d_h=64, d_n=128, d_r=16),        # three heads per group, d_n > d_h
    dict(H=8, G=8, d_h=128, d_n=128, d_r=16),       # one head per group
]


@pytest.mark.parametrize("num_splits", [0, 1, 3])
@pytest.mark.parametrize("shape", SHAPES)
def test_recon_ragged(shape, num_splits):
    w = synth.workload("C4", B=6, lengths_uniform=(0, 700), **shape)
    lens = synth.lengths(w)
    lens[:4] = [0, 1, 33, 64]
    c = Case(w, lens=lens)
    c.append_prefix()
    q, M, Mt = synth.recon_inputs(w)
    q_pos = np.maximum(lens - 1, 0)                 # the query is the last cached token
    out, lse = _run(c, q, q_pos, Mt, int(lens.max()) + 8, num_splits=num_splits)
    ref, ref_lse = _oracle(c, q, q_pos, M)
    check_output(out, ref, "bf16", f"recon {shape} S={num_splits}")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert c.err_flag() == 0


def test_recon_query_before_keys_and_far_ahead():
    """Query positions before most cached keys (negative offsets p - j0, read from the table row
    of the magnitude with the sine negated) and far beyond them."""
    w = synth.workload("C4", B=3, lengths_uniform=(300, 300), H=8, G=2, d_h=64, d_n=64, d_r=16)
    lens = synth.lengths(w)
    c = Case(w, lens=lens)
    c.append_prefix()
    q, M, Mt = synth.recon_inputs(w, stream=5)
    q_pos = np.array([5, 299, 4000])
    for S in (0, 1):
        out, lse = _run(c, q, q_pos, Mt, 4001, num_splits=S)
        ref, ref_lse = _oracle(c, q, q_pos, M)
        check_output(out, ref, "bf16", f"recon query positions S={S}")
        ok, e = lse_ok(lse, ref_lse, 1e-3)
        assert ok, e
    assert c.err_flag() == 0


def test_recon_single_long_sequence():
    """One sequence of 20000 positions at the ragged-batch shape (the split grid's chunks)."""
    w = synth.workload("C4", B=1, lengths_uniform=(20000, 20000), H=32, G=8, d_h=128, d_n=128,
                       d_r=24)
    lens = synth.lengths(w)
    c = Case(w, lens=lens)
    c.append_prefix()
    q, M, Mt = synth.recon_inputs(w)
    q_pos = lens - 1
    out, lse = _run(c, q, q_pos, Mt, int(lens.max()) + 1)
    ref, ref_lse = _oracle(c, q, q_pos, M)
    check_output(out, ref, "bf16", "recon one long sequence")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
    assert c.err_flag() == 0


@pytest.mark.parametrize("num_splits", [1, 2])
def test_recon_device_errors(num_splits):
    """A query position outside the RoPE table and a length above max_len give NaN rows and their
    error bits; the other sequence is unaffected."""
    w = synth.workload("C4", B=3, lengths_uniform=(100, 100), H=8, G=2, d_h=64, d_n=64, d_r=16)
    lens = synth.lengths(w)
    c = Case(w, lens=lens)
    c.append_prefix()
    q, M, Mt = synth.recon_inputs(w)
    q_pos = np.array([99, 500, 99])                 # sequence 1: beyond the 200-row table
    lens2 = lens.copy()
    lens2[2] = 101                                  # sequence 2: above max_len = 100
    out, lse = _run(c, q, q_pos, Mt, 200, max_len=100, num_splits=num_splits, lens=lens2)
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(lse[1]))
    assert np.all(np.isnan(out[2])) and np.all(np.isnan(lse[2]))
    ref, ref_lse = _oracle(c, q, q_pos, M, seqs=[0])
    check_output(out[:1], ref[:1], "bf16", f"recon beside errors S={num_splits}")
    ok, e = lse_ok(lse[:1], ref_lse[:1], 1e-3)
    assert ok, e
    flag = c.err_flag()
    assert flag & gb.DEVERR_ROPE and flag & gb.DEVERR_LENGTH, flag
