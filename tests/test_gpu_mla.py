"""GPU parity of the MLA-style latent comparator (gva_mla_decode): one latent of width d_c per
token plus the shared positional key, read by every head, against the oracle's absorbed decode
with one group whose value is the latent (decode_sequence with G = 1, d_h = d_c), which the
oracle pins tie to the textbook form with up-projected keys and values."""
import numpy as np
import pytest
import torch

from oracle import gva_oracle as O
from value_only_kv_amd import binding as gb
from value_only_kv_amd import synth
from tests.gpu_cases import Case, check_output, lse_ok

pytestmark = pytest.mark.gpu


def _latent_case(H, d_c, d_r, B, lengths_uniform, fixed=None):
    """A latent pool filled through gva_cache_append, each latent row described as d_c / 256
    groups of 256 laid out token-major, so that the groups of a row are contiguous."""
    w = synth.workload("C4", B=B, lengths_uniform=lengths_uniform, H=H, G=d_c // 256, d_h=256,
                       d_n=256, d_r=d_r)
    lens = synth.lengths(w)
    if fixed is not None:
        lens[:len(fixed)] = fixed
    c = Case(w, lens=lens, group_major=False)
    c.append_prefix()
    return c, lens, gb.GvaDims(H, 1, d_c, d_c, d_r), O.Dims(H, 1, d_c, d_c, d_r)


def _run(c, dims, lens, q_abs, scale, num_splits=0, max_len=None):
    B = len(lens)
    max_len = int(np.max(lens)) if max_len is None else max_len
    out = torch.full((B, dims.H, dims.d_h), float("nan"), device="cuda")
    lse = torch.full((B, dims.H), float("nan"), device="cuda")
    wsb = gb.gva_mla_decode_workspace_bytes(dims, B, max_len, num_splits)
    ws = torch.zeros(max(wsb, 256) // 4, dtype=torch.float32, device="cuda")
    gb.gva_mla_decode(dims, c.cache, B, torch.from_numpy(np.asarray(lens, np.int32)).cuda(),
                      max_len, torch.from_numpy(np.ascontiguousarray(q_abs, np.float32)).cuda(),
                      scale, out, lse, num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _oracle(c, odims, lens, q_abs, scale, seqs=None):
    B = len(lens)
    out = np.zeros((B, odims.H, odims.d_h))
    lse = np.full((B, odims.H), -np.inf)
    for b in (range(B) if seqs is None else seqs):
        n = int(lens[b])
        V, kr = O.gather(c.pool, c.dims, b, n)
        out[b], lse[b] = O.decode_sequence(V.reshape(n, 1, odims.d_h), kr, odims, q_abs[b], scale)
    return out, lse


SHAPES = [
    dict(H=32, d_c=512, d_r=64),      # the DeepSeek-V2 latent width with a 64-wide RoPE key
    dict(H=16, d_c=256, d_r=32),
    dict(H=8, d_c=256, d_r=16),       # a positional key narrower than its 32-element step
    dict(H=32, d_c=256, d_r=64),
    dict(H=8, d_c=512, d_r=64),       # one wave stages the whole tile: the three-buffer ring
    dict(H=16, d_c=512, d_r=24),      # two waves; a positional key of 24 in one 32-element step
]


@pytest.mark.parametrize("num_splits", [0, 1, 3])
@pytest.mark.parametrize("shape", SHAPES)
def test_mla_ragged(shape, num_splits):
    c, lens, dims, odims = _latent_case(**shape, B=5, lengths_uniform=(0, 600),
                                        fixed=[0, 1, 33, 64])
    q = synth.mla_queries(c.w, shape["H"], shape["d_c"], shape["d_r"])
    scale = 1.0 / float(np.sqrt(shape["d_c"] + shape["d_r"]))
    out, lse = _run(c, dims, lens, q, scale, num_splits=num_splits)
    ref, ref_lse = _oracle(c, odims, lens, q, scale)
    check_output(out, ref, "bf16", f"latent {shape} S={num_splits}")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert c.err_flag() == 0


def test_mla_single_long_sequence():
    """One sequence of 20000 positions at d_c = 512, d_r = 64 (the split grid's chunks)."""
    c, lens, dims, odims = _latent_case(H=32, d_c=512, d_r=64, B=1,
                                        lengths_uniform=(20000, 20000))
    q = synth.mla_queries(c.w, 32, 512, 64, stream=2)
    scale = 1.0 / float(np.sqrt(576))
    out, lse = _run(c, dims, lens, q, scale)
    ref, ref_lse = _oracle(c, odims, lens, q, scale)
    check_output(out, ref, "bf16", "latent one long sequence")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
    assert c.err_flag() == 0


@pytest.mark.parametrize("num_splits", [1, 2])
def test_mla_length_error(num_splits):
    """A length above max_len gives a NaN row and the LENGTH bit; the other rows are unaffected."""
    c, lens, dims, odims = _latent_case(H=16, d_c=256, d_r=32, B=3, lengths_uniform=(100, 100))
    q = synth.mla_queries(c.w, 16, 256, 32)
    scale = 1.0 / float(np.sqrt(288))
    lens2 = lens.copy()
    lens2[1] = 101
    out, lse = _run(c, dims, lens2, q, scale, num_splits=num_splits, max_len=100)
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(lse[1]))
    ref, ref_lse = _oracle(c, odims, lens, q, scale, seqs=[0, 2])
    check_output(out[[0, 2]], ref[[0, 2]], "bf16", f"latent beside an error S={num_splits}")
    assert c.err_flag() & gb.DEVERR_LENGTH


def test_mla_graph_replays():
    """The call captured in a graph (the work queue's reset kernel, the decode, the combine):
    three replays, each after an eager call on other queries, equal the eager result bit for bit
    (whichever work-group takes an item, its arithmetic is the same)."""
    c, lens, dims, odims = _latent_case(H=32, d_c=512, d_r=64, B=6, lengths_uniform=(500, 5000))
    B, H, d_c = len(lens), 32, 512
    scale = 1.0 / float(np.sqrt(576))
    max_len = int(lens.max())
    q = torch.from_numpy(synth.mla_queries(c.w, H, d_c, 64)).cuda()
    q_other = torch.from_numpy(synth.mla_queries(c.w, H, d_c, 64, stream=4)).cuda()
    seq_len = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    wsb = gb.gva_mla_decode_workspace_bytes(dims, B, max_len, 0)
    ws = torch.zeros(max(wsb, 256) // 4, dtype=torch.float32, device="cuda")
    out = torch.full((B, H, d_c), float("nan"), device="cuda")
    lse = torch.full((B, H), float("nan"), device="cuda")

    def call(qq, stream):
        gb.gva_mla_decode(dims, c.cache, B, seq_len, max_len, qq, scale, out, lse,
                          workspace=ws, stream=stream)

    call(q, torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager_out, eager_lse = out.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(q, side)                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(q, torch.cuda.current_stream())
    for rep in range(3):
        call(q_other, torch.cuda.current_stream())     # eager work between the replays
        torch.cuda.synchronize()
        assert not torch.equal(out, eager_out)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out), f"replay {rep}"
        assert torch.equal(lse, eager_lse), f"replay {rep}"
    assert c.err_flag() == 0
