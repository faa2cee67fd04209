"""GPU parity of gva_decode's merged plan against the oracle: small batches (B G <= 256
sequence-groups) at d_h of 32 or 64 with the automatic split count decode in ONE launch, in
which K work-groups split each (sequence, group)'s positions and the last of them to finish
merges their partials (through tickets in the workspace's first 1024 bytes)."""
import numpy as np
import pytest
import torch

from value_only_kv_amd import binding as gb
from value_only_kv_amd import synth
from tests.gpu_cases import Case, check_output, lse_ok

pytestmark = pytest.mark.gpu

# (id, batch, lengths, head and width overrides of the ragged paged workload)
SHAPES = [
    pytest.param(9, (100, 3000), dict(H=16, G=4, d_h=64, d_n=64, d_r=16), id="h16-g4-d64-K7"),
    pytest.param(5, (100, 2000), dict(H=8, G=8, d_h=32, d_n=32, d_r=8), id="one-head-per-group-d32"),
    pytest.param(3, (50, 1500), dict(H=16, G=2, d_h=64, d_n=64, d_r=24), id="eight-heads-per-group"),
    pytest.param(20, (70, 700), dict(H=8, G=4, d_h=32, d_n=32, d_r=16), id="two-heads-per-group-K3"),
    pytest.param(64, (70, 600), dict(H=16, G=4, d_h=64, d_n=64, d_r=16), id="256-pairs-K1"),
]


def _case(B, lo_hi, kw):
    w = synth.workload("C4", B=B, lengths_uniform=lo_hi, **kw)
    c = Case(w)
    c.append_prefix()
    return c


class Merged:
    """gva_decode with one workspace kept across calls (as a caller would keep it)."""

    def __init__(self, c, max_len):
        self.c = c
        wsb = gb.gva_decode_workspace_bytes(c.cdims, c.w.B, max_len, 0)
        self.ws = torch.zeros(max(wsb, 256) // 4, dtype=torch.int32, device="cuda")

    def __call__(self, lens, q, max_len):
        c, w = self.c, self.c.w
        out = torch.full((w.B, w.H, w.d_h), float("nan"), device="cuda")
        lse = torch.full((w.B, w.H), float("nan"), device="cuda")
        gb.gva_decode(c.cdims, c.cache, w.B, torch.from_numpy(np.asarray(lens, np.int32)).cuda(),
                      int(max_len), torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda(),
                      w.scale, out, lse, num_splits=0, workspace=self.ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy()

    def tickets_zero(self):
        return bool(torch.all(self.ws[:256] == 0).item())


@pytest.mark.parametrize("B,lo_hi,kw", SHAPES)
def test_merged_plan_matches_oracle(B, lo_hi, kw):
    c = _case(B, lo_hi, kw)
    w = c.w
    ml = int(c.lens.max())
    assert gb.gva_decode_num_ranges(c.cdims, B, ml) == 0          # the merged plan, not ranges
    lens = c.lens.copy()
    edge = [0, 1, 17, 31, 32, 33, 64, 65]              # at most the appended lengths (>= 70)
    lens[:min(len(edge), B)] = edge[:B]
    assert np.all(lens <= c.lens)
    q = synth.direct_q_abs(w, B)
    run = Merged(c, ml)
    out, lse = run(lens, q, ml)
    ref, ref_lse = c.oracle_decode(lens, q.astype(np.float64))
    check_output(out, ref, "bf16", "merged plan")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert run.tickets_zero()
    # the same call again: bit-identical, and the tickets are back at zero
    out2, lse2 = run(lens, q, ml)
    assert out2.tobytes() == out.tobytes() and lse2.tobytes() == lse.tobytes()
    assert run.tickets_zero()
    assert c.err_flag() == 0


def test_merged_plan_max_len_far_above_the_lengths():
    """max_len cuts the runs, so most work-groups find nothing of their sequence to read."""
    c = _case(6, (3000, 3100), dict(H=16, G=4, d_h=64, d_n=64, d_r=16))
    lens = np.array([0, 1, 5, 40, 100, 33])
    q = synth.direct_q_abs(c.w, c.w.B)
    run = Merged(c, 3000)
    out, lse = run(lens, q, 3000)
    ref, ref_lse = c.oracle_decode(lens, q.astype(np.float64))
    check_output(out, ref, "bf16", "max_len above the lengths")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
    assert run.tickets_zero()


def test_merged_plan_poisons_rows_then_recovers():
    """A bad block and a bad length make their rows NaN and raise their bits; every work-group
    still takes its ticket, so the next call on the same workspace is correct."""
    c = _case(4, (200, 900), dict(H=16, G=4, d_h=64, d_n=64, d_r=16))
    q = synth.direct_q_abs(c.w, c.w.B)
    ml = int(c.lens.max())
    run = Merged(c, ml)
    lens = c.lens.copy()
    saved = c.block_table[1, 2].item()
    c.block_table[1, 2] = c.lay.num_blocks + 5
    lens[2] = ml + 1
    try:
        out, lse = run(lens, q, ml)
    finally:
        c.block_table[1, 2] = saved
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[2]))
    assert np.all(np.isnan(lse[1])) and np.all(np.isnan(lse[2]))
    assert np.all(np.isfinite(out[0])) and np.all(np.isfinite(out[3]))
    assert c.err_flag() & gb.DEVERR_BLOCK and c.err_flag() & gb.DEVERR_LENGTH
    ref, ref_lse = c.oracle_decode(c.lens, q.astype(np.float64))
    check_output(out[[0, 3]], ref[[0, 3]], "bf16", "healthy rows")
    assert run.tickets_zero()
    c.cache.err_flag.zero_()
    out, lse = run(c.lens, q, ml)
    check_output(out, ref, "bf16", "after the poisoned call")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
    assert c.err_flag() == 0


def test_merged_plan_against_explicit_splits():
    """The merged plan and the split grid (an explicit split count) agree to rounding."""
    c = _case(8, (3000, 4096), dict(H=16, G=4, d_h=64, d_n=64, d_r=16))
    q = synth.direct_q_abs(c.w, c.w.B)
    merged, lm = c.decode(c.lens, q, num_splits=0)
    split, ls = c.decode(c.lens, q, num_splits=16)
    assert np.max(np.abs(merged - split)) < 1e-4
    assert np.max(np.abs(lm - ls)) < 1e-4
