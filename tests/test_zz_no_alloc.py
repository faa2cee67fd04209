"""gva_decode_noalloc (the allocation-free decode, partials in the library's static device scratch)
against gva_decode with a caller workspace: two calls in a row, the second with a smaller input,
each bit-identical to gva_decode on the same arguments and within the bf16 bar of the oracle."""
import numpy as np
import pytest
import torch

from value_only_kv_amd import binding as gb
from value_only_kv_amd import synth
from tests.gpu_cases import Case, check_output, lse_ok

pytestmark = pytest.mark.gpu


def _both(c, lens, q, num_splits=0, kernel=gb.GVA_KERNEL_AUTO):
    """(out, lse) of gva_decode_noalloc and of gva_decode on the same arguments."""
    w = c.w
    B, H = w.B, w.H
    lens = np.asarray(lens, np.int32)
    ml = int(lens.max())
    sl = torch.from_numpy(lens).cuda()
    qa = torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    res = []
    for noalloc in (True, False):
        out = torch.full((B, H, w.d_h), float("nan"), device="cuda")
        lse = torch.full((B, H), float("nan"), device="cuda")
        if noalloc:
            gb.gva_decode_noalloc(c.cdims, c.cache, B, sl, ml, qa, w.scale, out, lse,
                                  num_splits=num_splits, kernel=kernel)
        else:
            wsb = gb.gva_decode_workspace_bytes(c.cdims, B, ml, num_splits)
            ws = torch.zeros(max(wsb, 256) // 4, device="cuda")
            gb.gva_decode(c.cdims, c.cache, B, sl, ml, qa, w.scale, out, lse,
                          num_splits=num_splits, kernel=kernel, workspace=ws)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    return res


@pytest.mark.parametrize("num_splits,kernel", [(0, gb.GVA_KERNEL_AUTO), (5, gb.GVA_KERNEL_MFMA),
                                               (3, gb.GVA_KERNEL_GENERIC)])
def test_noalloc_matches_decode_twice_second_smaller(num_splits, kernel):
    w = synth.workload("C4", B=12, lengths_uniform=(200, 3000))
    c = Case(w)
    c.append_prefix()
    rng = np.random.default_rng(17)
    q = rng.standard_normal((w.B, w.H, w.d_h + w.d_r))
    # first call: every sequence at its full length
    (o1, l1), (r1, rl1) = _both(c, c.lens, q, num_splits, kernel)
    assert o1.tobytes() == r1.tobytes() and l1.tobytes() == rl1.tobytes()
    ref, ref_lse = c.oracle_decode(c.lens, q)
    check_output(o1, ref, "bf16", f"noalloc first call S={num_splits} k={kernel}")
    assert lse_ok(l1, ref_lse, 1e-3)[0]
    # second call: shorter histories (the scratch still holds the first call's partials)
    short = np.maximum(c.lens // 3, 1)
    short[0] = 0
    (o2, l2), (r2, rl2) = _both(c, short, q, num_splits, kernel)
    assert o2.tobytes() == r2.tobytes() and l2.tobytes() == rl2.tobytes()
    ref2, ref2_lse = c.oracle_decode(short, q)
    check_output(o2, ref2, "bf16", f"noalloc second call S={num_splits} k={kernel}")
    assert lse_ok(l2, ref2_lse, 1e-3)[0]
    assert np.all(o2[0] == 0) and np.all(np.isneginf(l2[0]))
    assert c.err_flag() == 0


def test_noalloc_merged_plan_twice_second_smaller():
    """The merged plan (d_h = 64, a small batch): its tickets live at the head of the static
    array, start at zero and are left at zero by every call."""
    w = synth.workload("C4", B=10, lengths_uniform=(300, 3000), H=16, G=4, d_h=64, d_n=64,
                       d_r=16)
    c = Case(w)
    c.append_prefix()
    assert gb.gva_decode_num_ranges(c.cdims, w.B, int(c.lens.max())) == 0
    rng = np.random.default_rng(23)
    q = rng.standard_normal((w.B, w.H, w.d_h + w.d_r))
    (o1, l1), (r1, rl1) = _both(c, c.lens, q)
    assert o1.tobytes() == r1.tobytes() and l1.tobytes() == rl1.tobytes()
    ref, ref_lse = c.oracle_decode(c.lens, q)
    check_output(o1, ref, "bf16", "noalloc merged first call")
    assert lse_ok(l1, ref_lse, 1e-3)[0]
    short = np.maximum(c.lens // 4, 1)
    short[3] = 0
    (o2, l2), (r2, rl2) = _both(c, short, q)
    assert o2.tobytes() == r2.tobytes() and l2.tobytes() == rl2.tobytes()
    ref2, ref2_lse = c.oracle_decode(short, q)
    check_output(o2, ref2, "bf16", "noalloc merged second call")
    assert lse_ok(l2, ref2_lse, 1e-3)[0]
    assert c.err_flag() == 0
