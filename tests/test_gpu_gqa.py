"""GPU parity of the GQA comparator (gva_gqa_decode): a cache of G keys and G values per token,
both filled through gva_cache_append into pools of the same paged layout, decoded on the
matrix-core kernel skeleton of gva_decode, against the oracle's GQA decode."""
import numpy as np
import pytest
import torch

from oracle import gva_oracle as O
from value_only_kv_amd import binding as gb
from value_only_kv_amd import synth
from tests.gpu_cases import Case, check_output, lse_ok

pytestmark = pytest.mark.gpu


def _gqa_cases(w, lens):
    """Value cache and key cache: two Cases with the same seeded layout; the key cache's value
    pool holds the keys (appended with the same rounding)."""
    cv = Case(w, lens=lens)
    ck = Case(w, lens=lens)
    for b in range(w.B):
        n = int(lens[b])
        if n == 0:
            continue
        v, kr = synth.sequence_tokens(w, b, n)
        k = synth.comparator_keys(w, b, n)
        cv.append_tokens(np.full(n, b), np.arange(n), v, kr)
        ck.append_tokens(np.full(n, b), np.arange(n), k, kr)
    return cv, ck


def _run(cv, ck, lens, q, max_len=None):
    w = cv.w
    max_len = int(np.max(lens)) if max_len is None else max_len
    out = torch.full((w.B, w.H, w.d_h), float("nan"), device="cuda")
    lse = torch.full((w.B, w.H), float("nan"), device="cuda")
    wsb = gb.gva_decode_workspace_bytes(cv.cdims, w.B, max_len, 0)
    ws = torch.zeros(max(wsb, 256) // 4, dtype=torch.float32, device="cuda")
    gb.gva_gqa_decode(cv.cdims, cv.cache, ck.cache.v, w.B,
                      torch.from_numpy(np.asarray(lens, np.int32)).cuda(), max_len,
                      torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda(), w.scale, out,
                      lse, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _oracle(cv, ck, lens, q):
    w = cv.w
    out = np.zeros((w.B, w.H, w.d_h))
    lse = np.full((w.B, w.H), -np.inf)
    for b in range(w.B):
        V, _ = O.gather(cv.pool, cv.dims, b, int(lens[b]))
        K, _ = O.gather(ck.pool, ck.dims, b, int(lens[b]))
        out[b], lse[b] = O.gqa_decode_sequence(K, V, cv.dims, q[b], w.scale)
    return out, lse


@pytest.mark.parametrize("shape", [
    dict(H=32, G=8, d_h=128, d_n=128, d_r=24),      # the ragged-batch shape (balanced plan)
    dict(H=8, G=2, d_h=64, d_n=64, d_r=16),
    dict(H=16, G=16, d_h=128, d_n=128, d_r=16),     # one head per group
])
def test_gqa_comparator_ragged(shape):
    w = synth.workload("C4", B=7, lengths_uniform=(0, 900), **shape)
    lens = synth.lengths(w)
    lens[:4] = [0, 1, 33, 64]
    cv, ck = _gqa_cases(w, lens)
    q = np.random.default_rng(3).standard_normal((w.B, w.H, w.d_h)).astype(np.float32)
    out, lse = _run(cv, ck, lens, q)
    ref, ref_lse = _oracle(cv, ck, lens, q)
    check_output(out, ref, "bf16", f"gqa comparator {shape}")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert cv.err_flag() == 0


def test_gqa_comparator_single_long_sequence():
    """One sequence (the split grid with 128 chunks) of 20000 positions."""
    w = synth.workload("C4", B=1, lengths_uniform=(20000, 20000), H=32, G=8, d_h=128, d_n=128,
                       d_r=16)
    lens = synth.lengths(w)
    cv, ck = _gqa_cases(w, lens)
    q = np.random.default_rng(4).standard_normal((1, w.H, w.d_h)).astype(np.float32)
    out, lse = _run(cv, ck, lens, q)
    ref, ref_lse = _oracle(cv, ck, lens, q)
    check_output(out, ref, "bf16", "gqa comparator, one long sequence")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e


def test_gqa_comparator_rejects_bad_keys():
    w = synth.workload("C4", B=2, lengths_uniform=(10, 20))
    cv = Case(w)
    q = torch.zeros((2, w.H, w.d_h), device="cuda")
    out = torch.empty((2, w.H, w.d_h), device="cuda")
    with pytest.raises(gb.GVAError) as ei:
        gb.gva_gqa_decode(cv.cdims, cv.cache, None, 2, torch.tensor([5, 5], dtype=torch.int32).cuda(),
                          5, q, w.scale, out)
    assert ei.value.status == gb.GVA_ERR_INVALID_ARG
