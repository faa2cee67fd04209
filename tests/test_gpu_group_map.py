"""GPU parity under a non-contiguous head -> group map (gva_dims.g_of_h): every entry point that
serves a group's heads reads the heads the map assigns to it. Each case runs the device path and
the oracle with the same map; a case where the map is ignored would read other groups' values."""
import numpy as np
import pytest
import torch

from oracle import gva_oracle as O
from value_only_kv_amd import binding as gb
from value_only_kv_amd import synth
from tests.gpu_cases import Case, absorbed_queries, check_output, lse_ok

pytestmark = pytest.mark.gpu

GENERIC, MFMA = gb.GVA_KERNEL_GENERIC, gb.GVA_KERNEL_MFMA


def _balanced_map(H, G, seed):
    """Every group holds exactly H / G heads, in a seeded shuffled order."""
    rng = np.random.default_rng(seed)
    m = np.repeat(np.arange(G), H // G)
    rng.shuffle(m)
    assert not np.array_equal(m, np.repeat(np.arange(G), H // G))
    return [int(g) for g in m]


def _decode_case(shape, seed, B=7, lo=0, hi=600):
    w = synth.workload("C4", B=B, lengths_uniform=(lo, hi), **shape)
    c = Case(w, g_of_h=_balanced_map(w.H, w.G, seed))
    c.append_prefix()
    return c


@pytest.mark.parametrize("kernel", [pytest.param(GENERIC, id="generic"), pytest.param(MFMA, id="mfma")])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
@pytest.mark.parametrize("shape", [
    dict(H=32, G=8, d_h=128, d_n=128, d_r=24),          # four heads per group
    dict(H=8, G=4, d_h=64, d_n=64, d_r=16),             # two heads per group
])
def test_decode_with_group_map(shape, num_splits, kernel):
    c = _decode_case(shape, 3)
    w = c.w
    q = np.random.default_rng(8).standard_normal((w.B, w.H, w.d_h + w.d_r))
    out, lse = c.decode(c.lens, q, num_splits=num_splits, kernel=kernel)
    ref, ref_lse = c.oracle_decode(c.lens, q)
    check_output(out, ref, "bf16", f"group map {shape} S={num_splits} k={kernel}")
    ok, e = lse_ok(lse, ref_lse, 1e-3)
    assert ok, e
    # the contiguous map gives a different answer on the same inputs
    plain = O.Dims(w.H, w.G, w.d_h, w.d_n, w.d_r)
    b = int(np.argmax(c.lens))
    V, kr = O.gather(c.pool, plain, b, int(c.lens[b]))
    o_plain, _ = O.decode_sequence(V, kr, plain, q[b], w.scale)
    assert np.max(np.abs(o_plain - out[b])) > 1e-2


@pytest.mark.parametrize("dtype", [pytest.param("bf16", id="matrix-core-one-launch"),
                                   pytest.param("f32", id="vector-alu-one-launch")])
def test_step_with_group_map(dtype):
    """gva_decode_step with a map: the append does not depend on it, the absorption and the
    decode follow it (both one-launch kernels)."""
    w = synth.workload("C4", B=5, lengths_uniform=(50, 500), H=16, G=4, d_h=64, d_n=64, d_r=16,
                       dtype=dtype)
    c = Case(w, g_of_h=_balanced_map(w.H, w.G, 5))
    assert gb.gva_decode_step_launches(c.cdims, c.cache, w.B, int(c.lens.max()) + 1, 0) == 1
    c.append_prefix()
    rng = np.random.default_rng(np.random.SeedSequence([4243, 1]))
    v_new = rng.standard_normal((w.B, w.G, w.d_h)).astype(np.float32)
    kr_raw = rng.standard_normal((w.B, w.d_r)).astype(np.float32)
    pos = c.lens.astype(np.int64)
    q_ref, (M, q_nope, q_rope) = absorbed_queries(w, w.B, pos, c.tab_ora)
    sl = pos + 1
    ml = int(sl.max())
    t = lambda x, dt: torch.from_numpy(np.ascontiguousarray(np.asarray(x, dt))).cuda()
    qa = torch.full((w.B, w.H, w.d_h + w.d_r), float("nan"), device="cuda")
    out = torch.full((w.B, w.H, w.d_h), float("nan"), device="cuda")
    lse = torch.full((w.B, w.H), float("nan"), device="cuda")
    wsb = gb.gva_decode_workspace_bytes(c.cdims, w.B, ml, 0)
    ws = torch.zeros(max(wsb, 256) // 4, device="cuda")
    gb.gva_decode_step(c.cdims, c.cache, w.B, t(pos, np.int32), t(v_new, np.float32),
                       t(kr_raw, np.float32), t(q_nope, np.float32), t(q_rope, np.float32),
                       t(M, np.float32), t(sl, np.int32), ml, w.scale, qa, out, lse, workspace=ws)
    torch.cuda.synchronize()
    O.append(c.pool, c.dims, np.arange(w.B), pos, v_new, kr_raw, c.tab_ora)
    v_dev, k_dev = c.device_bits()
    assert np.array_equal(v_dev, c.pool.v) and np.array_equal(k_dev, c.pool.kr)
    ref, ref_lse = c.oracle_decode(sl, q_ref)
    check_output(out.cpu().numpy(), ref, dtype, f"step with group map, {dtype}")
    ok, e = lse_ok(lse.cpu().numpy(), ref_lse, 1e-5 if dtype == "f32" else 1e-3)
    assert ok, e
    assert c.err_flag() == 0


def test_prefill_with_group_map():
    w = synth.workload("C5", B=3, T=0, chunk=70, append_one=False, lengths_uniform=None,
                       H=8, G=2, d_h=64, d_n=64, d_r=16)
    starts = np.array([100, 37, 0])
    c = Case(w, lens=starts, g_of_h=_balanced_map(w.H, w.G, 6))
    c.append_prefix()
    C = w.chunk
    v_new = np.zeros((w.B, C, w.G, w.d_h), np.float32)
    kr_new = np.zeros((w.B, C, w.d_r), np.float32)
    for b in range(w.B):
        v, kr = synth.sequence_tokens(w, b, int(starts[b]) + C)
        v_new[b], kr_new[b] = v[starts[b]:], kr[starts[b]:]
    q_abs = np.random.default_rng(5).standard_normal((w.B, C, w.H, w.d_h + w.d_r)).astype(np.float32)
    out = torch.full((w.B, C, w.H, w.d_h), float("nan"), device="cuda")
    lse = torch.full((w.B, C, w.H), float("nan"), device="cuda")
    gb.gva_prefill_chunk(c.cdims, c.cache, w.B, torch.from_numpy(starts.astype(np.int32)).cuda(),
                         int(starts.max()), C, torch.from_numpy(q_abs).cuda(),
                         torch.from_numpy(v_new).cuda(), torch.from_numpy(kr_new).cuda(), w.scale,
                         out, lse)
    torch.cuda.synchronize()
    ref, ref_lse, err = O.prefill(c.pool, c.dims, starts, C, q_abs.astype(np.float64), v_new,
                                  kr_new, w.scale, c.tab_ora)
    assert err == 0 and c.err_flag() == 0
    check_output(out.cpu().numpy(), ref, "bf16", "prefill with group map")
    ok, e = lse_ok(lse.cpu().numpy(), ref_lse, 1e-3)
    assert ok, e


def test_gqa_comparator_with_group_map():
    w = synth.workload("C4", B=4, lengths_uniform=(0, 500), H=16, G=4, d_h=64, d_n=64, d_r=16)
    gmap = _balanced_map(w.H, w.G, 7)
    lens = synth.lengths(w)
    cv, ck = Case(w, lens=lens, g_of_h=gmap), Case(w, lens=lens, g_of_h=gmap)
    for b in range(w.B):
        n = int(lens[b])
        if n:
            v, kr = synth.sequence_tokens(w, b, n)
            cv.append_tokens(np.full(n, b), np.arange(n), v, kr)
            ck.append_tokens(np.full(n, b), np.arange(n), synth.comparator_keys(w, b, n), kr)
    q = np.random.default_rng(9).standard_normal((w.B, w.H, w.d_h))
    ml = int(lens.max())
    out = torch.full((w.B, w.H, w.d_h), float("nan"), device="cuda")
    lse = torch.full((w.B, w.H), float("nan"), device="cuda")
    wsb = gb.gva_decode_workspace_bytes(cv.cdims, w.B, ml, 0)
    ws = torch.zeros(max(wsb, 256) // 4, device="cuda")
    gb.gva_gqa_decode(cv.cdims, cv.cache, ck.cache.v, w.B,
                      torch.from_numpy(lens.astype(np.int32)).cuda(), ml,
                      torch.from_numpy(q.astype(np.float32)).cuda(), w.scale, out, lse, workspace=ws)
    torch.cuda.synchronize()
    ref = np.zeros((w.B, w.H, w.d_h))
    for b in range(w.B):
        V, _ = O.gather(cv.pool, cv.dims, b, int(lens[b]))
        K, _ = O.gather(ck.pool, ck.dims, b, int(lens[b]))
        ref[b], _ = O.gqa_decode_sequence(K, V, cv.dims, q[b], w.scale)
    check_output(out.cpu().numpy(), ref, "bf16", "GQA comparator with group map")


def test_recon_comparator_with_group_map():
    w = synth.workload("C4", B=4, lengths_uniform=(1, 400), H=8, G=2, d_h=64, d_n=64, d_r=16)
    lens = synth.lengths(w)
    c = Case(w, lens=lens, g_of_h=_balanced_map(w.H, w.G, 10))
    c.append_prefix()
    q, M, Mt = synth.recon_inputs(w)
    q_pos = lens - 1
    max_pos, ml = int(lens.max()) + 8, int(lens.max())
    rope = torch.from_numpy(gb.gva_rope_table_fill(max_pos, w.d_n, w.base)).cuda()
    out = torch.full((w.B, w.H, w.d_h), float("nan"), device="cuda")
    wsb = gb.gva_recon_decode_workspace_bytes(c.cdims, w.B, ml, 0)
    ws = torch.zeros(max(wsb, 256) // 4, device="cuda")
    scale = 1.0 / float(np.sqrt(w.d_n))
    gb.gva_recon_decode(c.cdims, c.cache, w.B, torch.from_numpy(lens.astype(np.int32)).cuda(), ml,
                        torch.from_numpy(q.astype(np.float32)).cuda(),
                        torch.from_numpy(q_pos.astype(np.int32)).cuda(),
                        torch.from_numpy(np.ascontiguousarray(Mt).view(np.int16)).cuda(), rope,
                        max_pos, scale, out, None, workspace=ws)
    torch.cuda.synchronize()
    ref = np.zeros((w.B, w.H, w.d_h))
    for b in range(w.B):
        V, _ = O.gather(c.pool, c.dims, b, int(lens[b]))
        ref[b], _ = O.recon_decode_sequence(V, c.dims, q[b], int(q_pos[b]), M, scale, w.base)
    check_output(out.cpu().numpy(), ref, "bf16", "recon comparator with group map")
