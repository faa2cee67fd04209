"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: values printed on the
pages (tests/golden), closed forms, invariants, library routines used as independent
definitions (torch's scaled_dot_product_attention, scipy's logsumexp, complex
multiplication), and pure-Python brute force on tiny inputs.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import gva_oracle as O
from value_only_kv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------------------
# RoPE table and rotation
# ----------------------------------------------------------------------------------------


def test_rope_table_closed_forms():
    d_r, base = 16, 10000.0
    tab = O.rope_table(300, d_r, base)
    assert tab.shape == (300, 8, 2)
    # position 0 is the identity rotation, exactly
    assert np.all(tab[0, :, 0] == 1.0) and np.all(tab[0, :, 1] == 0.0)
    # pair 0 has frequency 1: the angle is the position itself
    for p in (1, 2, 17, 299):
        assert tab[p, 0, 0] == math.cos(p) and tab[p, 0, 1] == math.sin(p)
    # frequencies fall geometrically: theta_i = base^(-2i/d_r)
    th = O.rope_theta(d_r, base)
    assert th[0] == 1.0
    ratios = [th[i + 1] / th[i] for i in range(len(th) - 1)]
    assert np.allclose(ratios, base ** (-2 / d_r), rtol=1e-14)
    # an independent evaluation (numpy's vectorised cos/sin) agrees to rounding
    p = np.arange(300)[:, None] * np.array(th)[None, :]
    assert np.max(np.abs(tab[..., 0] - np.cos(p))) < 4e-16 * 300
    assert np.max(np.abs(tab[..., 1] - np.sin(p))) < 4e-16 * 300
    # cos^2 + sin^2 = 1
    assert np.max(np.abs(tab[..., 0] ** 2 + tab[..., 1] ** 2 - 1)) < 1e-15
    # the row-only helper gives the same rows, bit for bit
    rows = O.rope_rows(np.array([0, 5, 299]), d_r, base)
    assert np.array_equal(rows, tab[[0, 5, 299]])


def test_rotate_matches_complex_multiplication():
    rng = np.random.default_rng(1)
    d_r = 24
    x = rng.standard_normal((50, d_r))
    pos = rng.integers(0, 5000, size=50)
    tab = O.rope_rows(pos, d_r)
    y = O.rotate(x, tab)
    th = O.rope_theta(d_r, 10000.0)
    for k in range(50):
        for i in range(d_r // 2):
            z = complex(x[k, 2 * i], x[k, 2 * i + 1]) * cmath.exp(1j * pos[k] * th[i])
            assert abs(y[k, 2 * i] - z.real) < 1e-12 and abs(y[k, 2 * i + 1] - z.imag) < 1e-12


def test_rotate_invariants():
    rng = np.random.default_rng(2)
    d_r = 16
    q = rng.standard_normal(d_r)
    k = rng.standard_normal(d_r)
    # position 0 is the identity, exactly
    assert np.array_equal(O.rotate(q, O.rope_rows([0], d_r)[0]), q)
    # rotation keeps the norm
    for p in (1, 100, 9999):
        y = O.rotate(q, O.rope_rows([p], d_r)[0])
        assert abs(np.linalg.norm(y) - np.linalg.norm(q)) < 1e-14 * np.linalg.norm(q)
    # the positional score depends only on the offset between query and key positions
    def score(pq, pk):
        return O.rotate(q, O.rope_rows([pq], d_r)[0]) @ O.rotate(k, O.rope_rows([pk], d_r)[0])
    for pq, pk, delta in ((10, 3, 100), (500, 20, 1234), (7, 7, 31)):
        assert abs(score(pq, pk) - score(pq + delta, pk + delta)) < 1e-11
    # a wrong sign in either rotated component breaks the offset property
    bad = O.rotate(q, O.rope_rows([10], d_r)[0]) * np.tile([1, -1], d_r // 2)
    assert abs(bad @ O.rotate(k, O.rope_rows([3], d_r)[0]) - score(10, 3)) > 1e-6


# ----------------------------------------------------------------------------------------
# Rounding to the cache type
# ----------------------------------------------------------------------------------------


def _all_bf16_sorted():
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    keep = np.isfinite(vals)
    return vals[keep], bits[keep].astype(np.uint16)


def _brute_bf16(x, vals_sorted, bits_sorted):
    """Nearest bfloat16 by search over every finite value; ties go to the even pattern."""
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0x0000
    maxv = float(vals_sorted[-1])
    if abs(x) >= maxv + (maxv - float(np.nextafter(np.float32(maxv), 0))) / 2 \
            and abs(x) > maxv:
        # beyond the midpoint between the largest finite value and the next power: infinity
        half_ulp = 2.0 ** (127 - 8)
        if abs(x) >= maxv + half_ulp:
            return 0xFF80 if x < 0 else 0x7F80
    j = int(np.searchsorted(vals_sorted, x))
    cands = []
    for k in (j - 1, j):
        if 0 <= k < len(vals_sorted):
            cands.append((abs(float(vals_sorted[k]) - x), int(bits_sorted[k]), float(vals_sorted[k])))
    best = min(c[0] for c in cands)
    tied = [c for c in cands if c[0] == best]
    if len(tied) == 1:
        b = tied[0][1]
    else:
        b = [c[1] for c in tied if (c[1] & 1) == 0][0]
    # the two zeros have equal value; keep the sign of x
    if float(np.uint32(b << 16).view(np.float32)) == 0.0:
        return 0x8000 if x < 0 else 0x0000
    return b


def test_bf16_rounding_against_brute_force():
    vals, bits = _all_bf16_sorted()
    order = np.argsort(vals, kind="stable")
    vals, bits = vals[order], bits[order]
    # drop the duplicate zero so searchsorted sees distinct values
    keep = np.ones(len(vals), dtype=bool)
    zero = np.nonzero(vals == 0.0)[0]
    keep[zero[1:]] = False
    vals, bits = vals[keep], bits[keep]
    rng = np.random.default_rng(3)
    xs = list(rng.standard_normal(3000))
    xs += list(rng.standard_normal(500) * 1e-39)          # bfloat16 subnormals
    xs += list(rng.standard_normal(300) * 1e38)           # near the top of the range
    # exact midpoints between neighbours (ties) and their immediate neighbours
    for _ in range(400):
        k = int(rng.integers(0, len(vals) - 1))
        a, b = float(vals[k]), float(vals[k + 1])
        mid = (a + b) / 2
        xs += [mid, float(np.nextafter(mid, -np.inf)), float(np.nextafter(mid, np.inf))]
    xs += [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8, 3.3895313892515355e38,
           3.4e38, -3.5e38, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 0.0, -0.0]
    got = O.bf16_bits(np.array(xs))
    for x, g in zip(xs, got):
        want = _brute_bf16(x, vals, bits)
        assert int(g) == want, (x, hex(int(g)), hex(want))


def test_bf16_known_patterns():
    cases = {1.0: 0x3F80, -2.0: 0xC000, 1.0 + 2.0 ** -8: 0x3F80, 1.0 + 3 * 2.0 ** -8: 0x3F82,
             0.1: 0x3DCD, 3.0e38: 0x7F62, 1e39: 0x7F80}
    got = O.bf16_bits(np.array(list(cases.keys())))
    assert [int(g) for g in got] == list(cases.values())
    # float64 rounding happens once: 1 + 2^-8 + 2^-30 rounds up, although a detour through
    # float32 would first land on the tie 1 + 2^-8 and then round down to even
    assert int(O.bf16_bits(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0]) == 0x3F81
    # bits -> value -> bits round-trips every finite pattern
    b = np.arange(0, 1 << 16, dtype=np.uint16)
    v = O.bf16_value(b)
    fin = np.isfinite(v)
    assert np.array_equal(O.bf16_bits(v[fin]), b[fin])


def test_f32_rounding_known_values():
    xs = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 1.0 + 2.0 ** -24 + 2.0 ** -40])
    got = O.f32_value(O.f32_bits(xs))
    assert list(got) == [1.0, 1.0 + 2.0 ** -22, 1.0 + 2.0 ** -23]


def test_cache_bits_known_patterns():
    """The cache's storage conversion for both element types, against bit patterns written out
    by hand: 1 is 0x3f80 / 0x3f800000, pi rounds to 0x4049 (3.140625) in bfloat16, 1 + 2^-8 is
    a tie that goes to the even pattern 0x3f80, -2 is 0xc000 / 0xc0000000."""
    xs = np.array([1.0, np.pi, 1.0 + 2.0 ** -8, -2.0])
    assert list(O.to_cache_bits(xs, "bf16")) == [0x3F80, 0x4049, 0x3F80, 0xC000]
    assert list(O.to_cache_bits(xs, "f32")) == [0x3F800000, 0x40490FDB, 0x3F808000, 0xC0000000]
    assert list(O.from_cache_bits(np.array([0x3F80, 0x4049, 0xC000], np.uint16), "bf16")) == \
        [1.0, 3.140625, -2.0]
    assert list(O.from_cache_bits(np.array([0x3F808000], np.uint32), "f32")) == [1.0 + 2.0 ** -8]


# ----------------------------------------------------------------------------------------
# Cache accounting against the pages' numbers
# ----------------------------------------------------------------------------------------


def test_cache_ledger_against_pages():
    g = _golden("gva_cache_ledger.json")
    G, d_h = g["G"], g["d_h"]
    T = 4096
    for row in g["savings_percent_rounded"]:
        ratio = O.gva_cache_scalars(T, G, d_h, row["d_r"]) / O.gqa_cache_scalars(T, G, d_h)
        assert ratio == 0.5 + row["d_r"] / (2 * G * d_h)
        assert round(100 * (1 - ratio)) == row["percent"]
    assert O.gva_cache_scalars(T, G, d_h, 0) / O.gqa_cache_scalars(T, G, d_h) == \
        g["without_positional_slice_ratio"]
    # exact values at G d_h = 256: 46.875% and 45.3125%
    assert 1 - O.gva_cache_scalars(T, 4, 64, 16) / O.gqa_cache_scalars(T, 4, 64) == 0.46875
    assert 1 - O.gva_cache_scalars(T, 4, 64, 24) / O.gqa_cache_scalars(T, 4, 64) == 0.453125
    # streams per layer: G value streams plus one shared positional stream
    G8, H = 8, 32
    assert O.gva_cache_scalars(1, G8, 128, 16) == G8 * 128 + 16
    assert O.mha_cache_scalars(1, H, 128) == 2 * H * 128


def test_kv_byte_accounting_against_pages():
    g = _golden("kvcache_bytes.json")
    for row in g["per_token_per_layer"]:
        assert O.kv_cache_bytes(1, 1, 1, row["kv_heads"], row["d_h"], row["elem_bytes"]) == row["bytes"]
    st = g["shape_table"]
    for row in st["rows"]:
        per_tok = O.kv_cache_bytes(1, 1, 1, row["kv_heads"], st["d_h"], st["elem_bytes"])
        assert per_tok / 1024 == row["per_token_per_layer_KiB"]
        total = O.kv_cache_bytes(st["layers"], st["batch"], st["T"], row["kv_heads"], st["d_h"],
                                 st["elem_bytes"])
        assert total / 2 ** 20 == row["model_total_MiB"]


def test_decode_bytes_definition():
    # C3: T = 131072, G = 8, d_h = 128, d_r = 16, bf16 -> 272,629,760 bytes
    assert O.gva_decode_bytes(131072, 8, 128, 16, 2) == 272629760
    assert O.gva_decode_bytes(131072, 8, 128, 24, 2) == 274726912
    # one token's flops: H (2 (d_h + d_r) + 2 d_h)
    assert O.gva_decode_flops(1, 32, 128, 16) == 32 * (2 * 144 + 256)


# ----------------------------------------------------------------------------------------
# Attention: printed example, library definitions, brute force, special cases
# ----------------------------------------------------------------------------------------


def test_worked_example_from_kvcache_page():
    """The MQA example is GVA with d_h = d_n = 2, M = 0.1 I (so K = V M = I), no positional
    slice and no scaling."""
    g = _golden("kvcache_mqa_worked_example.json")
    V = np.array(g["values"], dtype=np.float64)
    M = 0.1 * np.eye(2)
    assert np.array_equal(V @ M, np.array(g["keys"], dtype=np.float64))
    dims = O.Dims(H=1, G=1, d_h=2, d_n=2, d_r=0)
    for case in g["cases"]:
        q = np.array(case["query"], dtype=np.float64)
        qt = M @ q
        s = V @ qt
        assert np.allclose(s, case["scores"], rtol=0, atol=1e-15)
        o, lse, w = O.softmax_attend(g["scale"] * s, V)
        assert [round(x, 2) for x in w] == case["weights_2dp"]
        assert [round(x, 1) for x in o] == case["output_1dp"]
        # closed form: w = (e^2, 1) / (e^2 + 1) for scores (2, 0)
        e2 = math.exp(2.0)
        big = e2 / (e2 + 1)
        assert abs(max(w) - big) < 1e-15 and abs(min(w) - 1 / (e2 + 1)) < 1e-15
        assert abs(lse - math.log(e2 + 1)) < 1e-15
        # the materialised form gives the same result
        o2, lse2 = O.decode_materialized(V[:, None, :], np.zeros((2, 0)), dims, q[None],
                                         np.zeros((1, 0)), M[None], g["scale"])
        assert np.allclose(o2[0], o, rtol=0, atol=1e-14)


def _tiny_case(seed, H=4, G=2, n=7, d_h=6, d_n=5, d_r=4):
    rng = np.random.default_rng(seed)
    V = rng.standard_normal((n, G, d_h))
    kr = rng.standard_normal((n, d_r))
    q_nope = rng.standard_normal((H, d_n))
    r = rng.standard_normal((H, d_r))
    M = rng.standard_normal((H, d_h, d_n)) / math.sqrt(d_h)
    return V, kr, q_nope, r, M, O.Dims(H=H, G=G, d_h=d_h, d_n=d_n, d_r=d_r)


def _brute_force_attention(V, kr, q_nope, r, M, dims, scale):
    """Pure-Python loops: build every content key K_h[j] = V_g(h)[j] M_h, score, softmax."""
    n = len(V)
    out = [[0.0] * dims.d_h for _ in range(dims.H)]
    lse = [0.0] * dims.H
    per = dims.H // dims.G
    for h in range(dims.H):
        g = h // per
        scores = []
        for j in range(n):
            key = [sum(V[j][g][i] * M[h][i][k] for i in range(dims.d_h)) for k in range(dims.d_n)]
            s = sum(q_nope[h][k] * key[k] for k in range(dims.d_n))
            s += sum(r[h][i] * kr[j][i] for i in range(dims.d_r))
            scores.append(scale * s)
        mx = max(scores)
        ex = [math.exp(s - mx) for s in scores]
        z = sum(ex)
        lse[h] = mx + math.log(z)
        for i in range(dims.d_h):
            out[h][i] = sum(ex[j] / z * V[j][g][i] for j in range(n))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_absorbed_decode_equals_brute_force_materialized(seed):
    V, kr, q_nope, r, M, dims = _tiny_case(seed)
    scale = 0.37
    qt = np.einsum("hik,hk->hi", M, q_nope)
    q_abs = np.concatenate([qt, r], axis=-1)
    out, lse = O.decode_sequence(V, kr, dims, q_abs, scale)
    out_m, lse_m = O.decode_materialized(V, kr, dims, q_nope, r, M, scale)
    out_b, lse_b = _brute_force_attention(V.tolist(), kr.tolist(), q_nope.tolist(), r.tolist(),
                                          M.tolist(), dims, scale)
    for o2, l2 in ((out_m, lse_m), (out_b, lse_b)):
        assert np.max(np.abs(out - o2)) < 1e-12 * max(1.0, np.max(np.abs(o2)))
        assert np.max(np.abs(lse - l2)) < 1e-12 * max(1.0, np.max(np.abs(l2)))
    # the oracle's absorb produces the same q~ as the einsum above
    tab = np.zeros((1, dims.d_r // 2, 2))
    tab[0, :, 0] = 1.0
    qt2, r2 = O.absorb(q_nope[None], r[None], [0], M, tab)
    assert np.max(np.abs(qt2[0] - qt)) < 1e-13 and np.array_equal(r2[0], r)


def test_absorbed_decode_transposed_map_is_detected():
    """Using M_h^T instead of M_h (same square shape) must change the result."""
    V, kr, q_nope, r, M, dims = _tiny_case(5, d_h=5, d_n=5)
    qt_bad = np.einsum("hki,hk->hi", M, q_nope)
    out_bad, _ = O.decode_sequence(V, kr, dims, np.concatenate([qt_bad, r], -1), 0.5)
    out_m, _ = O.decode_materialized(V, kr, dims, q_nope, r, M, 0.5)
    assert np.max(np.abs(out_bad - out_m)) > 1e-3


def _sdpa_reference(V, kr, q_nope, r, M, dims, scale, mask=None):
    """torch scaled_dot_product_attention in float64 on the CPU, with the keys written out:
    Q_h = [q_nope_h ; r_h], K_h = [V_g M_h ; kr], values V_g."""
    H = dims.H
    per = H // dims.G
    Vt = torch.tensor(V, dtype=torch.float64)
    krt = torch.tensor(kr, dtype=torch.float64)
    outs = []
    for h in range(H):
        g = h // per
        K = torch.cat([Vt[:, g, :] @ torch.tensor(M[h], dtype=torch.float64), krt], dim=1)
        Q = torch.cat([torch.tensor(q_nope[h], dtype=torch.float64).reshape(-1, dims.d_n),
                       torch.tensor(r[h], dtype=torch.float64).reshape(-1, dims.d_r)], dim=1)
        o = torch.nn.functional.scaled_dot_product_attention(
            Q[None, None], K[None, None], Vt[:, g, :][None, None], attn_mask=mask, scale=scale)
        outs.append(o[0, 0])
    return torch.stack(outs, dim=0).numpy()


def test_decode_against_sdpa_at_c1_size():
    w = synth.workload("C1")
    dims = O.Dims(w.H, w.G, w.d_h, w.d_n, w.d_r)
    v, kr_raw = synth.sequence_tokens(w, 0, w.T)
    M = synth.weights(w)
    q_nope, q_rope = synth.queries(w, 1)
    tab = O.rope_table(w.T + 1, w.d_r)
    kr = O.rotate(kr_raw, tab[: w.T])
    V = v.astype(np.float64)
    qt, r = O.absorb(q_nope, q_rope, [w.T], M, tab)
    out, lse = O.decode_sequence(V, kr, dims, O.q_abs_of(qt, r)[0], w.scale)
    ref = _sdpa_reference(V, kr, q_nope[0].astype(np.float64), r[0], M.astype(np.float64), dims,
                          w.scale)
    assert np.max(np.abs(out - ref[:, 0, :])) < 1e-12
    # lse against scipy's logsumexp of the materialised scores
    for h in range(w.H):
        g = h // w.heads_per_group
        K = V[:, g, :] @ M[h].astype(np.float64)
        s = w.scale * (K @ q_nope[0, h].astype(np.float64) + kr @ r[0, h])
        assert abs(lse[h] - logsumexp(s)) < 1e-12
        # softmax weights sum to one
        _, _, wts = O.softmax_attend(s, V[:, g, :])
        assert abs(wts.sum() - 1.0) < 1e-14


def test_decode_special_cases():
    V, kr, q_nope, r, M, dims = _tiny_case(11, H=4, G=2, n=9, d_h=6, d_n=6, d_r=4)
    # one cached entry: the output is that entry's value, exactly
    q_abs = np.random.default_rng(0).standard_normal((dims.H, dims.d_h + dims.d_r))
    out, lse = O.decode_sequence(V[:1], kr[:1], dims, q_abs, 0.7)
    for h in range(dims.H):
        assert np.array_equal(out[h], V[0, dims.group_of(h)])
    # zero query: uniform weights, the output is the mean of the group's values
    out, lse = O.decode_sequence(V, kr, dims, np.zeros_like(q_abs), 0.7)
    for h in range(dims.H):
        assert np.allclose(out[h], V[:, dims.group_of(h)].mean(axis=0), atol=1e-15)
        assert abs(lse[h] - math.log(V.shape[0])) < 1e-15
    # M = c I: q~ = c q_nope, i.e. GQA attention with keys equal to (scaled) values
    c = 0.25
    Mi = np.stack([c * np.eye(6)] * dims.H)
    qt, _ = O.absorb(q_nope[None], r[None], [0], Mi, np.tile([1.0, 0.0], (1, 2, 1)))
    assert np.allclose(qt[0], c * q_nope, atol=1e-15)
    out_m, _ = O.decode_materialized(V, kr, dims, q_nope, r, Mi, 0.7)
    out_a, _ = O.decode_sequence(V, kr, dims, np.concatenate([qt[0], r], -1), 0.7)
    assert np.allclose(out_m, out_a, atol=1e-14)
    # empty history: output 0 and lse = -inf
    out, lse = O.decode_sequence(V[:0], kr[:0], dims, q_abs, 0.7)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("num_splits", [1, 2, 3, 64, 256])
def test_split_combine_equals_direct(num_splits):
    rng = np.random.default_rng(num_splits)
    n, d = 700, 8
    s = rng.standard_normal(n) * 3
    Vv = rng.standard_normal((n, d))
    o_ref, lse_ref, _ = O.softmax_attend(s, Vv)
    chunk = -(-n // num_splits)
    # some splits past the end are empty when num_splits does not divide evenly
    parts = O.decode_partials(s, Vv, chunk, num_splits + 3)
    o, lse = O.combine(parts)
    assert np.max(np.abs(o - o_ref)) < 1e-13 and abs(lse - lse_ref) < 1e-13


# ----------------------------------------------------------------------------------------
# Append: paging indices, sentinels, one rounding
# ----------------------------------------------------------------------------------------


def _small_paged(dtype="bf16", bs=4, group_major=True):
    w = synth.workload("C4", B=5, H=4, G=2, d_h=8, d_n=8, d_r=4, lengths_uniform=(3, 13),
                       block_size=bs, dtype=dtype)
    lens = synth.lengths(w)
    lay = synth.layout(w, lens, group_major=group_major)
    return w, lens, lay


@pytest.mark.parametrize("group_major", [True, False])
def test_paging_is_a_bijection_and_append_leaves_other_bytes(group_major):
    w, lens, lay = _small_paged(group_major=group_major)
    dims = O.Dims(w.H, w.G, w.d_h, w.d_n, w.d_r)
    sentinel = 0x7FC1
    pool = O.Pool.empty(w.dtype, lay.v_elems, lay.kr_elems,
                        (lay.v_sb, lay.v_st, lay.v_sg, lay.kr_sb, lay.kr_st),
                        lay.num_blocks, lay.block_size, lay.block_table, sentinel=sentinel)
    tab = O.rope_table(64, w.d_r)
    seen = set()
    written = np.zeros(lay.v_elems, dtype=bool)
    kwritten = np.zeros(lay.kr_elems, dtype=bool)
    cap = synth.capacity(w, lens)
    for b in range(w.B):
        for p in range(int(cap[b])):
            blk, off = pool.slot(b, p)
            assert 0 <= blk < lay.num_blocks and (blk, off) not in seen
            seen.add((blk, off))
            for g in range(w.G):
                o = blk * lay.v_sb + off * lay.v_st + g * lay.v_sg
                written[o:o + w.d_h] = True
            o = blk * lay.kr_sb + off * lay.kr_st
            kwritten[o:o + w.d_r] = True
        v, kr_raw = synth.sequence_tokens(w, b, int(cap[b]))
        err = O.append(pool, dims, np.full(int(cap[b]), b), np.arange(int(cap[b])), v, kr_raw, tab)
        assert err == 0
        V, kr = O.gather(pool, dims, b, int(cap[b]))
        assert np.array_equal(V, O.round_bf16(v.astype(np.float64)))
        rot = O.rotate(kr_raw, tab[: int(cap[b])])
        assert np.array_equal(kr, O.round_bf16(rot))
        # position 0 stores the raw key after one rounding
        assert np.array_equal(kr[0], O.round_bf16(kr_raw[0].astype(np.float64)))
    assert len(seen) == lay.num_blocks * lay.block_size or len(seen) == int(cap.sum())
    assert np.all(pool.v[~written] == sentinel) and np.all(pool.kr[~kwritten] == sentinel)
    assert not np.any(pool.v[written] == sentinel)


def test_append_error_bits():
    w, lens, lay = _small_paged()
    dims = O.Dims(w.H, w.G, w.d_h, w.d_n, w.d_r)
    pool = O.Pool.empty(w.dtype, lay.v_elems, lay.kr_elems,
                        (lay.v_sb, lay.v_st, lay.v_sg, lay.kr_sb, lay.kr_st),
                        lay.num_blocks, lay.block_size, lay.block_table)
    tab = O.rope_table(16, w.d_r)
    v = np.ones((1, w.G, w.d_h), np.float32)
    kr = np.ones((1, w.d_r), np.float32)
    assert O.append(pool, dims, [w.B], [0], v, kr, tab) == O.ERR_SEQ
    assert O.append(pool, dims, [0], [-1], v, kr, tab) == O.ERR_LENGTH
    cap = lay.max_blocks * lay.block_size
    assert O.append(pool, dims, [0], [cap], v, kr, tab) == O.ERR_CAPACITY
    # a position inside the table's capacity but beyond the RoPE table
    b0 = int(np.argmax((lay.block_table >= 0).sum(axis=1)))
    assert O.append(pool, dims, [b0], [cap - 1], v, kr, O.rope_table(cap - 1, w.d_r)) == O.ERR_ROPE
    # an unused table slot (-1) is a bad block
    b = int(np.argmin(lens))
    p = (lay.block_table[b] >= 0).sum() * lay.block_size
    if p < cap:
        assert O.append(pool, dims, [b], [p], v, kr, O.rope_table(cap + 1, w.d_r)) == O.ERR_BLOCK
    assert np.all(pool.v == 0)


# ----------------------------------------------------------------------------------------
# Prefill against a causal library attention
# ----------------------------------------------------------------------------------------


def test_prefill_against_sdpa_with_causal_mask():
    w = synth.workload("C5", B=2, T=11, H=4, G=2, d_h=8, d_n=8, d_r=4, chunk=6, block_size=4,
                       append_one=False)
    dims = O.Dims(w.H, w.G, w.d_h, w.d_n, w.d_r)
    lens = synth.lengths(w)
    lay = synth.layout(w, lens)
    pool = O.Pool.empty(w.dtype, lay.v_elems, lay.kr_elems,
                        (lay.v_sb, lay.v_st, lay.v_sg, lay.kr_sb, lay.kr_st),
                        lay.num_blocks, lay.block_size, lay.block_table)
    tab = O.rope_table(64, w.d_r)
    M = synth.weights(w).astype(np.float64)
    C = w.chunk
    q_nope, q_rope = synth.queries(w, w.B * C)
    q_pos = np.concatenate([np.arange(w.T, w.T + C)] * w.B)
    qt, r = O.absorb(q_nope, q_rope, q_pos, M, tab)
    q_abs = O.q_abs_of(qt, r).reshape(w.B, C, w.H, -1)
    v_new = np.zeros((w.B, C, w.G, w.d_h), np.float32)
    kr_new = np.zeros((w.B, C, w.d_r), np.float32)
    for b in range(w.B):
        v, kr_raw = synth.sequence_tokens(w, b, w.T + C)
        O.append(pool, dims, np.full(w.T, b), np.arange(w.T), v[: w.T], kr_raw[: w.T], tab)
        v_new[b], kr_new[b] = v[w.T:], kr_raw[w.T:]
    out, lse, err = O.prefill(pool, dims, [w.T] * w.B, C, q_abs, v_new, kr_new, w.scale, tab)
    assert err == 0
    n = w.T + C
    mask = torch.zeros(C, n, dtype=torch.bool)
    for i in range(C):
        mask[i, : w.T + i + 1] = True
    for b in range(w.B):
        V, kr = O.gather(pool, dims, b, n)
        ref = _sdpa_reference(V, kr, q_nope.reshape(w.B, C, w.H, -1)[b].transpose(1, 0, 2),
                              r.reshape(w.B, C, w.H, -1)[b].transpose(1, 0, 2), M, dims, w.scale,
                              mask=mask)
        assert np.max(np.abs(out[b].transpose(1, 0, 2) - ref)) < 1e-12


def test_synthetic_m_scale_is_matched():
    """Scale-matched M: with unit query and value variance the keys K = V M have RMS near 1
    (the initialisation formula in the review's section 关键技巧三); a sanity check."""
    w = synth.workload("C3")
    M = synth.weights(w)[:4].astype(np.float64)
    v, _ = synth.sequence_tokens(w, 0, 4096)
    K = np.einsum("ti,hik->htk", v[:, 0, :].astype(np.float64), M)
    assert abs(np.sqrt(np.mean(K ** 2)) - 1.0) < 0.02


# ----------------------------------------------------------------------------------------
# GQA comparator (the cache a matched grouped-query model keeps)
# ----------------------------------------------------------------------------------------


def test_gqa_comparator_worked_example():
    """The [kvcache] section 3 example is itself an MQA step: G = 1 key/value head."""
    g = _golden("kvcache_mqa_worked_example.json")
    K = np.array(g["keys"], dtype=np.float64)[:, None, :]
    V = np.array(g["values"], dtype=np.float64)[:, None, :]
    dims = O.Dims(H=1, G=1, d_h=2, d_n=2, d_r=0)
    for case in g["cases"]:
        o, lse = O.gqa_decode_sequence(K, V, dims, np.array([case["query"]], float), g["scale"])
        assert [round(x, 1) for x in o[0]] == case["output_1dp"]
        e2 = math.exp(2.0)
        assert abs(lse[0] - math.log(e2 + 1)) < 1e-15


@pytest.mark.parametrize("seed", [0, 1])
def test_gqa_comparator_against_sdpa(seed):
    """A library routine: scaled_dot_product_attention in float64 with the group's key and value
    repeated for each of its heads."""
    rng = np.random.default_rng(seed)
    H, G, n, d_h = 8, 2, 37, 16
    K = rng.standard_normal((n, G, d_h))
    V = rng.standard_normal((n, G, d_h))
    q = rng.standard_normal((H, d_h))
    dims = O.Dims(H=H, G=G, d_h=d_h, d_n=d_h, d_r=0)
    out, lse = O.gqa_decode_sequence(K, V, dims, q, 0.3)
    per = H // G
    Kh = torch.from_numpy(np.repeat(K.transpose(1, 0, 2), per, axis=0))   # [H, n, d_h]
    Vh = torch.from_numpy(np.repeat(V.transpose(1, 0, 2), per, axis=0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], Kh, Vh, scale=0.3)[:, 0, :].numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-12)
    s = 0.3 * np.einsum("hd,hnd->hn", q, Kh.numpy())
    assert np.allclose(lse, np.log(np.exp(s).sum(-1)), rtol=0, atol=1e-12)


def test_gqa_with_keys_equal_values_is_gva_with_identity_map():
    """Shared K = V ([review] 第一次尝试) is both a GQA cache with K = V and a GVA cache with
    M_h = I and no positional slice: the two decode definitions must agree."""
    rng = np.random.default_rng(4)
    H, G, n, d = 6, 3, 23, 8
    V = rng.standard_normal((n, G, d))
    q = rng.standard_normal((H, d))
    dims = O.Dims(H=H, G=G, d_h=d, d_n=d, d_r=0)
    a, la = O.gqa_decode_sequence(V, V, dims, q, 0.5)
    b, lb = O.decode_sequence(V, np.zeros((n, 0)), dims, q, 0.5)
    assert np.allclose(a, b, rtol=0, atol=1e-13) and np.allclose(la, lb, rtol=0, atol=1e-13)


def test_gqa_bytes_against_kvcache_page():
    """The per-token byte count a GQA step reads is the [kvcache] section 5 figure: 8 KV heads
    of 128 fp16 values, keys and values, 4 KiB per token per layer for MHA-8 (= GQA with G = 8)."""
    assert O.gqa_decode_bytes(1, 8, 128, 2) == 4096
    assert O.gqa_decode_bytes(1, 1, 128, 2) == 512
    # the GVA step at the ragged-batch shape reads 2096 B per token, 51.2% of GQA's 4096 B
    assert O.gva_decode_bytes(1, 8, 128, 24, 2) == 2096


# ----------------------------------------------------------------------------------------
# Non-absorbable variant: ordinary RoPE on the reconstructed key
# ----------------------------------------------------------------------------------------


def test_recon_decode_closed_form_two_tokens():
    """Worked by hand. d_h = 1, d_n = 2 (one pair, theta_0 = 1), two cached values v = (1, 2)
    at positions 0 and 1, the query q = (1, 0) at p = 1, scale 1.
    With M = [1, 0] the key is k_j = v_j (cos j, sin j) and s_j = v_j cos(j - 1); with
    M = [0, 1] it is v_j (-sin j, cos j) and s_j = v_j sin(1 - j)."""
    dims = O.Dims(H=1, G=1, d_h=1, d_n=2, d_r=0)
    V = np.array([[[1.0]], [[2.0]]])
    q = np.array([[1.0, 0.0]])
    for M, s in (([1.0, 0.0], (math.cos(1.0), 2.0)), ([0.0, 1.0], (math.sin(1.0), 0.0))):
        out, lse = O.recon_decode_sequence(V, dims, q, 1, np.array([[M]]), 1.0)
        e0, e1 = math.exp(s[0]), math.exp(s[1])
        assert abs(out[0, 0] - (e0 * 1.0 + e1 * 2.0) / (e0 + e1)) < 1e-15
        assert abs(lse[0] - math.log(e0 + e1)) < 1e-15


@pytest.mark.parametrize("seed", [0, 1])
def test_recon_decode_against_complex_relative_angles(seed):
    """An independent definition: the key k = M_h^T v (einsum over the named index), pairs as
    complex numbers, and the score Re(sum_i conj(q_i) k_i e^{i (j - p) theta_i}), which is what
    rotating the key by j and the query by p gives. d_h != d_n, so a transposed map fails."""
    rng = np.random.default_rng(seed)
    H, G, n, d_h, d_n, p, base, scale = 4, 2, 19, 6, 8, 25, 10000.0, 0.4
    V = rng.standard_normal((n, G, d_h))
    M = rng.standard_normal((H, d_h, d_n))
    q = rng.standard_normal((H, d_n))
    dims = O.Dims(H=H, G=G, d_h=d_h, d_n=d_n, d_r=0)
    out, lse = O.recon_decode_sequence(V, dims, q, p, M, scale, base)
    theta = np.array([math.pow(base, -2.0 * i / d_n) for i in range(d_n // 2)])
    for h in range(H):
        g = h // (H // G)
        k = np.einsum("ni,ik->nk", V[:, g, :], M[h])
        kc = k[:, 0::2] + 1j * k[:, 1::2]
        qc = q[h, 0::2] + 1j * q[h, 1::2]
        rel = np.exp(1j * (np.arange(n)[:, None] - p) * theta[None, :])
        s = scale * np.real((np.conj(qc)[None, :] * kc * rel).sum(-1))
        ls = logsumexp(s)
        assert abs(lse[h] - ls) < 1e-12
        assert np.allclose(out[h], np.exp(s - ls) @ V[:, g, :], rtol=0, atol=1e-12)


def test_recon_decode_depends_only_on_relative_position():
    """RoPE on both sides makes the score a function of p - j: moving the query and every key
    by the same offset changes nothing (a rotation dropped on either side breaks this)."""
    rng = np.random.default_rng(7)
    H, G, n, d_h, d_n = 4, 2, 11, 8, 8
    V = rng.standard_normal((n, G, d_h))
    M = rng.standard_normal((H, d_h, d_n))
    q = rng.standard_normal((H, d_n))
    dims = O.Dims(H=H, G=G, d_h=d_h, d_n=d_n, d_r=0)
    a, la = O.recon_decode_sequence(V, dims, q, n, M, 0.3)
    b, lb = O.recon_decode_sequence(V, dims, q, n + 1000, M, 0.3, key_pos=np.arange(n) + 1000)
    assert np.allclose(a, b, rtol=0, atol=1e-10) and np.allclose(la, lb, rtol=0, atol=1e-10)
    # and moving only the query does change the result
    c, _ = O.recon_decode_sequence(V, dims, q, n + 3, M, 0.3)
    assert not np.allclose(a, c, rtol=0, atol=1e-6)


def test_recon_decode_empty_and_flops():
    dims = O.Dims(H=2, G=1, d_h=4, d_n=4, d_r=0)
    out, lse = O.recon_decode_sequence(np.zeros((0, 1, 4)), dims, np.ones((2, 4)), 0,
                                       np.ones((2, 4, 4)), 1.0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    # per token and head: a d_h x d_n rebuild, a d_n score and a d_h weighted sum
    assert O.recon_decode_flops(3, 2, 4, 6) == 2 * 3 * (2 * 4 * 6 + 2 * 6 + 2 * 4)


# ----------------------------------------------------------------------------------------
# MLA-style latent comparator
# ----------------------------------------------------------------------------------------


@pytest.mark.parametrize("seed", [0, 1])
def test_mla_absorbed_decode_equals_textbook(seed):
    """The textbook MLA step (keys and values projected up from the cached latents per head) equals
    the absorbed decode with one group whose value is the latent (q~_h = W^UK_h q_nope_h),
    followed by the value up-projection. d_c, d_k and d_v all differ, so a transposed
    projection fails."""
    rng = np.random.default_rng(seed)
    H, n, d_c, d_k, d_v, d_r, scale = 6, 29, 12, 8, 10, 4, 0.3
    C = rng.standard_normal((n, d_c))
    kr = rng.standard_normal((n, d_r))
    q_nope = rng.standard_normal((H, d_k))
    r = rng.standard_normal((H, d_r))
    W_uk = rng.standard_normal((H, d_c, d_k))
    W_uv = rng.standard_normal((H, d_c, d_v))
    out, lse = O.mla_decode_materialized(C, kr, q_nope, r, W_uk, W_uv, scale)
    dims = O.Dims(H=H, G=1, d_h=d_c, d_n=d_k, d_r=d_r)
    q_abs = np.concatenate([np.einsum("hck,hk->hc", W_uk, q_nope), r], axis=1)
    lat, lse_a = O.decode_sequence(C[:, None, :], kr, dims, q_abs, scale)
    assert np.allclose(np.einsum("hc,hcv->hv", lat, W_uv), out, rtol=0, atol=1e-12)
    assert np.allclose(lse_a, lse, rtol=0, atol=1e-12)
    # and against torch's attention on the up-projected keys and values
    Kh = torch.from_numpy(np.einsum("nc,hck->hnk", C, W_uk))
    Vh = torch.from_numpy(np.einsum("nc,hcv->hnv", C, W_uv))
    qh = torch.from_numpy(q_nope)[:, None, :]
    s = scale * (torch.einsum("hqk,hnk->hqn", qh, Kh) + torch.from_numpy(r @ kr.T)[:, None, :])
    ref = (torch.softmax(s, dim=-1) @ Vh)[:, 0, :].numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def test_mla_cache_ledger_against_pages():
    """[review] section 问题: MLA caches T (d_c + d_r) scalars; with the DeepSeek-V2 latent of
    [mla] section 3.1 (d_c = 512) and a 64-wide shared RoPE channel that is 576 per token, and
    the latent alone replaces h (d_k + d_v) = 128 x 256 = 32768 per token."""
    assert O.mla_cache_scalars(1, 512, 64) == 576
    assert O.mla_cache_scalars(1000, 512, 0) * 64 == 1000 * 128 * (128 + 128)
    # beside the matched GVA cache of the ragged-batch shape (G = 8, d_h = 128, d_r = 24)
    assert O.mla_cache_scalars(1, 512, 64) / O.gva_cache_scalars(1, 8, 128, 24) < 0.55


# ----------------------------------------------------------------------------------------
# The GVA path's positional term, end to end through append -> absorb -> decode_sequence
# ([review] section 关键技巧二: the shared key is cached rotated at its own position j, the
# query's slice is rotated at the query position p, so their product depends on j - p only)
# ----------------------------------------------------------------------------------------


def _f32_pool_pipeline(V, kr_raw, q_nope, q_rope, M, dims, scale, key_pos, q_pos):
    """Appends the n keys at positions key_pos (one contiguous float32 sequence), absorbs the
    query at q_pos and decodes over those keys. Returns (out, lse, kr as cached, r)."""
    n = len(V)
    top = int(max(int(np.max(key_pos)), q_pos)) + 1
    bs = 1 << int(math.ceil(math.log2(top)))
    pool = O.Pool.empty("f32", bs * dims.G * dims.d_h, bs * dims.d_r,
                        (bs * dims.G * dims.d_h, dims.G * dims.d_h, dims.d_h, bs * dims.d_r,
                         dims.d_r), 1, bs, np.zeros((1, 1), np.int64))
    tab = O.rope_table(top, dims.d_r)
    assert O.append(pool, dims, np.zeros(n, np.int64), key_pos, V, kr_raw, tab) == 0
    Vg, krg = O.gather(pool, dims, 0, top)
    Vg, krg = Vg[key_pos], krg[key_pos]
    qt, r = O.absorb(q_nope[None], q_rope[None], [q_pos], M, tab)
    out, lse = O.decode_sequence(Vg, krg, dims, O.q_abs_of(qt, r)[0], scale)
    return out, lse, krg, r[0]


def _positional_pin_failures():
    """Runs the positional-term pins of the GVA path and returns the names of those that fail
    (an empty list when the oracle is right). Tolerances: the float32 cache rounds each rotated
    key element once (relative 2^-24), which moves a score by at most
    scale * sum_i |r_i| |kr_i| 2^-24 < 1e-5 at these sizes; everything else is float64."""
    fails = []
    rng = np.random.default_rng(41)
    H, G, n, d_h, d_n, d_r, scale = 4, 2, 23, 6, 5, 8, 0.5
    dims = O.Dims(H=H, G=G, d_h=d_h, d_n=d_n, d_r=d_r)
    V = rng.standard_normal((n, G, d_h)).astype(np.float32)
    kr_raw = (3.0 * rng.standard_normal((n, d_r))).astype(np.float32)
    q_nope = rng.standard_normal((H, d_n)).astype(np.float32)
    q_rope = (3.0 * rng.standard_normal((H, d_r))).astype(np.float32)
    M = rng.standard_normal((H, d_h, d_n)) / math.sqrt(d_h)
    p, delta = 40, 977
    j = np.arange(n)
    a_out, a_lse, kr_a, r_a = _f32_pool_pipeline(V, kr_raw, q_nope, q_rope, M, dims, scale, j, p)
    # 1. shifting the query and every key by the same offset changes nothing
    b_out, b_lse, _, _ = _f32_pool_pipeline(V, kr_raw, q_nope, q_rope, M, dims, scale,
                                            j + delta, p + delta)
    if not (np.max(np.abs(a_out - b_out)) < 1e-5 and np.max(np.abs(a_lse - b_lse)) < 1e-5):
        fails.append("shift invariance")
    # 2. moving only the query does change the result
    c_out, c_lse, _, _ = _f32_pool_pipeline(V, kr_raw, q_nope, q_rope, M, dims, scale, j, p + 3)
    if not np.max(np.abs(c_lse - a_lse)) > 1e-3:
        fails.append("query position matters")
    # 3. each positional product r_h . kr_j equals Re(sum_i conj(q_i) k_i e^{i (j - p) theta_i})
    #    of the raw pairs taken as complex numbers (theta_i from math.pow, not the oracle)
    theta = np.array([math.pow(10000.0, -2.0 * i / d_r) for i in range(d_r // 2)])
    kc = kr_raw[:, 0::2].astype(np.float64) + 1j * kr_raw[:, 1::2].astype(np.float64)
    qc = q_rope[:, 0::2].astype(np.float64) + 1j * q_rope[:, 1::2].astype(np.float64)
    rel = np.exp(1j * (j[:, None] - p) * theta[None, :])                      # [n, d_r/2]
    want = np.real(np.einsum("hi,ni,ni->hn", np.conj(qc), kc, rel))          # [H, n]
    got = r_a @ kr_a.T
    if not np.max(np.abs(got - want)) < 1e-5 * max(1.0, np.max(np.abs(want))):
        fails.append("complex relative angle")
    # 4. the full score and softmax against the materialised form with that positional term
    for h in range(H):
        g = h // (H // G)
        K = V[:, g, :].astype(np.float64) @ M[h]
        s = scale * (K @ q_nope[h].astype(np.float64) + want[h])
        ls = logsumexp(s)
        if not (abs(a_lse[h] - ls) < 1e-5 and
                np.max(np.abs(a_out[h] - np.exp(s - ls) @ V[:, g, :].astype(np.float64))) < 1e-5):
            fails.append(f"score of head {h}")
            break
    return fails


def test_gva_positional_term_pins():
    assert _positional_pin_failures() == []


def _rotate_sine_flipped(x, cs):
    """A planted mistake: the rotation with the sine's sign flipped (a rotation by -angle)."""
    x = np.asarray(x, dtype=np.float64)
    c, s = cs[..., 0], cs[..., 1]
    y = np.empty(np.broadcast(x[..., 0::2], c).shape[:-1] + (x.shape[-1],))
    y[..., 0::2] = x[..., 0::2] * c + x[..., 1::2] * s
    y[..., 1::2] = -x[..., 0::2] * s + x[..., 1::2] * c
    return y


@pytest.mark.parametrize("mistake", ["query_unrotated", "query_at_p_minus_1", "sine_flipped"])
def test_planted_positional_mistakes_fail_a_pin(mistake, monkeypatch):
    """Each plausible mistake in the oracle's positional path, planted in the oracle on the CPU,
    fails at least one of the pins above."""
    real_absorb = O.absorb
    if mistake == "query_unrotated":
        def bad(q_nope, q_rope, q_pos, M, table):
            qt, _ = real_absorb(q_nope, q_rope, q_pos, M, table)
            return qt, np.asarray(q_rope, dtype=np.float64)
        monkeypatch.setattr(O, "absorb", bad)
    elif mistake == "query_at_p_minus_1":
        def bad(q_nope, q_rope, q_pos, M, table):
            return real_absorb(q_nope, q_rope, np.asarray(q_pos) - 1, M, table)
        monkeypatch.setattr(O, "absorb", bad)
    else:
        monkeypatch.setattr(O, "rotate", _rotate_sine_flipped)
    assert _positional_pin_failures() != []


# ----------------------------------------------------------------------------------------
# decode(): every sequence of a paged pool, against pure-Python loops over the raw pool
# ----------------------------------------------------------------------------------------


def _brute_force_pool_decode(pool, dims, seq_len, q_abs, scale, group_of):
    """Reads the pool's float32 bits element by element through the block table and decodes
    each (b, h) with Python loops; group_of(h) names the head's value group."""
    B = len(seq_len)
    out = np.zeros((B, dims.H, dims.d_h))
    lse = np.full((B, dims.H), -np.inf)
    f32 = lambda bits: float(np.array(bits, dtype=np.uint32).view(np.float32))
    for b in range(B):
        n = int(seq_len[b])
        rows_v, rows_k = [], []
        for p in range(n):
            blk = int(pool.block_table[b][p // pool.block_size])
            off = p % pool.block_size
            rows_v.append([[f32(pool.v[blk * pool.v_sb + off * pool.v_st + g * pool.v_sg + i])
                            for i in range(dims.d_h)] for g in range(dims.G)])
            rows_k.append([f32(pool.kr[blk * pool.kr_sb + off * pool.kr_st + i])
                           for i in range(dims.d_r)])
        for h in range(dims.H):
            if n == 0:
                continue
            g = group_of(h)
            qt = q_abs[b][h][:dims.d_h]
            r = q_abs[b][h][dims.d_h:]
            s = [scale * (sum(qt[i] * rows_v[p][g][i] for i in range(dims.d_h)) +
                          sum(r[i] * rows_k[p][i] for i in range(dims.d_r))) for p in range(n)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = sum(e)
            lse[b, h] = mx + math.log(z)
            for i in range(dims.d_h):
                out[b, h, i] = sum(e[p] / z * rows_v[p][g][i] for p in range(n))
    return out, lse


def test_pool_decode_against_brute_force():
    w, lens, lay = _small_paged(dtype="f32")
    dims = O.Dims(w.H, w.G, w.d_h, w.d_n, w.d_r)
    pool = O.Pool.empty("f32", lay.v_elems, lay.kr_elems,
                        (lay.v_sb, lay.v_st, lay.v_sg, lay.kr_sb, lay.kr_st),
                        lay.num_blocks, lay.block_size, lay.block_table)
    tab = O.rope_table(64, w.d_r)
    for b in range(w.B):
        v, kr_raw = synth.sequence_tokens(w, b, int(lens[b]))
        assert O.append(pool, dims, np.full(int(lens[b]), b), np.arange(int(lens[b])), v,
                        kr_raw, tab) == 0
    seq_len = lens.copy()
    seq_len[1] = 0                                   # an empty history
    q_abs = np.random.default_rng(3).standard_normal((w.B, w.H, w.d_h + w.d_r))
    out, lse = O.decode(pool, dims, seq_len, q_abs, 0.6)
    ref, ref_lse = _brute_force_pool_decode(pool, dims, seq_len, q_abs, 0.6,
                                            lambda h: h // (w.H // w.G))
    assert np.max(np.abs(out - ref)) < 1e-12 and np.all(out[1] == 0)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse)) and np.max(np.abs(lse[fin] - ref_lse[fin])) < 1e-12


def test_pool_decode_with_a_permuted_group_map():
    """With a non-contiguous head -> group map every head reads the values of its own group:
    decode() equals the brute force that looks the group up in the same map, and differs from the
    contiguous map's result."""
    w, lens, lay = _small_paged(dtype="f32")
    gmap = (1, 0, 0, 1)                              # H = 4, G = 2: two heads per group
    dims = O.Dims(w.H, w.G, w.d_h, w.d_n, w.d_r, gmap)
    pool = O.Pool.empty("f32", lay.v_elems, lay.kr_elems,
                        (lay.v_sb, lay.v_st, lay.v_sg, lay.kr_sb, lay.kr_st),
                        lay.num_blocks, lay.block_size, lay.block_table)
    tab = O.rope_table(64, w.d_r)
    for b in range(w.B):
        v, kr_raw = synth.sequence_tokens(w, b, int(lens[b]))
        O.append(pool, dims, np.full(int(lens[b]), b), np.arange(int(lens[b])), v, kr_raw, tab)
    q_abs = np.random.default_rng(4).standard_normal((w.B, w.H, w.d_h + w.d_r))
    out, lse = O.decode(pool, dims, lens, q_abs, 0.6)
    ref, ref_lse = _brute_force_pool_decode(pool, dims, lens, q_abs, 0.6, lambda h: gmap[h])
    assert np.max(np.abs(out - ref)) < 1e-12 and np.max(np.abs(lse - ref_lse)) < 1e-12
    contiguous, _ = O.decode(pool, O.Dims(w.H, w.G, w.d_h, w.d_n, w.d_r), lens, q_abs, 0.6)
    assert np.max(np.abs(contiguous - out)) > 1e-3
    # decode_sequence (used by the parity tests) agrees with decode() under the map
    for b in range(w.B):
        V, kr = O.gather(pool, dims, b, int(lens[b]))
        o2, l2 = O.decode_sequence(V, kr, dims, q_abs[b], 0.6)
        assert np.max(np.abs(o2 - out[b])) < 1e-12
