#!/usr/bin/env python3
"""GVA decode benchmark on one MI355X.

One step is one pass of the decode hot path over one batch of the ragged paged workload:
append one token per sequence (gva_cache_append), absorb its query (gva_absorb_query), split
decode + combine over len_b + 1 cached positions (gva_decode). Inputs are resident in HBM
before the timed region. The value is the cache bytes the step must read, len (G d_h + d_r) s
summed over the batch, divided by the step time.

Also measured: the decode kernel alone (HIP events on the library's stream) for the roofline
line, the GQA comparator (the cache a matched grouped-query model keeps) on the same batch, the
long-context single-sequence decode (T = 131072) with cache replicas rotated so the 256 MB
last-level cache cannot serve them, the chunked prefill, and the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_BF16 = 2.5e15         # MI355X dense bf16 matrix-core flop/s
METRIC = "GVA decode attention cache-read GB/s (% of HBM peak) and seq-steps/s per GPU"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# Untimed work issued before each secondary timed series. At the start of a burst of work the
# GPU's clocks dip and recover over about 10-15 ms (the ragged-batch decode kernel's launches go
# 1.62 -> 1.32 ms in a kernel trace of this bench), so those series start on a settled GPU.
SETTLE_S = 0.03


def kernel_medians(fn, n, torch, call_s):
    """Median device time (us) of each kernel that the last n of a settling burst plus n calls
    of fn launch, from the PyTorch profiler's device activity records (hardware timestamps of
    every kernel the process launches, the library's included). None when another profiler is
    loaded (rocprofv3's tool takes the same hooks), when the profiler cannot record, or when the
    kernels' medians do not add up to within 50% of call_s, the event-timed call."""
    if "rocprofiler" in os.environ.get("LD_PRELOAD", "") or any(
            k.startswith("ROCPROFILER_") for k in os.environ):
        log("kernel durations not recorded: another profiler is loaded")
        return None
    try:
        from torch.profiler import profile, ProfilerActivity
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            settle(fn, torch)
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
        by = {}
        for e in prof.events():
            if e.device_type.name != "CUDA":
                continue
            name = e.name.replace("void (anonymous namespace)::", "").split("(gva::")[0]
            dur = float(getattr(e, "device_time", None) or e.cuda_time)
            by.setdefault(name, []).append((e.time_range.start, dur))
        med = {}
        for k, v in by.items():
            last = [d for _, d in sorted(v)[-n:]]          # the n calls after the burst
            med[k] = round(float(np.median(last)), 2)
        total = sum(med.values())
        if not med or not 0.5 * call_s * 1e6 <= total <= 1.5 * call_s * 1e6:
            log(f"kernel durations not recorded: {med} against a {call_s * 1e6:.1f} us call")
            return None
        return med
    except Exception as exc:  # a profiler that cannot start leaves the measurement out
        log(f"kernel durations not recorded: {exc!r}")
        return None


def settle(fn, torch):
    """Issues about SETTLE_S seconds of calls of fn back to back and does not wait for them, so
    the timed series that follows starts with the GPU still busy. One call, waited for, sizes
    the burst."""
    torch.cuda.synchronize()
    t = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    dt = max(time.perf_counter() - t, 1e-6)
    for _ in range(min(int(SETTLE_S / dt) + 1, 4000)):
        fn()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--kernel", type=int, default=0, help="0 auto, 1 generic, 2 matrix-core")
    p.add_argument("--splits", type=int, default=0)
    p.add_argument("--no-long", action="store_true", help="skip the T=131072 measurement")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill measurement")
    p.add_argument("--no-gqa", action="store_true", help="skip the GQA comparator measurement")
    p.add_argument("--no-small", action="store_true", help="skip the small-batch step latencies")
    p.add_argument("--no-recon", action="store_true",
                   help="skip the non-absorbable comparator measurement")
    p.add_argument("--no-mla", action="store_true",
                   help="skip the MLA-style latent comparator measurement")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the streaming-read ceiling measurement")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    return p.parse_args()


class DeviceCache:
    """A workload's cache on the device, filled through gva_cache_append with seeded data."""

    def __init__(self, w, lens, fill_seed, torch, gb, synth, group_major=True):
        self.w = w
        self.lens = lens
        self.lay = synth.layout(w, lens, group_major)
        cap = synth.capacity(w, lens)
        self.max_pos = int(cap.max()) + 1
        self.dims = gb.GvaDims(w.H, w.G, w.d_h, w.d_n, w.d_r)
        rope = torch.from_numpy(gb.gva_rope_table_fill(self.max_pos, w.d_r, w.base)).cuda()
        self.block_table = torch.from_numpy(self.lay.block_table).cuda()
        lay = self.lay
        self.cache = gb.GvaCache.allocate(self.dims, w.dtype, lay.num_blocks, lay.block_size,
                                          self.block_table, rope,
                                          (lay.v_sb, lay.v_st, lay.v_sg, lay.kr_sb, lay.kr_st))
        # fill positions 0..len_b-1 of every sequence, in batches of tokens
        gen = torch.Generator(device="cuda")
        gen.manual_seed(fill_seed)
        seqs = np.repeat(np.arange(w.B, dtype=np.int32), lens)
        poss = np.concatenate([np.arange(n, dtype=np.int32) for n in lens])
        step = 1 << 16
        for o in range(0, seqs.size, step):
            n = min(step, seqs.size - o)
            v = torch.randn((n, w.G, w.d_h), generator=gen, device="cuda")
            kr = torch.randn((n, w.d_r), generator=gen, device="cuda")
            gb.gva_cache_append(self.dims, self.cache, w.B,
                                torch.from_numpy(seqs[o:o + n]).cuda(),
                                torch.from_numpy(poss[o:o + n]).cuda(), v, kr)
        torch.cuda.synchronize()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the decode path shards "
              "by sequence across GPUs with no exchange, so run one process per GPU.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from value_only_kv_amd import binding as gb
    from value_only_kv_amd import synth

    gb.lib()  # fails loudly when the HIP library is not built
    dev = torch.cuda.get_device_name(0)
    log("device:", dev, "| library:", gb.gva_version())

    # ---------------- ragged paged batch (the headline workload) ----------------
    w = synth.workload("C4")
    lens = synth.lengths(w)
    t_setup = time.time()
    dc = DeviceCache(w, lens, 1234, torch, gb, synth)
    log(f"C4 cache filled: {dc.lay.num_blocks} blocks, {int(lens.sum())} tokens, "
        f"{(dc.cache.v.numel() + dc.cache.kr.numel()) * 2 / 1e9:.2f} GB in {time.time() - t_setup:.1f}s")
    B, H = w.B, w.H
    row = w.d_h + w.d_r
    max_len = int(lens.max()) + 1
    seq = torch.arange(B, dtype=torch.int32, device="cuda")
    pos = torch.from_numpy(lens.astype(np.int32)).cuda()          # the appended token's position
    seq_len = pos + 1
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    v_new = torch.randn((B, w.G, w.d_h), generator=gen, device="cuda")
    kr_new = torch.randn((B, w.d_r), generator=gen, device="cuda")
    q_nope = torch.randn((B, H, w.d_n), generator=gen, device="cuda")
    q_rope = torch.randn((B, H, w.d_r), generator=gen, device="cuda")
    M = torch.randn((H, w.d_h, w.d_n), generator=gen, device="cuda") * w.m_sigma
    q_abs = torch.empty((B, H, row), device="cuda")
    out = torch.empty((B, H, w.d_h), device="cuda")
    lse = torch.empty((B, H), device="cuda")
    S = gb.gva_decode_num_splits(dc.dims, B, max_len, args.splits)
    R = gb.gva_decode_num_ranges(dc.dims, B, max_len) if args.splits == 0 and args.kernel != 1 else 0
    plan = (f"balanced: {R} equal tile ranges over all sequences" if R > 0
            else f"split: {S} chunks per sequence")
    wsb = gb.gva_decode_workspace_bytes(dc.dims, B, max_len, args.splits)
    ws = torch.zeros(max(wsb, 256) // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        # append + absorb (one launch), then the decode
        gb.gva_decode_step(dc.dims, dc.cache, B, pos, v_new, kr_new, q_nope, q_rope, M, seq_len,
                           max_len, w.scale, q_abs, out, lse, num_splits=args.splits,
                           kernel=args.kernel, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    assert torch.isfinite(out).all().item(), "non-finite decode output"
    assert int(dc.cache.err_flag.item()) == 0, "device error flag raised"

    elem = 2
    tok_bytes = (w.G * w.d_h + w.d_r) * elem
    read_bytes = int((lens + 1).sum()) * tok_bytes                 # algorithmic, per step
    value = read_bytes / t_step / 1e9
    log(f"C4 step: {t_step * 1e3:.3f} ms, {value:.1f} GB/s, {plan}")

    # decode launches alone, timed with HIP events on the launch stream after a settling burst
    def dec_call():
        gb.gva_decode(dc.dims, dc.cache, B, seq_len, max_len, q_abs, w.scale, out, lse,
                      num_splits=args.splits, kernel=args.kernel, workspace=ws, stream=stream)

    settle(dec_call, torch)
    n_ev = max(args.steps, 100)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_ev)]
    for e0, e1 in ev:
        e0.record(stream)
        gb.gva_decode(dc.dims, dc.cache, B, seq_len, max_len, q_abs, w.scale, out, lse,
                      num_splits=args.splits, kernel=args.kernel, workspace=ws, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    t_ev = np.array([e0.elapsed_time(e1) for e0, e1 in ev]) / 1e3
    t_dec = float(t_ev.mean())
    p10, p50, p90 = (float(x) for x in np.percentile(t_ev, [10, 50, 90]))
    dec_gbs = read_bytes / t_dec / 1e9
    log(f"C4 decode (split decode + combine): mean {t_dec * 1e3:.3f} ms (p10 {p10 * 1e3:.3f}, "
        f"median {p50 * 1e3:.3f}, p90 {p90 * 1e3:.3f}), {dec_gbs:.1f} GB/s")
    # the same calls' kernels one by one (the call above adds the combine's launch)
    dec_kernels = kernel_medians(dec_call, 20, torch, t_dec)
    log(f"C4 decode kernels (median us): {dec_kernels}")
    # HBM bytes per call from the committed counter runs, when they were taken on these sources
    # and this configuration
    traffic = None
    if args.kernel == 0 and args.splits == 0:
        from value_only_kv_amd.profile_summary import read_traffic
        traffic = read_traffic(os.path.join(ROOT, "profiles", "gva_decode_ragged_batch_hbm_traffic.md"),
                               read_bytes)

    # ---------------- GQA comparator on the same batch ----------------
    # The cache a matched grouped-query model keeps: the same value pool plus a key pool of the
    # same layout (G keys per token instead of one shared positional key), decoded by the same
    # kernel skeleton, plan and combine; its own cache bytes are 2 G d_h per token.
    gqa = None
    if not args.no_gqa:
        keys = torch.randn(dc.cache.v.shape, generator=gen, device="cuda").to(torch.bfloat16)
        q_g = torch.randn((B, H, w.d_h), generator=gen, device="cuda")
        settle(lambda: gb.gva_gqa_decode(dc.dims, dc.cache, keys, B, seq_len, max_len, q_g, w.scale,
                                         out, lse, workspace=ws, stream=stream), torch)
        evg = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_ev)]
        for e0, e1 in evg:
            e0.record(stream)
            gb.gva_gqa_decode(dc.dims, dc.cache, keys, B, seq_len, max_len, q_g, w.scale, out, lse,
                              workspace=ws, stream=stream)
            e1.record(stream)
        torch.cuda.synchronize()
        t_gqa = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evg])) / 1e3
        gqa_bytes = int((lens + 1).sum()) * 2 * w.G * w.d_h * 2
        gqa = {"workload": "same batch, lengths and paged layout; keys [T][G][d_h] bf16 in place "
                           "of the shared positional key",
               "ms": round(t_gqa * 1e3, 4), "cache_bytes": gqa_bytes,
               "GB_s": round(gqa_bytes / t_gqa / 1e9, 1),
               "frac_of_hbm_peak": round(gqa_bytes / t_gqa / 1e9 / HBM_PEAK_GBS, 4),
               "seq_steps_per_s": round(B / t_gqa, 1),
               "gva_bytes_over_gqa_bytes": round(read_bytes / gqa_bytes, 4),
               "gva_speedup_over_gqa": round(t_gqa / t_dec, 3)}
        log(f"GQA comparator decode: {t_gqa * 1e3:.3f} ms ({gqa_bytes / t_gqa / 1e9:.1f} GB/s of its "
            f"{gqa_bytes / 1e9:.2f} GB); GVA decode is {t_gqa / t_dec:.2f}x faster")
        del keys
        torch.cuda.empty_cache()

    # ---------------- non-absorbable comparator on the same batch ----------------
    # The scale-matched row's decode: the same value pool (its positional-key pool is not read),
    # every head's content keys rebuilt from the values and rotated at their positions at every
    # step, with the maps in bf16. Its cost is the key rebuild, H d_h d_n multiply-adds per token.
    recon = None
    if not args.no_recon:
        q_r, _, mt_bits = synth.recon_inputs(w)
        q_r_t = torch.from_numpy(q_r).cuda()
        mt_t = torch.from_numpy(mt_bits.view(np.int16)).cuda()
        max_pos_r = max_len + 1
        rope_r = torch.from_numpy(gb.gva_rope_table_fill(max_pos_r, w.d_n, w.base)).cuda()
        wsb_r = gb.gva_recon_decode_workspace_bytes(dc.dims, B, max_len, 0)
        ws_r = torch.zeros(max(wsb_r, 256) // 4, dtype=torch.float32, device="cuda")
        scale_r = 1.0 / float(np.sqrt(w.d_n))

        def recon_call():
            gb.gva_recon_decode(dc.dims, dc.cache, B, seq_len, max_len, q_r_t, pos, mt_t, rope_r,
                                max_pos_r, scale_r, out, lse, workspace=ws_r, stream=stream)

        settle(recon_call, torch)
        evr = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(20)]
        for e0, e1 in evr:
            e0.record(stream)
            recon_call()
            e1.record(stream)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all().item(), "non-finite comparator output"
        assert int(dc.cache.err_flag.item()) == 0, "device error flag raised"
        t_rec = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evr])) / 1e3
        toks = int((lens + 1).sum())
        v_bytes = toks * w.G * w.d_h * elem
        rebuild = 2 * H * toks * w.d_h * w.d_n
        recon = {"workload": "same batch, lengths and paged value pool (positional-key pool not "
                             "read); maps M [H][d_h][d_n] in bf16; query at the appended position",
                 "ms": round(t_rec * 1e3, 4), "value_bytes": v_bytes,
                 "GB_s": round(v_bytes / t_rec / 1e9, 1),
                 "key_rebuild_flop": rebuild,
                 "key_rebuild_TFLOP_s": round(rebuild / t_rec / 1e12, 1),
                 "key_rebuild_frac_of_bf16_dense_peak": round(rebuild / t_rec / MFMA_PEAK_BF16, 4),
                 "gva_speedup_over_recon": round(t_rec / t_dec, 3)}
        log(f"non-absorbable comparator decode: {t_rec * 1e3:.3f} ms ({rebuild / t_rec / 1e12:.1f} "
            f"TFLOP/s of key rebuild); the absorbed GVA decode is {t_rec / t_dec:.2f}x faster")
        del rope_r, mt_t, q_r_t, ws_r
        torch.cuda.empty_cache()

    # ---------------- MLA-style latent comparator on the same lengths ----------------
    # A latent cache of d_c = 512 (the DeepSeek-V2 latent width) plus a 64-wide shared RoPE key,
    # 576 scalars per token against GVA's 1048, for the same 256 sequences of len_b + 1 tokens
    # and 32 heads, decoded absorbed (the latent output before the value up-projection). The
    # pool is filled through gva_cache_append, each latent row as two token-major groups of 256.
    mla = None
    if not args.no_mla:
        d_c, d_r_m = 512, 64
        wm = synth.workload("C4", G=d_c // 256, d_h=256, d_n=256, d_r=d_r_m)
        dm = DeviceCache(wm, lens + 1, 4321, torch, gb, synth, group_major=False)
        mdims = gb.GvaDims(H, 1, d_c, d_c, d_r_m)
        q_m = torch.randn((B, H, d_c + d_r_m), generator=gen, device="cuda")
        out_m = torch.empty((B, H, d_c), device="cuda")
        lse_m = torch.empty((B, H), device="cuda")
        wsb_m = gb.gva_mla_decode_workspace_bytes(mdims, B, max_len, 0)
        ws_m = torch.zeros(max(wsb_m, 256) // 4, dtype=torch.float32, device="cuda")
        scale_m = 1.0 / float(np.sqrt(d_c + d_r_m))

        def mla_call():
            gb.gva_mla_decode(mdims, dm.cache, B, seq_len, max_len, q_m, scale_m, out_m, lse_m,
                              workspace=ws_m, stream=stream)

        settle(mla_call, torch)
        evm = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(50)]
        for e0, e1 in evm:
            e0.record(stream)
            mla_call()
            e1.record(stream)
        torch.cuda.synchronize()
        assert torch.isfinite(out_m).all().item(), "non-finite latent comparator output"
        assert int(dm.cache.err_flag.item()) == 0, "device error flag raised"
        t_mla = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evm])) / 1e3
        mla_bytes = int((lens + 1).sum()) * (d_c + d_r_m) * elem
        mla = {"workload": "same 256 sequences and lengths (len_b + 1 tokens); latent d_c = 512 "
                           "and shared RoPE key d_r = 64 per token, 32 heads, bf16 paged "
                           "16-token blocks; absorbed queries, output before the value "
                           "up-projection",
               "ms": round(t_mla * 1e3, 4), "cache_bytes": mla_bytes,
               "GB_s": round(mla_bytes / t_mla / 1e9, 1),
               "frac_of_hbm_peak": round(mla_bytes / t_mla / 1e9 / HBM_PEAK_GBS, 4),
               "mla_bytes_over_gva_bytes": round(mla_bytes / read_bytes, 4),
               "mla_time_over_gva_time": round(t_mla / t_dec, 3),
               # what its bytes alone would take: at the data-sheet peak, and at the GVA
               # decode's own measured rate (the rate the MLA kernel would need to match)
               "mla_floor_ms_at_hbm_peak": round(mla_bytes / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
               "mla_ms_at_gva_rate": round(mla_bytes / (read_bytes / t_dec) * 1e3, 4)}
        log(f"MLA-style latent comparator decode: {t_mla * 1e3:.3f} ms ({mla_bytes / t_mla / 1e9:.1f} "
            f"GB/s of its {mla_bytes / 1e9:.2f} GB); {t_mla / t_dec:.2f}x the GVA decode's time "
            f"for {mla_bytes / read_bytes:.2f}x its bytes")
        del dm, q_m, out_m, ws_m
        torch.cuda.empty_cache()

    result_extra = {}
    # ---------------- long context, one sequence ----------------
    if not args.no_long:
        for d_r, name in ((16, "C3"), (24, "C3r24")):
            wl = synth.workload(name)
            lens_l = synth.lengths(wl)
            reps = [DeviceCache(wl, lens_l, 99 + k, torch, gb, synth) for k in range(3)]
            ml = int(lens_l.max())
            qa = torch.randn((1, wl.H, wl.d_h + wl.d_r), generator=gen, device="cuda")
            sl = torch.from_numpy(lens_l.astype(np.int32)).cuda()
            o1 = torch.empty((1, wl.H, wl.d_h), device="cuda")
            rb = int(lens_l.sum()) * (wl.G * wl.d_h + wl.d_r) * 2
            per_s = {}
            for S_l in (64, 128, 256, 0):
                wsb_l = gb.gva_decode_workspace_bytes(reps[0].dims, 1, ml, S_l)
                ws_l = torch.zeros(max(wsb_l, 256) // 4, dtype=torch.float32, device="cuda")
                rot = [0]

                def long_call():
                    r = reps[rot[0] % 3]
                    rot[0] += 1
                    gb.gva_decode(r.dims, r.cache, 1, sl, ml, qa, wl.scale, o1, None,
                                  num_splits=S_l, kernel=args.kernel, workspace=ws_l, stream=stream)

                settle(long_call, torch)
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(30)]
                for e0, e1 in evs:                       # the rotation goes on from the burst's
                    e0.record(stream)
                    long_call()
                    e1.record(stream)
                torch.cuda.synchronize()
                ts = sorted(e0.elapsed_time(e1) / 1e3 for e0, e1 in evs)
                t_med = ts[len(ts) // 2]
                per_s[str(S_l) if S_l else "auto"] = {"us": round(t_med * 1e6, 2),
                                   "GB_s": round(rb / t_med / 1e9, 1),
                                   "frac_of_hbm_peak": round(rb / t_med / 1e9 / HBM_PEAK_GBS, 4),
                                   "seq_steps_per_s": round(1.0 / t_med, 1)}
                log(f"{name} T={ml} S={S_l or 'auto'}: {t_med * 1e6:.1f} us, {rb / t_med / 1e9:.1f} GB/s")
                if S_l == 0:
                    # the same calls' kernels one by one: the decode kernel's own rate beside
                    # the call's (which adds the combine launch)
                    km = kernel_medians(long_call, 30, torch, t_med)
                    dk = [v for k, v in (km or {}).items() if k.startswith("k_decode_mfma")]
                    per_s["auto"]["kernel_us"] = km
                    if dk:
                        per_s["auto"]["decode_kernel_GB_s"] = round(rb / dk[0] / 1e3, 1)
                        per_s["auto"]["decode_kernel_frac_of_hbm_peak"] = round(
                            rb / dk[0] / 1e3 / HBM_PEAK_GBS, 4)
                        log(f"{name} S=auto kernels: {km}; decode kernel "
                            f"{rb / dk[0] / 1e3:.1f} GB/s")
            result_extra[name] = {"T": ml, "d_r": d_r, "cache_bytes": rb,
                                  "replicas_rotated": 3, "by_splits": per_s}
            del reps
            torch.cuda.empty_cache()

    # ---------------- chunked prefill + decode mix ----------------
    prefill = None
    if not args.no_prefill:
        prefill = bench_prefill(torch, gb, synth, gen, stream)

    # ---------------- small-batch step latency ----------------
    small = None
    if not args.no_small:
        small = bench_small(torch, gb, synth, gen, stream)

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        bcopy = torch.empty_like(a)
        for _ in range(3):
            bcopy.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB write, 3 launches")

    # ---------------- the streaming-read ceiling ----------------
    ceiling = None
    if not args.no_ceiling:
        ceiling = bench_ceiling(torch, gb, stream, read_bytes,
                                long_bytes=272629760)

    # ---------------- CPU oracle on a bounded sample ----------------
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, lens)

    roofline = {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "split decode + combine (gva_decode), ragged paged batch",
                "bytes_per_launch": read_bytes, "launch_ms": round(t_dec * 1e3, 4),
                "traffic_over_algorithmic": (round(traffic / read_bytes, 4) if traffic else None)}
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) values, seeded lengths and block permutation)",
        "config": {"workload": "ragged paged batch decode step: B=256, len_b ~ U[512, 32768], "
                               "append 1 token then decode over len_b+1; H=32, G=8, d_h=d_n=128, "
                               "d_r=24; bf16 cache in 16-token blocks",
                   "global_batch": B, "cached_tokens": int((lens + 1).sum()),
                   "decode_plan": plan, "parallelism": "single GPU"},
        "seq_steps_per_s": round(B / t_step, 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "decode_only": {"ms": round(t_dec * 1e3, 4), "GB_s": round(dec_gbs, 1),
                        "seq_steps_per_s": round(B / t_dec, 1), "launches": n_ev,
                        "ms_p10_p50_p90": [round(p10 * 1e3, 4), round(p50 * 1e3, 4),
                                           round(p90 * 1e3, 4)],
                        "kernel_us": dec_kernels},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "long_context": result_extra,
        "prefill": prefill,
        "small_batch_step": small,
        "gqa_comparator": gqa,
        "recon_comparator": recon,
        "mla_comparator": mla,
        "streaming_ceiling": ceiling,
        "device": dev,
    }
    print(json.dumps(res), flush=True)


def bench_ceiling(torch, gb, stream, big_bytes, long_bytes, iters=10):
    """The rate at which plain 16-byte non-temporal streaming reads leave HBM
    (gva_diag_stream_read, each load instruction reading 1 KiB of consecutive bytes), at the
    ragged batch's cache size (one buffer, far above the 256 MB last-level cache) and at the
    T = 131072 cache size (three buffers rotated, as the long-context decode is timed), over a
    small sweep of grid sizes and loads in flight; and a plain device copy of 1 GiB (read and
    write) for reference. Median of HIP-event times on the launch stream."""
    res = {}
    sink = torch.empty(65536, dtype=torch.int32, device="cuda")

    def timed(fn, n):
        ctr = [0]                  # fn(k) reads buffer k mod the buffer count: the rotation goes
                                   # on from the settling burst into the timed calls

        def nxt():
            fn(ctr[0])
            ctr[0] += 1

        settle(nxt, torch)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for e0, e1 in evs:
            e0.record(stream)
            nxt()
            e1.record(stream)
        torch.cuda.synchronize()
        return sorted(e0.elapsed_time(e1) / 1e3 for e0, e1 in evs)[n // 2]

    for label, nbytes, nbuf in (("ragged_batch_size", big_bytes, 1),
                                ("long_context_size", long_bytes, 3)):
        nb = (nbytes + 255) // 256 * 256
        bufs = [torch.empty(nb // 2, dtype=torch.int16, device="cuda").fill_(k + 1)
                for k in range(nbuf)]
        sweep = {}
        for wg in (1024, 2048, 4096, 8192):
            for f in (2, 4, 8):
                t = timed(lambda k: gb.gva_diag_stream_read(bufs[k % nbuf], nb, wg, f, sink,
                                                            stream=stream), iters)
                sweep[f"{wg}x{f}"] = round(nb / t / 1e9, 1)
        best = max(sweep, key=sweep.get)
        res[label] = {"bytes": nb, "buffers_rotated": nbuf, "best_GB_s": sweep[best],
                      "best_frac_of_hbm_peak": round(sweep[best] / HBM_PEAK_GBS, 4),
                      "best_config": best, "GB_s_by_workgroups_x_loads_in_flight": sweep}
        log(f"streaming ceiling at {nb / 1e9:.3f} GB: {sweep[best]:.1f} GB/s ({best})")
        del bufs
        torch.cuda.empty_cache()
    a = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
    b = torch.empty_like(a)
    t = timed(lambda k: b.copy_(a), iters)
    res["copy_1GiB"] = {"GB_s_read_plus_write": round(2 * a.numel() * 2 / t / 1e9, 1)}
    log(f"1 GiB device copy: {2 * a.numel() * 2 / t / 1e9:.1f} GB/s read + write")
    del a, b
    torch.cuda.empty_cache()
    return res


def bench_prefill(torch, gb, synth, gen, stream, iters=20):
    """Chunked prefill of 512 causal queries over 8192 cached positions for 4 sequences
    (H=32, G=8, d_h=128, d_r=16, 16-token blocks), then one decode step per sequence."""
    w = synth.workload("C5")
    lens = synth.lengths(w)
    dc = DeviceCache(w, lens, 4321, torch, gb, synth)
    B, C, H = w.B, w.chunk, w.H
    row = w.d_h + w.d_r
    start = torch.from_numpy(lens.astype(np.int32)).cuda()
    q = torch.randn((B, C, H, row), generator=gen, device="cuda")
    v_new = torch.randn((B, C, w.G, w.d_h), generator=gen, device="cuda")
    kr_new = torch.randn((B, C, w.d_r), generator=gen, device="cuda")
    out = torch.empty((B, C, H, w.d_h), device="cuda")
    lse = torch.empty((B, C, H), device="cuda")
    ms = int(lens.max())

    def run():
        gb.gva_prefill_chunk(dc.dims, dc.cache, B, start, ms, C, q, v_new, kr_new, w.scale, out,
                             lse, stream=stream)

    settle(run, torch)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for e0, e1 in evs:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) / 1e3 for e0, e1 in evs)[iters // 2]
    n_pairs = sum(int(lens[b]) * C + C * (C + 1) // 2 for b in range(B))
    flop = n_pairs * H * (2 * (w.d_h + w.d_r) + 2 * w.d_h)
    tflops = flop / t / 1e12
    # the decode step that follows (gva_decode_step): append one token at start + C, absorb its
    # query, decode over start + C + 1
    pos = start + C
    sl = pos + 1
    v1 = torch.randn((B, w.G, w.d_h), generator=gen, device="cuda")
    k1 = torch.randn((B, w.d_r), generator=gen, device="cuda")
    qn1 = torch.randn((B, H, w.d_n), generator=gen, device="cuda")
    qr1 = torch.randn((B, H, w.d_r), generator=gen, device="cuda")
    M1 = torch.randn((H, w.d_h, w.d_n), generator=gen, device="cuda") * w.m_sigma
    q1 = torch.empty((B, H, row), device="cuda")
    o1 = torch.empty((B, H, w.d_h), device="cuda")
    ml = int(lens.max()) + C + 1
    wsb = gb.gva_decode_workspace_bytes(dc.dims, B, ml, 0)
    ws = torch.zeros(max(wsb, 256) // 4, dtype=torch.float32, device="cuda")
    launches = gb.gva_decode_step_launches(dc.dims, dc.cache, B, ml, 0)

    def step():
        gb.gva_decode_step(dc.dims, dc.cache, B, pos, v1, k1, qn1, qr1, M1, sl, ml, w.scale, q1,
                           o1, None, workspace=ws, stream=stream)

    settle(step, torch)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    td = sorted(e0.elapsed_time(e1) / 1e3 for e0, e1 in evs)[iters // 2]
    dec_bytes = int((lens + C + 1).sum()) * (w.G * w.d_h + w.d_r) * 2
    log(f"C5 prefill: {t * 1e6:.1f} us, {tflops:.1f} TFLOP/s "
        f"({tflops * 1e12 / MFMA_PEAK_BF16:.1%} of bf16 dense peak); mix decode step {td * 1e6:.1f} us "
        f"({launches} launches)")
    assert torch.isfinite(out).all().item()
    res = {"workload": "4 sequences x (8192 cached + 512 causal queries), H=32, G=8, d_h=d_n=128, "
                       "d_r=16, bf16 cache in 16-token blocks; chunk append included",
           "us": round(t * 1e6, 2), "flop": flop, "TFLOP_s": round(tflops, 1),
           "mfma_util_bf16_dense": round(tflops * 1e12 / MFMA_PEAK_BF16, 4),
           "decode_step_after_us": round(td * 1e6, 2),
           "decode_step_after_launches": launches,
           "decode_step_after_GB_s": round(dec_bytes / td / 1e9, 1)}
    del dc
    torch.cuda.empty_cache()
    return res


def bench_small(torch, gb, synth, gen, stream, iters=50):
    """Latency of one decode step (append one token per sequence, absorb, decode) at the
    small-batch shapes, as three calls and as gva_decode_step (one launch at these shapes; the
    number is reported). Median of HIP-event times on the launch stream."""
    res = {}
    shapes = (("C2", dict(append_one=True, block_size=8192),
               "B=8, T=4096 (+1 appended), H=16, G=4, d_h=d_n=64, d_r=16, bf16 contiguous"),
              ("C1", dict(append_one=True, block_size=512),
               "B=1, T=256 (+1 appended), H=8, G=4, d_h=d_n=64, d_r=16, fp32 contiguous"))
    for name, kw, desc in shapes:
        w = synth.workload(name, **kw)
        lens = synth.lengths(w)
        dc = DeviceCache(w, lens, 99, torch, gb, synth)
        B, H = w.B, w.H
        seq = torch.arange(B, dtype=torch.int32, device="cuda")
        pos = torch.from_numpy(lens.astype(np.int32)).cuda()
        sl = pos + 1
        ml = int(lens.max()) + 1
        v = torch.randn((B, w.G, w.d_h), generator=gen, device="cuda")
        kr = torch.randn((B, w.d_r), generator=gen, device="cuda")
        qn = torch.randn((B, H, w.d_n), generator=gen, device="cuda")
        qr = torch.randn((B, H, w.d_r), generator=gen, device="cuda")
        M = torch.randn((H, w.d_h, w.d_n), generator=gen, device="cuda") * w.m_sigma
        qa = torch.empty((B, H, w.d_h + w.d_r), device="cuda")
        out = torch.empty((B, H, w.d_h), device="cuda")
        lse = torch.empty((B, H), device="cuda")
        wsb = gb.gva_decode_workspace_bytes(dc.dims, B, ml, 0)
        ws = torch.zeros(max(wsb, 256) // 4, dtype=torch.float32, device="cuda")

        def three_calls():
            gb.gva_cache_append(dc.dims, dc.cache, B, seq, pos, v, kr, stream=stream)
            gb.gva_absorb_query(dc.dims, qn, qr, pos, M, dc.cache.rope, dc.max_pos, qa,
                                stream=stream)
            gb.gva_decode(dc.dims, dc.cache, B, sl, ml, qa, w.scale, out, lse, workspace=ws,
                          stream=stream)

        def fused():
            gb.gva_decode_step(dc.dims, dc.cache, B, pos, v, kr, qn, qr, M, sl, ml, w.scale, qa,
                               out, lse, workspace=ws, stream=stream)

        r = {"workload": desc,
             "decode_step_launches": gb.gva_decode_step_launches(dc.dims, dc.cache, B, ml, 0)}
        if name == "C2":
            # the decode alone with the cache warm in the 256 MB last-level cache, and with 32
            # replicas rotated (570 MB) so that each call reads its cache from HBM
            reps = [dc] + [DeviceCache(w, lens, 100 + k, torch, gb, synth) for k in range(31)]
            fused()                                      # the absorbed queries the decode reads

            def dec(k):
                rc = reps[k % len(reps)]
                gb.gva_decode(rc.dims, rc.cache, B, sl, ml, qa, w.scale, out, lse, workspace=ws,
                              stream=stream)
            for label, rot in (("decode_mall_warm_us", False), ("decode_mall_defeated_us", True)):
                ctr = [0]

                def dec_next():
                    dec(ctr[0] if rot else 0)
                    ctr[0] += 1

                settle(dec_next, torch)
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(iters)]
                for k, (e0, e1) in enumerate(evs):
                    e0.record(stream)
                    dec(k if rot else 0)
                    e1.record(stream)
                torch.cuda.synchronize()
                r[label] = round(sorted(e0.elapsed_time(e1) for e0, e1 in evs)[iters // 2] * 1e3, 1)
            del reps
        for label, fn in (("three_calls_us", three_calls), ("decode_step_us", fused)):
            settle(fn, torch)
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(iters)]
            for e0, e1 in evs:
                e0.record(stream)
                fn()
                e1.record(stream)
            torch.cuda.synchronize()
            r[label] = round(sorted(e0.elapsed_time(e1) for e0, e1 in evs)[iters // 2] * 1e3, 1)
        assert torch.isfinite(out).all().item() and int(dc.cache.err_flag.item()) == 0
        log(f"{name} step ({desc}): three calls {r['three_calls_us']} us, "
            f"gva_decode_step {r['decode_step_us']} us ({r['decode_step_launches']} launches)")
        res[name] = r
        del dc
        torch.cuda.empty_cache()
    return res


def cpu_baseline(w, lens, budget_s=15.0):
    """The oracle, as it stands, decoding whole sequences of the same workload one by one until
    the time budget is spent: cache gather (bits -> float64) + absorbed decode of all heads."""
    from oracle import gva_oracle as O
    from value_only_kv_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    dims = O.Dims(w.H, w.G, w.d_h, w.d_n, w.d_r)
    tab = None
    done_bytes = 0
    done_seq = 0
    t_work = 0.0
    for b in range(w.B):
        n = int(lens[b]) + 1
        v, kr_raw = synth.sequence_tokens(w, b, n)
        # one sequence's own pool (contiguous), filled by the oracle's append
        pool = O.Pool.empty("bf16", n * w.G * w.d_h, n * w.d_r,
                            (n * w.G * w.d_h, w.G * w.d_h, w.d_h, n * w.d_r, w.d_r),
                            1, 1 << int(np.ceil(np.log2(n))), np.zeros((1, 1)))
        if tab is None or tab.shape[0] < n + 1:
            tab = O.rope_rows(np.arange(n + 1), w.d_r, w.base)
        O.append(pool, dims, np.zeros(n, np.int64), np.arange(n), v, kr_raw, tab)
        q = np.random.default_rng(b).standard_normal((w.H, w.d_h + w.d_r))
        t0 = time.perf_counter()
        V, kr = O.gather(pool, dims, 0, n)
        O.decode_sequence(V, kr, dims, q, w.scale)
        t_work += time.perf_counter() - t0
        done_bytes += n * (w.G * w.d_h + w.d_r) * 2
        done_seq += 1
        if t_work >= budget_s:
            break
    gbs = done_bytes / t_work / 1e9
    log(f"CPU oracle: {done_seq} sequences, {t_work:.1f}s, {gbs:.3f} GB/s, threads={threads}")
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seq_steps_per_s": round(done_seq / t_work, 3),
            "sample": f"first {done_seq} sequences of the ragged batch (len_b + 1 positions each), "
                      f"decode only (gather + fp64 attention), {t_work:.1f}s of CPU work"}


if __name__ == "__main__":
    main()
