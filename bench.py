#!/usr/bin/env python
"""DMS compact decode (and prefill) benchmark on one MI355X.

Decode workload (the headline): Qwen3-8B-shaped decode -- 36 layers, 32 q / 8 kv
heads, head_dim 128, bf16 K/V/Q ~ N(0,1), batch 1, an 8192-token prompt
compacted by prefill, then 128 decode steps (positions 8192..8319), delay window
w = 512, per-(layer, kv head) keep-score mean ~ U(-2, 0) (keep rates ~2%-50%).
All inputs are seeded synthetic data (synth/), resident in HBM before timing.

A step is one token through the whole DMS decode path of every layer: eviction
decision, expiry, slot reclaim, K/V append and split-K attention with merge.
`value` is decode tokens per second with one dms_decode_step call per token that
covers all 36 layers (their inputs are independent in this synthetic workload).
Two model-faithful modes are timed beside it ("modes"): one call per layer (36
calls per token) and a HIP graph of those 36 calls.

Prefill leg ("prefill"): Qwen3-8B-shaped DMS prefill of one 32768-token prompt
(32 q / 8 kv heads, D=128, w=512, keep score N(-1.2,1)), one layer's inputs
prefilled into 36 layer slots: masked causal attention on MFMA plus compaction.

Prints one JSON line.  --gpus N with N > 1 exits: the library runs on one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import re
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "DMS compact decode tok/s + achieved HBM GB/s (% peak), Qwen3-8B shape, 8K ctx"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# Kernel sources whose HBM traffic the committed counter summary describes; the
# figure is reported only while these files are unchanged.
TRAFFIC_SOURCES = ["compact_decode_attention_amd/csrc/dms_kernels.hip",
                   "compact_decode_attention_amd/csrc/dms_internal.h"]
TRAFFIC_SUMMARY = "profiles/decode_attend_qwen3-8b_hbm_traffic.md"
TRAFFIC_SUMMARY_FP8 = "profiles/decode_attend_fp8_qwen3-8b_hbm_traffic.md"


def sources_sha256(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(summary=TRAFFIC_SUMMARY):
    """HBM bytes per launch of a decode attention kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (each scaled by the same counter's
    reading for a plain copy of known size), or None when the summary is missing
    or was taken on other kernel sources."""
    path = os.path.join(ROOT, summary)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^- (\w+): (\S+)\s*$", line)
            if m:
                kv[m.group(1)] = m.group(2)
    if kv.get("source_sha256") != sources_sha256(TRAFFIC_SOURCES):
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, mib):
    """A plain device-to-device copy of known size, three times, so a counter
    run over this process can scale FETCH_SIZE / WRITE_SIZE to bytes."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: 3 copies of %d bytes" % n)
    del src, dst


def live_counts(logits_hd, t_values, window):
    """Live tokens of one head at each query position t (byte / flop accounting):
    #{s <= t-w : logit_s <= 0} + min(t+1, w)."""
    unmarked = (logits_hd <= 0).astype(np.int64)
    csum = np.concatenate([[0], np.cumsum(unmarked)])  # csum[i] = #unmarked in [0, i)
    t = np.asarray(t_values, np.int64)
    return csum[np.maximum(t - window + 1, 0)] + np.minimum(t + 1, window)


def live_counts_all(logits, t, window):
    """Live tokens of every head (columns of logits [positions][heads]) at position t."""
    unmarked = np.sum(logits[:max(t - window + 1, 0)] <= 0, axis=0).astype(np.int64)
    return unmarked + min(t + 1, window)


def bf16_tensor(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
KEEP_LAW = {"normal": "keep score N(-1.2,1) (about 1 in 8 kept)",
            "uniform_mu": "keep-score mean U(-2,0) per head",
            "beta": "keep rate Beta(2,14) per head"}


def bench_decode(args, torch, dms, kv_format=0, modes=None, cpu_steps=None, logit_channel=None, workload=None,
                 marks="keep_score"):
    """The decode leg; kv_format 1 runs it on an FP8 (E4M3) pool; logit_channel c
    carries each token's eviction logit (as bf16) in channel c of its K row and
    the pool reads it from there (no logits input; the same marks); marks
    "literal" hands the keep scores over as logits unchanged (mark iff s > 0:
    about 11.5% marked instead of about 88.5%)."""
    fp8 = kv_format == 1
    wl = synth.WORKLOADS[workload or args.workload]
    if wl.prefill_only or wl.n_seqs != 1:
        raise SystemExit("decode workload must be a single-sequence decode workload")
    inp = synth.SynthInputs(wl, marks=marks)
    L, Hq, H, D, w = wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    ctx = int(inp.ctx_lens()[0])
    K, W = args.steps, args.warmup
    if K > wl.gen_len:
        raise SystemExit("--steps beyond the workload's %d generated tokens" % wl.gen_len)
    S_all = max(K, W)
    total = ctx + S_all
    dev = torch.device("cuda:0")

    t0 = time.time()
    pk, pv, plg, host_k, host_v, host_lg = [], [], [], [], [], []
    for l in range(L):
        k, v, lg = inp.k(0, l, 0, total), inp.v(0, l, 0, total), inp.logits(0, l, 0, total)
        if logit_channel is not None:
            u = lg.view(np.uint32).astype(np.uint64)
            k[:, :, logit_channel] = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        host_k.append(k)
        host_v.append(v)
        host_lg.append(lg)
        pk.append(bf16_tensor(k[:ctx], torch).to(dev))
        pv.append(bf16_tensor(v[:ctx], torch).to(dev))
        plg.append(torch.from_numpy(lg[:ctx]).to(dev))
    q_host = np.stack([inp.q(0, l, ctx, S_all) for l in range(L)], axis=1)  # [S][L][Hq][D]
    dq = bf16_tensor(q_host, torch).to(dev).view(S_all, L, 1, Hq, D)
    dk = bf16_tensor(np.stack([x[ctx:total] for x in host_k], axis=1), torch).to(dev).view(S_all, L, 1, H, D)
    dv = bf16_tensor(np.stack([x[ctx:total] for x in host_v], axis=1), torch).to(dev).view(S_all, L, 1, H, D)
    dl = torch.from_numpy(np.stack([x[ctx:total] for x in host_lg], axis=1)).to(dev).view(S_all, L, 1, H)
    dout = torch.empty((S_all, L, 1, Hq, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log("decode inputs ready in %.1fs (ctx %d, %d layers)" % (time.time() - t0, ctx, L))

    pool = dms.Pool(n_layers=L, n_q_heads=Hq, n_kv_heads=H, head_dim=D, window=w, max_seqs=1,
                    max_positions=total, max_pages=L * H * ((total + 63) // 64), kv_format=kv_format,
                    logit_channel=logit_channel, device=dev)
    arena_bytes = pool.nbytes
    from_k = logit_channel is not None  # the pool reads the logits from K
    stream = torch.cuda.current_stream(dev)
    row_bytes = D + 4 if fp8 else 2 * D  # one stored K (or V) row

    def reset():
        pool.release(0)
        for l in range(L):
            pool.prefill(0, l, pk[l], pv[l], None if from_k else plg[l])
        torch.cuda.synchronize()

    # The timed loops call the C entry point through the binding with device
    # pointers computed beforehand (the Pool wrapper's per-call tensor checks
    # would otherwise cost the GPU idle time between steps).
    lib, vp = dms.lib(), ctypes.c_void_p
    seq0 = (ctypes.c_int32 * 1)(0)
    sp = vp(stream.cuda_stream)
    row = lambda t, i, l=None: vp(t[i].data_ptr() if l is None else t[i, l].data_ptr())
    lgp = (lambda i, l=None: vp(None)) if from_k else (lambda i, l=None: row(dl, i, l))
    batched_args = [(vp(pool.handle), 1, seq0, 0, L, row(dq, i), row(dk, i), row(dv, i), lgp(i), row(dout, i), sp)
                    for i in range(S_all)]
    layer_args = [[(vp(pool.handle), 1, seq0, l, 1, row(dq, i, l), row(dk, i, l), row(dv, i, l), lgp(i, l),
                    row(dout, i, l), sp) for l in range(L)] for i in range(S_all)]

    def run_batched(i):
        dms._check(lib.dms_decode_step(*batched_args[i]))

    def run_per_layer(i):
        for args_l in layer_args[i]:
            dms._check(lib.dms_decode_step(*args_l))

    # graph mode: static buffers, 36 captured per-layer calls, inputs copied in per step
    sq, sk, sv = torch.empty_like(dq[0]), torch.empty_like(dk[0]), torch.empty_like(dv[0])
    sl, so = torch.empty_like(dl[0]), torch.empty_like(dout[0])
    graph = [None]

    def capture_graph():
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for l in range(L):
                    pool.decode_step([0], l, sq[l:l + 1], sk[l:l + 1], sv[l:l + 1], sl[l:l + 1], so[l:l + 1])
        stream.wait_stream(side)
        graph[0] = g

    def run_graph(i):
        sq.copy_(dq[i]); sk.copy_(dk[i]); sv.copy_(dv[i]); sl.copy_(dl[i])
        graph[0].replay()
        dout[i].copy_(so)

    runners = {"batched": run_batched, "per_layer": run_per_layer, "graph": run_graph}
    modes = modes or [m for m in args.modes.split(",") if m]
    results, outs = {}, {}
    for mode in modes:
        fn = runners[mode]
        reset()
        if mode == "graph":
            capture_graph()  # nothing runs during capture; positions live on the device
            reset()
        for i in range(W):
            fn(i)
        reset()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(K):
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1)
        st, _ = pool.stats(0)
        results[mode] = {"ms_per_step": ms / K, "tok_per_s": K / (ms / 1e3), "live_slots_end": int(st.live_slots)}
        outs[mode] = dout[:K].clone()
        log("decode%s %s: %.4f ms/step, %.1f tok/s" % (" (fp8 pool)" if fp8 else "", mode, ms / K, K / (ms / 1e3)))
    # the modes cut the page axis at different points (split-K rounding may
    # differ in the last bits): report the largest difference to the first mode
    diff = {m: float((outs[m].float() - outs[modes[0]].float()).abs().max()) for m in modes[1:]}

    # byte accounting from the logits: live slots read per step (the new token
    # comes from the inputs), q, out, k/v append, logits
    live = np.stack([np.stack([live_counts(host_lg[l][:, h], np.arange(ctx, ctx + K), w) for h in range(H)])
                     for l in range(L)])  # [L][H][K]
    st, live_end = pool.stats(0, per_head=True)
    assert np.array_equal(live[:, :, -1], live_end), "live counts differ from the logits"
    kv_read = int(np.sum(live - 1)) * 2 * row_bytes
    q_bytes = K * L * Hq * D * 2
    step_bytes = kv_read + q_bytes + K * L * (Hq * D * 2 + H * 2 * (2 * D + row_bytes) + H * 4)
    attend_bytes = (kv_read + q_bytes) / K  # per launch of the attention kernel

    roofline = None
    if not args.no_timing_pass:
        reset()
        dms.dms_timing_enable(pool.handle, True)
        for i in range(K):
            run_batched(i)
        tm = dms.dms_timing_read(pool.handle)
        dms.dms_timing_enable(pool.handle, False)
        n = tm.decode_launches
        avg_att, avg_mer = tm.decode_attend_ms / n, tm.decode_merge_ms / n
        achieved = attend_bytes / (avg_att / 1e3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    # the counter summaries were taken on the headline workload only
                    "traffic": measured_traffic(TRAFFIC_SUMMARY_FP8 if fp8 else TRAFFIC_SUMMARY)
                    if wl.name == "qwen3-8b_ctx8192" and marks == "keep_score" else None,
                    "kernel": "decode_attend_kernel<%d,%d,%s>" % (D, Hq // H, "fp8" if fp8 else "bf16"),
                    "cache": "K/V pages read with the non-temporal policy: they are not kept in the 256 MB "
                             "last-level cache between steps, so the bytes come from HBM",
                    "avg_launch_us": round(avg_att * 1e3, 2),
                    "bytes_per_launch": int(attend_bytes), "launches": int(n),
                    "merge_kernel_avg_launch_us": round(avg_mer * 1e3, 2)}
        log("decode attend kernel%s: %.2f us/launch, %.1f GB/s (%.1f%% of peak); merge kernel %.2f us"
            % (" (fp8)" if fp8 else "", avg_att * 1e3, achieved, 100 * achieved / HBM_PEAK_GBPS, avg_mer * 1e3))

    cpu = None
    S = min(args.cpu_baseline_steps if cpu_steps is None else cpu_steps, K)
    if S > 0:
        import oracle  # the CPU baseline is the oracle, timed as it stands
        cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        mk = [oracle.marks(host_lg[l]) for l in range(L)]
        tc = time.perf_counter()
        for i in range(S):
            t = ctx + i
            for l in range(L):
                oracle.attend(q_host[i, l][None], [t], host_k[l][:t + 1], host_v[l][:t + 1], mk[l][:t + 1], w)
        cpu_s = time.perf_counter() - tc
        cpu = {"value": round(S / cpu_s, 3), "unit": "tok/s", "cores": cores, "kind": "oracle",
               "sample": "%s: the first %d of the %d decode steps, all %d layers x %d q heads, masked "
                         "attention over the full uncompressed K/V; %.1f s" % (wl.name, S, K, L, Hq, cpu_s)}
        log("cpu oracle: %.2f tok/s on %d threads" % (S / cpu_s, cores))

    main = "batched" if "batched" in results else modes[0]
    step_gbps = step_bytes / (results[main]["ms_per_step"] * K / 1e3) / 1e9
    out = {
        "value": results[main]["tok_per_s"], "ms_per_step": results[main]["ms_per_step"],
        "achieved_step_GBps": round(step_gbps, 1),
        # the whole step, beside the attention kernel alone (roofline): algorithmic
        # bytes of a step over the step's time (both kernels and the gaps between)
        "step_roofline": {"bound": "hbm", "achieved": round(step_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": round(step_gbps / HBM_PEAK_GBPS, 4),
                          "scope": "whole decode step (attention + merge/append kernels + launch gaps), "
                                   "%s mode" % main, "bytes_per_step": int(step_bytes / K)},
        "roofline": roofline, "cpu_baseline": cpu,
        "modes": {m: {k: round(v, 5) if isinstance(v, float) else v for k, v in r.items()}
                  for m, r in results.items()},
        "modes_max_abs_diff": diff,
        "kv_gib": {"live": round(st.kv_bytes_live / 2**30, 4), "allocated": round(st.kv_bytes_allocated / 2**30, 4),
                   "dense_equivalent": round(st.kv_bytes_dense_equiv / 2**30, 4),
                   "arena": round(arena_bytes / 2**30, 4)},
        "config": {"workload": "%s decode: %d layers, %d q / %d kv heads, head_dim %d, batch 1, ctx %d, "
                               "%d decode steps, w %d, %s%s"
                               % (wl.name, L, Hq, H, D, ctx, K, w, KEEP_LAW[wl.keep_law],
                                  ", literal marks (logit = +keep score)" if marks == "literal" else ""),
                   "call": "one dms_decode_step per token over all %d layers" % L,
                   "parallelism": "single GPU"},
    }
    pool.close()
    return out


# ---------------------------------------------------------------------------
# batched ragged decode (the bandwidth-scale workload)
# ---------------------------------------------------------------------------
def bench_ragged(args, torch, dms):
    """32 sequences with prompts of 4096..32768 tokens in one shared pool, 64
    decode steps, one dms_decode_step per token over all sequences and layers.
    Eviction logits (hence live sets, pages and bytes) come from the counter-based
    generator; K/V/q values from torch's seeded device generator (their values do
    not change the work)."""
    wl = synth.WORKLOADS["qwen3-8b_batch32_ragged"]
    inp = synth.SynthInputs(wl)
    L, Hq, H, D, w, B, S = (wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.n_seqs,
                            wl.gen_len)
    ctx = [int(c) for c in inp.ctx_lens()]
    dev = torch.device("cuda:0")
    t0 = time.time()
    logits = {}  # (seq, layer) -> [ctx + S][H]
    pages = 0
    for s_ in range(B):
        for l in range(L):
            lg = inp.logits(s_, l, 0, ctx[s_] + S)
            logits[(s_, l)] = lg
            n_end = live_counts_all(lg, ctx[s_] + S - 1, w)
            pages += int(np.sum((n_end + 63) // 64))
    pool = dms.Pool(n_layers=L, n_q_heads=Hq, n_kv_heads=H, head_dim=D, window=w, max_seqs=B,
                    max_positions=max(ctx) + S, max_pages=pages, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    for s_ in range(B):
        for l in range(L):
            T = ctx[s_]
            k = torch.randn((T, H, D), generator=gen, device=dev).to(torch.bfloat16)
            v = torch.randn((T, H, D), generator=gen, device=dev).to(torch.bfloat16)
            pool.prefill(s_, l, k, v, torch.from_numpy(logits[(s_, l)][:T]).to(dev))
            del k, v
    lg_steps = torch.from_numpy(np.stack([np.stack([logits[(s_, l)][ctx[s_]:ctx[s_] + S] for s_ in range(B)], axis=1)
                                          for l in range(L)], axis=1)).to(dev)  # [S][L][B][H]
    q = torch.randn((S, L, B, Hq, D), generator=gen, device=dev).to(torch.bfloat16)
    kd = torch.randn((S, L, B, H, D), generator=gen, device=dev).to(torch.bfloat16)
    vd = torch.randn((S, L, B, H, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((L, B, Hq, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log("ragged inputs ready in %.1fs (%d sequences, prompts %d..%d, %d pages)" % (time.time() - t0, B, min(ctx),
                                                                                  max(ctx), pages))
    seqs = list(range(B))
    stream = torch.cuda.current_stream(dev)
    dms.dms_timing_enable(pool.handle, True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(S):
        pool.decode_step(seqs, 0, q[i], kd[i], vd[i], lg_steps[i], out)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    tm = dms.dms_timing_read(pool.handle)
    dms.dms_timing_enable(pool.handle, False)
    # algorithmic bytes of the attention launches: live slots read before each append + q
    kv_read = 0
    for (s_, l), lg in logits.items():
        for h in range(H):
            kv_read += int(np.sum(live_counts(lg[:, h], np.arange(ctx[s_], ctx[s_] + S), w) - 1))
    attend_bytes = kv_read * 2 * D * 2 + S * L * B * Hq * D * 2
    achieved = attend_bytes / (tm.decode_attend_ms / 1e3) / 1e9
    st, _ = pool.stats()
    log("ragged decode: %.3f ms/step, %.1f tok/s; attention kernels %.1f GB/s (%.1f%% of peak)"
        % (ms / S, B * S / (ms / 1e3), achieved, 100 * achieved / HBM_PEAK_GBPS))
    res = {"workload": "%s: %d sequences, prompts U{%d..%d} (%d..%d drawn), %d layers, %d q / %d kv heads, "
                       "head_dim %d, w %d, keep rate Beta(2,14) per (layer, kv head), %d decode steps, "
                       "one shared page pool" % (wl.name, B, wl.ctx_len, wl.ctx_max, min(ctx), max(ctx), L, Hq, H,
                                                 D, w, S),
           "call": "one dms_decode_step per token over all %d sequences x %d layers (%d launches per step)"
                   % (B, L, tm.decode_launches // S),
           "tok_per_s": round(B * S / (ms / 1e3), 1), "ms_per_step": round(ms / S, 4),
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBPS, 4), "kernel": "decode_attend_kernel<128,4>",
                        "bytes_all_launches": int(attend_bytes), "launches": int(tm.decode_launches),
                        "attend_ms_total": round(tm.decode_attend_ms, 3),
                        "merge_ms_total": round(tm.decode_merge_ms, 3)},
           "kv_gib": {"live": round(st.kv_bytes_live / 2**30, 3), "allocated": round(st.kv_bytes_allocated / 2**30, 3),
                      "dense_equivalent": round(st.kv_bytes_dense_equiv / 2**30, 3)},
           "data": "logits from the counter-based generator; K/V/q from torch's seeded device generator"}
    pool.close()
    return res


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def bench_prefill(args, torch, dms):
    wl = synth.WORKLOADS["qwen3-8b_prefill32k"]
    inp = synth.SynthInputs(wl)
    T, Hq, H, D, w, R = wl.ctx_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.layer_repeats
    dev = torch.device("cuda:0")
    t0 = time.time()
    lg = inp.logits(0, 0, 0, T)
    q = bf16_tensor(inp.q(0, 0, 0, T), torch).to(dev)
    k = bf16_tensor(inp.k(0, 0, 0, T), torch).to(dev)
    v = bf16_tensor(inp.v(0, 0, 0, T), torch).to(dev)
    dl = torch.from_numpy(lg).to(dev)
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log("prefill inputs ready in %.1fs" % (time.time() - t0))
    pool = dms.Pool(n_layers=R, n_q_heads=Hq, n_kv_heads=H, head_dim=D, window=w, max_seqs=1,
                    max_positions=T, max_pages=R * H * (T // 64), device=dev)

    def run_all():
        for l in range(R):
            pool.prefill(0, l, k, v, dl, q=q, out=out)

    run_all()
    pool.release(0)
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    run_all()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    st, _ = pool.stats(0)
    pool.release(0)
    dms.dms_timing_enable(pool.handle, True)
    run_all()
    tm = dms.dms_timing_read(pool.handle)
    dms.dms_timing_enable(pool.handle, False)
    avg_att = tm.prefill_attend_ms / tm.prefill_calls
    avg_cmp = tm.prefill_compact_ms / tm.prefill_calls
    # algorithmic flops of one layer: 4 * D per (q head, visible pair)
    pairs = sum(int(np.sum(live_counts(lg[:, h], np.arange(T), w))) for h in range(H))
    flops = 4.0 * D * (Hq // H) * pairs
    dense = 4.0 * D * Hq * T * (T + 1) / 2
    tflops = flops / (avg_att / 1e3) / 1e12
    log("prefill: %.3f ms for %d layers (%.0f tok/s); attend kernel %.1f us = %.1f TFLOP/s (%.1f%% of bf16 "
        "MFMA peak); compaction %.1f us" % (ms, R, T / (ms / 1e3), avg_att * 1e3, tflops,
                                            100 * tflops / MFMA_BF16_PEAK_TFLOPS, avg_cmp * 1e3))
    res = {"workload": "%s: one %d-token prompt, %d q / %d kv heads, head_dim %d, w %d, keep score "
                       "N(-1.2,1), one layer's inputs prefilled into %d layer slots" % (wl.name, T, Hq, H, D, w, R),
           "tok_per_s": round(T / (ms / 1e3), 1), "ms_all_layers": round(ms, 4),
           "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                        "kernel": "prefill_attend3_kernel<128,4> (fp16 weights; its bf16-weights fallback, "
                                  "launched beside it, returns at once)", "avg_launch_us": round(avg_att * 1e3, 2),
                        "flops_per_launch": flops, "dense_causal_flops": dense},
           "compaction_avg_us": round(avg_cmp * 1e3, 2),
           "kv_gib": {"live": round(st.kv_bytes_live / 2**30, 4),
                      "dense_equivalent": round(st.kv_bytes_dense_equiv / 2**30, 4)}}
    pool.close()
    return res


def bench_extend(args, torch, dms):
    """Chunked prefill of the 32K prompt through dms_extend: the first 8192 tokens
    prefilled (no output), the other 24576 appended in 12 chunks of 2048 with
    output (the same outputs as the one-shot prefill's rows 8192..), one layer's
    inputs in 36 layer slots."""
    wl = synth.WORKLOADS["qwen3-8b_prefill32k"]
    inp = synth.SynthInputs(wl)
    T, Hq, H, D, w, R = wl.ctx_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.layer_repeats
    P0, C = 8192, 2048
    dev = torch.device("cuda:0")
    lg = inp.logits(0, 0, 0, T)
    q = bf16_tensor(inp.q(0, 0, 0, T), torch).to(dev)
    k = bf16_tensor(inp.k(0, 0, 0, T), torch).to(dev)
    v = bf16_tensor(inp.v(0, 0, 0, T), torch).to(dev)
    dl = torch.from_numpy(lg).to(dev)
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev)
    pool = dms.Pool(n_layers=R, n_q_heads=Hq, n_kv_heads=H, head_dim=D, window=w, max_seqs=1,
                    max_positions=T, max_pages=R * H * (T // 64), device=dev)
    stream = torch.cuda.current_stream(dev)

    def setup():
        pool.release(0)
        for l in range(R):
            pool.prefill(0, l, k[:P0], v[:P0], dl[:P0])

    def run_chunks():
        for t0 in range(P0, T, C):
            for l in range(R):
                pool.extend(0, l, k[t0:t0 + C], v[t0:t0 + C], dl[t0:t0 + C], q=q[t0:t0 + C], out=out[t0:t0 + C])

    setup()
    run_chunks()  # warm-up
    setup()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    run_chunks()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    setup()
    torch.cuda.synchronize()
    dms.dms_timing_enable(pool.handle, True)
    run_chunks()
    tm = dms.dms_timing_read(pool.handle)
    dms.dms_timing_enable(pool.handle, False)
    avg_att = tm.extend_attend_ms / tm.extend_calls
    pairs = sum(int(np.sum(live_counts(lg[:, h], np.arange(P0, T), w))) for h in range(H))
    flops = 4.0 * D * (Hq // H) * pairs / ((T - P0) // C)  # per launch (one chunk of one layer)
    tflops = flops / (avg_att / 1e3) / 1e12
    n_tok = T - P0
    log("chunked extend: %.3f ms for %d chunks x %d layers (%.0f tok/s); attend kernel %.1f us = %.1f TFLOP/s "
        "(%.1f%% of bf16 MFMA peak)" % (ms, (T - P0) // C, R, n_tok / (ms / 1e3), avg_att * 1e3, tflops,
                                        100 * tflops / MFMA_BF16_PEAK_TFLOPS))
    pool.close()
    return {"workload": "%s as a chunked prefill: %d tokens prefilled, then %d chunks of %d appended with "
                        "output by dms_extend, one layer's inputs in %d layer slots"
                        % (wl.name, P0, (T - P0) // C, C, R),
            "tok_per_s": round(n_tok / (ms / 1e3), 1), "ms_all_chunks_all_layers": round(ms, 4),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "kernel": "prefill_attend_kernel<128,4,bf16,extend>", "avg_launch_us": round(avg_att * 1e3, 2),
                         "flops_per_launch": flops}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128, help="timed decode steps (tokens)")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="qwen3-8b_ctx8192")
    ap.add_argument("--modes", default="batched,per_layer,graph")
    ap.add_argument("--cpu-baseline-steps", type=int, default=128,
                    help="decode steps the oracle is timed on (all layers); 0 disables")
    ap.add_argument("--no-timing-pass", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-ragged", action="store_true", help="skip the 32-sequence ragged batch leg")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-pool decode leg")
    ap.add_argument("--no-logit-channel", action="store_true", help="skip the K-channel-logits decode leg")
    ap.add_argument("--no-extend", action="store_true", help="skip the chunked-prefill (dms_extend) leg")
    ap.add_argument("--no-llama", action="store_true", help="skip the Llama-3.2-1B-shaped decode leg")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain copy of this many MiB (for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only (the library has no multi-GPU path); got --gpus %d" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import compact_decode_attention_amd as dms

    if args.copy_calibration_mib > 0:
        copy_calibration(torch, args.copy_calibration_mib)
    dec = bench_decode(args, torch, dms)
    f8 = None
    if not args.no_fp8:
        d8 = bench_decode(args, torch, dms, kv_format=1, modes=["batched", "per_layer"], cpu_steps=0)
        f8 = {"tok_per_s": round(d8["value"], 2), "ms_per_step": round(d8["ms_per_step"], 5),
              "achieved_step_GBps": d8["achieved_step_GBps"], "roofline": d8["roofline"], "kv_gib": d8["kv_gib"],
              "modes": d8["modes"], "modes_max_abs_diff": d8["modes_max_abs_diff"],
              "workload": "the decode workload above on an FP8 (OCP E4M3) pool: K/V rows stored as codes "
                          "with one fp32 scale each, one dms_decode_step per token over all layers "
                          "(modes.per_layer: one call per layer, 36 per token)"}
    lk = None
    if not args.no_logit_channel:
        dk_ = bench_decode(args, torch, dms, modes=["batched"], cpu_steps=0, logit_channel=0)
        lk = {"tok_per_s": round(dk_["value"], 2), "ms_per_step": round(dk_["ms_per_step"], 5),
              "attend_avg_launch_us": dk_["roofline"]["avg_launch_us"] if dk_["roofline"] else None,
              "merge_avg_launch_us": dk_["roofline"]["merge_kernel_avg_launch_us"] if dk_["roofline"] else None,
              "workload": "the decode workload above with each token's eviction logit carried (bf16) in "
                          "channel 0 of its K rows and read by the pool from there (no logits input)"}
    llama = None
    if not args.no_llama:
        l2 = bench_decode(args, torch, dms, modes=["batched", "per_layer"], cpu_steps=0,
                          workload="llama3.2-1b_ctx8192")
        l2lit = bench_decode(args, torch, dms, modes=["batched"], cpu_steps=0, workload="llama3.2-1b_ctx8192",
                             marks="literal")
        llama = {"workload": l2["config"]["workload"], "call": l2["config"]["call"],
                 "tok_per_s": round(l2["value"], 2), "ms_per_step": round(l2["ms_per_step"], 5),
                 "modes": l2["modes"], "step_roofline": l2["step_roofline"],
                 "kv_gib": l2["kv_gib"],
                 "cache_note": "the live compact cache (%.0f MB) fits the GPU's 256 MB last-level cache, so "
                               "the GB/s figures are effective bandwidth, not HBM bandwidth"
                               % (l2["kv_gib"]["live"] * 2**30 / 1e6),
                 "literal_marks": {"tok_per_s": round(l2lit["value"], 2), "ms_per_step": round(l2lit["ms_per_step"], 5),
                                   "kv_gib": l2lit["kv_gib"], "step_roofline": l2lit["step_roofline"],
                                   "cache_note": "%.0f MB live against the 256 MB last-level cache: at most partly "
                                                 "resident" % (l2lit["kv_gib"]["live"] * 2**30 / 1e6),
                                   "workload": l2lit["config"]["workload"]},
                 "pages_context": {"note": "the FastDMS announcement's tables for Llama-3.2-1B at ctx 8192 / gen "
                                           "128, c = 1, end-to-end model inference on unstated hardware: context, "
                                           "not a target",
                                   "kv_gib_vllm_bf16": 0.312, "kv_gib_fastdms": 0.056,
                                   "decode_tok_per_s_vllm_bf16": 459.4}}
    pre = None if args.no_prefill else bench_prefill(args, torch, dms)
    ext = None if args.no_extend else bench_extend(args, torch, dms)
    rag = None if args.no_ragged else bench_ragged(args, torch, dms)
    rec = {
        "metric": METRIC,
        "value": round(dec["value"], 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dec["config"],
        "achieved_step_GBps": dec["achieved_step_GBps"],
        "roofline": dec["roofline"],
        "step_roofline": dec["step_roofline"],
        "cpu_baseline": dec["cpu_baseline"],
        "modes": dec["modes"],
        "modes_max_abs_diff": dec["modes_max_abs_diff"],
        "kv_gib": dec["kv_gib"],
        "fp8_kv": f8,
        "llama3.2-1b_ctx8192": llama,
        "logits_from_k_channel": lk,
        "prefill": pre,
        "chunked_extend": ext,
        "batched_ragged": rag,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
