"""Benchmark of one LongCat Sparse Attention layer forward on one MI355X.

Workload (decode sweep): a batch of 32 single-token decode queries, bf16; Lightning Indexer with
64 heads x 128 dims over the middle region, flat top-1024, 16 sink + 1024 window + 1024 sparse
tokens, attention of 128 heads over the 576-dim MLA latent; 64 planted needles per sequence;
inputs seeded and resident in HBM before timing starts.  A step is one full layer forward
(lsa_layer_fwd: indexer scoring, top-K, hybrid attention) over the batch.  The headline value is
the layer latency at KV length 1M; the 128K leg is reported beside it.

Prints one JSON line.  Single GPU only.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12        # B/s, MI355X HBM3E
BF16_PEAK = 2.5e15       # FLOP/s dense MFMA
MALL_FLUSH_BYTES = 512 << 20  # more than the 256 MB last-level (Infinity) cache: a "cold" call reads HBM


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_on_stream(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps * 1e-3  # seconds per call


SETTLE_S = 0.05


def settle(fn, seconds=SETTLE_S):
    """Runs fn back to back for about `seconds` of GPU time before the warm-up steps.  After any idle
    period the GPU's power management brings its clocks back over some tens of milliseconds: on the
    1M decode step the first ~20 calls take 50-200 us longer than the later ones, then settle.  Returns
    the number of calls run (reported with the result)."""
    import torch
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()  # (the first call also pays one-off costs: it does not size the loop)
    e0.record(s)
    fn()
    e1.record(s)
    torch.cuda.synchronize()
    n = max(1, int(seconds / max(e0.elapsed_time(e1) * 1e-3, 1e-6)))
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    return n + 2


def step_distribution(fn, reps, flush_bytes=0):
    """Per-call times (us) with one event pair around each call: p10 / median / p90. With flush_bytes > 0
    a scratch buffer of that size is written before every call (outside its events), so that the call starts
    with the last-level cache holding none of its inputs ("cold")."""
    import torch
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda") if flush_bytes else None
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    fn()
    torch.cuda.synchronize()
    for i in range(reps):
        if scratch is not None:
            scratch.fill_(i & 0xff)
        ev[i][0].record(s)
        fn()
        ev[i][1].record(s)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    q = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
    del scratch
    return dict(p10=q(0.1), p50=q(0.5), p90=q(0.9))


TRAFFIC_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "index_topk_fused_decode_b32_1m_traffic.md")
TRAFFIC_L = 1048576
TRAFFIC_SOURCES = ("index_score.hip", "topk.hip", "topk_block.hpp", "lsa_dev.hpp", "lsa_kernels.hpp")


def measured_traffic():
    """HBM bytes per lsa_index_topk call (its kernels summed) from the committed rocprofv3 counter summary,
    or None when the kernels' sources changed since the counters were taken (their hash differs)."""
    import hashlib
    try:
        line = [v for v in open(TRAFFIC_PROFILE).read().splitlines() if v.startswith("traffic:")][0]
    except (OSError, IndexError):
        return None
    f = dict(kv.split("=", 1) for kv in line.split()[1:])
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_sparse_weighted_amd", "csrc")
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != f["source_sha256"]:
        return None
    return round(float(f["fetch_kib"]) * float(f["fetch_scale"]) * 1024 +
                 float(f["write_kib"]) * float(f["write_scale"]) * 1024)


def run_length(L, batch, steps, warmup, seed=0):
    import torch

    import long_context_sparse_weighted_amd as lsa
    import synth
    t0 = time.time()
    x = synth.decode_sweep(L, device="cuda", seed=seed, batch=batch)
    torch.cuda.synchronize()
    log(f"[bench] L={L}: inputs ready in {time.time() - t0:.1f}s")
    c = x["cfg"]
    rows = lsa.RowsDesc(x["kv_off"], x["row_seq"], x["row_pos"], x["max_len"])
    layer = lsa.Layer(c, rows, torch.bfloat16, "cuda")
    n = batch
    idx = torch.full((n, c["k_sparse"]), -1, dtype=torch.int32, device="cuda")
    out = torch.empty((n, c["H"], c["Dv"]), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((n, c["H"]), dtype=torch.float32, device="cuda")

    def step():
        layer(x["q"], x["kv"], idx, out, lse, q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"])

    # Whole-step timing: K steps between two synchronisations, after the clocks have settled and the
    # W warm-up steps.
    n_settle = settle(step)
    torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t_start) / steps
    t_step_ev = time_on_stream(step, steps, 0)
    warm = step_distribution(step, steps)
    cold = step_distribution(step, steps, flush_bytes=MALL_FLUSH_BYTES)
    # The dominant kernel: the layer's flat selection (scoring fused with the first top-K level, then the
    # top-K levels over the candidate lists), as lsa_index_topk launches it for the layer, same stream.
    bud = (c["k_sink"], c["k_swa"], c["k_sparse"])
    sel = torch.empty((n, c["k_sparse"]), dtype=torch.int32, device="cuda")
    sel_ws = lsa.lsa_index_topk_workspace(rows, x["q_idx"], c["k_sparse"])
    t_sel = time_on_stream(lambda: lsa.lsa_index_topk(rows, x["q_idx"], x["w"], x["k_idx"], bud, idx=sel, ws=sel_ws),
                           steps, warmup)
    assert torch.equal(sel, idx), "lsa_index_topk and the layer disagree"
    # For comparison: the scoring kernel alone when it writes the fp32 scores (the unfused pass).
    scores = torch.empty((n, L), dtype=torch.float32, device="cuda")
    t_score = time_on_stream(lambda: lsa.lsa_index_score(rows, x["q_idx"], x["w"], x["k_idx"], bud, scores=scores),
                             steps, warmup)
    # Needle sanity (not timed): every planted needle is selected.
    got = idx.cpu().numpy()
    recall = sum(len(set(p) & set(got[b].tolist())) for b, p in enumerate(x["needles"])) / max(
        1, sum(len(p) for p in x["needles"]))
    mid = L - c["k_sink"] - c["k_swa"]
    k_bytes = n * mid * 128 * 2                       # indexer keys (the dominant stream)
    attn_bytes = n * (c["k_sink"] + c["k_swa"] + c["k_sparse"]) * 576 * 2
    io_bytes = n * (64 * 128 * 2 + 64 * 4 + 128 * 576 * 2 + 128 * 512 * 2 + 128 * 4 + c["k_sparse"] * 4)
    alg_bytes = k_bytes + attn_bytes + io_bytes
    flops = n * (mid * 64 * 128 * 2 + (c["k_sink"] + c["k_swa"] + c["k_sparse"]) * 128 * (576 + 512) * 2)
    del scores, sel, sel_ws
    res = dict(L=L, batch=n, settle_calls=n_settle, latency_us=t_step * 1e6, latency_us_events=t_step_ev * 1e6,
               warm_us_p10=warm["p10"], warm_us_p50=warm["p50"], warm_us_p90=warm["p90"],
               cold_us_p10=cold["p10"], cold_us_p50=cold["p50"], cold_us_p90=cold["p90"],
               select_us=t_sel * 1e6, select_gbs=k_bytes / t_sel / 1e9, score_kernel_bytes=k_bytes,
               unfused_score_kernel_us=t_score * 1e6, unfused_score_kernel_gbs=k_bytes / t_score / 1e9,
               alg_bytes=alg_bytes, flops=flops, hbm_frac_layer=alg_bytes / t_step / HBM_PEAK, needle_recall=recall)
    log(f"[bench] L={L}: layer {t_step * 1e6:.1f} us ({res['hbm_frac_layer'] * 100:.1f}% HBM), flat selection "
        f"{t_sel * 1e6:.1f} us = {res['select_gbs']:.0f} GB/s of keys (unfused scoring alone {t_score * 1e6:.1f} us), "
        f"needle recall {recall:.3f}; per call "
        f"warm p10/p50/p90 {warm['p10']:.1f}/{warm['p50']:.1f}/{warm['p90']:.1f} us, cold (cache flushed) "
        f"{cold['p10']:.1f}/{cold['p50']:.1f}/{cold['p90']:.1f} us")
    del x, layer, idx, out, lse
    torch.cuda.empty_cache()
    return res


def bench_fp8(steps, warmup, lengths=(131072, 1048576), batch=32):
    """Decode step with the FP8 indexer (the decode batch of the headline, same inputs): per step the
    queries are quantized, the FP8 key cache (quantized once, outside the step) is scored and selected
    from (lsa_index_topk_fp8), then the bf16 hybrid attention, all through the C ABI on one stream."""
    import torch

    import long_context_sparse_weighted_amd as lsa
    import synth
    res = {}
    for L in lengths:
        x = synth.decode_sweep(L, device="cuda", batch=batch)
        c = x["cfg"]
        bud = (c["k_sink"], c["k_swa"], c["k_sparse"])
        rows = lsa.RowsDesc(x["kv_off"], x["row_seq"], x["row_pos"], x["max_len"], L)
        t_kq = time_on_stream(lambda: lsa.lsa_quantize_fp8(x["k_idx"]), 2, 1)
        k8, ks = lsa.lsa_quantize_fp8(x["k_idx"])
        q8 = torch.empty(x["q_idx"].shape, dtype=torch.uint8, device="cuda")
        qs = torch.empty(x["q_idx"].shape[:2], dtype=torch.float32, device="cuda")
        scores = torch.empty((batch, L), dtype=torch.float32, device="cuda")
        idx = torch.empty((batch, c["k_sparse"]), dtype=torch.int32, device="cuda")
        out = torch.empty((batch, c["H"], c["Dv"]), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((batch, c["H"]), dtype=torch.float32, device="cuda")
        lsa.lsa_quantize_fp8(x["q_idx"], q8, qs)
        sel_ws = lsa.lsa_index_topk_fp8_workspace(rows, q8, c["k_sparse"])

        def step():
            lsa.lsa_quantize_fp8(x["q_idx"], q8, qs)
            lsa.lsa_index_topk_fp8(rows, q8, qs, x["w"], k8, ks, bud, idx=idx, ws=sel_ws)
            lsa.lsa_hybrid_attn(rows, x["q"], x["kv"], c["Dv"], c["scale"], bud, idx, out=out, lse=lse)
        t_step = time_on_stream(step, steps, warmup)
        t_sel = time_on_stream(lambda: lsa.lsa_index_topk_fp8(rows, q8, qs, x["w"], k8, ks, bud, idx=idx, ws=sel_ws),
                               steps, warmup)
        t_score = time_on_stream(lambda: lsa.lsa_index_score_fp8(rows, q8, qs, x["w"], k8, ks, bud, scores=scores),
                                 steps, warmup)
        assert torch.equal(idx, lsa.lsa_topk(scores, c["k_sparse"])), "fused and separate FP8 selections disagree"
        got = idx.cpu().numpy()
        recall = sum(len(set(p) & set(got[b].tolist())) for b, p in enumerate(x["needles"])) / max(
            1, sum(len(p) for p in x["needles"]))
        mid = L - c["k_sink"] - c["k_swa"]
        k_bytes = batch * mid * 132                     # E4M3 codes + fp32 scale per key
        res[str(L)] = dict(step_us=t_step * 1e6, select_us=t_sel * 1e6, select_gbs=k_bytes / t_sel / 1e9,
                           unfused_score_kernel_us=t_score * 1e6, score_kernel_bytes=k_bytes,
                           unfused_score_kernel_gbs=k_bytes / t_score / 1e9, key_cache_quantize_us=t_kq * 1e6,
                           needle_recall=recall)
        log(f"[bench] FP8 indexer L={L}: step {t_step * 1e6:.1f} us, FP8 selection (fused scoring + top-K) "
            f"{t_sel * 1e6:.1f} us = {k_bytes / t_sel / 1e9:.0f} GB/s of keys (unfused scoring alone "
            f"{t_score * 1e6:.1f} us), key cache quantize {t_kq * 1e6:.0f} us, needle recall {recall:.3f}")
        del x, k8, ks, scores, sel_ws
        torch.cuda.empty_cache()
    return res


def cpu_threads():
    """Host threads for the oracle: every CPU this process may run on, capped by the job's thread share
    (OMP_NUM_THREADS; 16 when unset), so that a large shared host is not oversubscribed."""
    avail = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    return max(1, min(avail, share)), avail


def cpu_baseline(L=1048576, batch=32, seed=0):
    """The oracle on a bounded sample of the benchmark's own workload: as many rows of the L-token decode
    batch as there are host threads (one row per thread, rows run concurrently), timed on the host; the
    whole-batch figure is that wall time scaled by batch / rows."""
    import torch

    import oracle as ref
    import synth
    threads, avail = cpu_threads()
    rows = min(batch, threads)
    x = synth.decode_batch([L] * rows, device="cuda", seed=seed)
    h = synth.to_host
    o = dict(kv_off=x["kv_off_host"].numpy(), row_seq=x["row_seq_host"].numpy(), row_pos=x["row_pos_host"].numpy(),
             q_idx=h(x["q_idx"]), w=h(x["w"]), k_idx=h(x["k_idx"]), q=h(x["q"]), kv=h(x["kv"]))
    del x
    torch.cuda.empty_cache()
    t0 = time.perf_counter()
    ref.layer_fwd(dict(HI=64, dI=128, H=128, Dqk=576, Dv=512, scale=1 / math.sqrt(576), k_sink=16, k_swa=1024,
                       k_sparse=1024, is_owner=1), o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"],
                  o["k_idx"], o["q"], o["kv"], threads=threads)
    dt = time.perf_counter() - t0
    del o
    scale = batch / rows
    batch_us = dt * scale * 1e6
    log(f"[bench] oracle: {rows} rows at L={L} in {dt:.1f}s on {threads} threads ({avail} CPUs available)")
    return dict(value=batch_us, unit="us", cores=threads, threads=threads, host_cpus=avail, kind="oracle",
                extrapolated=scale != 1.0,
                sample=f"{rows} of the {batch} rows of the L={L} decode batch, one row per thread on {threads} host "
                       f"threads ({avail} CPUs in the process's affinity set), {dt:.2f} s wall; the value is that "
                       f"time x{scale:g} for the whole {batch}-row batch")


def time_layer(x, cfg, steps, warmup, idx_row=None, sb_off=None, k_mean=None, q=None, kv=None, idx=None):
    """Seconds per lsa_layer_fwd call (events on the stream the library launches on)."""
    import torch

    import long_context_sparse_weighted_amd as lsa
    rows = lsa.RowsDesc(x["kv_off"], x["row_seq"], x["row_pos"], x["max_len"], min(x["lengths"]))
    n = x["row_pos"].numel()
    layer = lsa.Layer(cfg, rows, torch.bfloat16, "cuda", use_hi=k_mean is not None)
    if idx is None:
        idx = torch.full((n, cfg["k_sparse"]), -1, dtype=torch.int32, device="cuda")
    out = torch.empty((n, cfg["H"], cfg["Dv"]), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((n, cfg["H"]), dtype=torch.float32, device="cuda")
    qq, kk = (x["q"] if q is None else q), (x["kv"] if kv is None else kv)
    t = time_on_stream(lambda: layer(qq, kk, idx, out, lse, q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"],
                                     idx_row=idx_row, sb_off=sb_off, k_mean=k_mean), steps, warmup)
    return t, idx


def bench_hi(steps, warmup, lengths=(262144, 524288, 1048576), batch=8, B=128):
    """Long-context decode with HI (batch 8, P = 128, sub-blocks of B, M = 1024) against the flat indexer
    on the same inputs; also the one-off mean build and the per-step mean upkeep (one appended token
    per sequence)."""
    import torch

    import long_context_sparse_weighted_amd as lsa
    import synth
    res = {}
    for L in lengths:
        x = synth.hi_decode(device="cuda", L=L, batch=batch, B=B)
        c = x["cfg"]
        sb_off = lsa.sb_offsets(x["lengths"], B).to("cuda")
        t_means = time_on_stream(lambda: lsa.lsa_page_means(x["kv_off"], sb_off, x["k_idx"], B, L), 3, 1)
        km = lsa.lsa_page_means(x["kv_off"], sb_off, x["k_idx"], B, L)
        t_upkeep = time_on_stream(lambda: lsa.lsa_page_means_append(x["kv_off"], sb_off, x["k_idx"], B, km, 1),
                                  steps, warmup)
        t_hi, idx_hi = time_layer(x, c, steps, warmup, sb_off=sb_off, k_mean=km)
        t_flat, idx_flat = time_layer(x, dict(c, hi_min_len=1 << 62), steps, warmup)
        # k_mean of the causal pages (stage 1), the recalled pages' keys (stage 2), the selected KV rows
        hi_bytes = batch * (L // B * 256 + 1024 * 128 * 256 + 2064 * 1152)
        res[str(L)] = dict(B=B, hi_us=t_hi * 1e6, flat_us=t_flat * 1e6, speedup=t_flat / t_hi,
                           page_means_build_us=t_means * 1e6, page_means_upkeep_us=t_upkeep * 1e6,
                           hi_alg_bytes=hi_bytes, hi_hbm_frac=hi_bytes / t_hi / HBM_PEAK,
                           same_sets_rows=int((idx_hi == idx_flat).all(1).sum().item()))
        log(f"[bench] HI B={B} L={L}: HI {t_hi * 1e6:.1f} us, flat {t_flat * 1e6:.1f} us ({t_flat / t_hi:.2f}x), "
            f"mean build {t_means * 1e6:.0f} us, per-step upkeep {t_upkeep * 1e6:.1f} us")
        del x, km
        torch.cuda.empty_cache()
    return res


def bench_hi_prefill(steps, warmup, lengths=(32768, 65536, 131072, 262144, 524288, 1048576), q_len=2048):
    """HI against the flat indexer in chunked prefill (q_len rows at the end of an L-token sequence;
    P = 128, B = 8, M = 1024; K = 1024 picks): stage 1 = page recall (sub-block scoring, page sums,
    page top-M), stage 2 = token scoring over the recalled pages + top-K; flat = scoring + top-K."""
    import torch

    import long_context_sparse_weighted_amd as lsa
    import synth
    res = {}
    for L in lengths:
        x = synth.hi_prefill(L, device="cuda", q_len=q_len)
        c = x["cfg"]
        P, B, M, K = c["P"], c["B"], c["M"], c["k_sparse"]
        bud = (c["k_sink"], c["k_swa"], K)
        rows = lsa.RowsDesc(x["kv_off"], x["row_seq"], x["row_pos"], x["max_len"], L)
        sb_off = lsa.sb_offsets(x["lengths"], B).to("cuda")
        t_means = time_on_stream(lambda: lsa.lsa_page_means(x["kv_off"], sb_off, x["k_idx"], B, L), 3, 1)
        km = lsa.lsa_page_means(x["kv_off"], sb_off, x["k_idx"], B, L)
        ps = torch.empty((q_len, (L + P - 1) // P), dtype=torch.float32, device="cuda")
        st = {}

        def stage1():
            st["pages"], _ = lsa.lsa_page_recall(rows, sb_off, x["q_idx"], x["w"], km, P, B, M, page_scores=ps)
        t1 = time_on_stream(stage1, steps, warmup)
        comp = torch.empty((q_len, M * P), dtype=torch.float32, device="cuda")
        idx_hi = torch.empty((q_len, K), dtype=torch.int32, device="cuda")

        def stage2():
            lsa.lsa_index_score(rows, x["q_idx"], x["w"], x["k_idx"], bud, scores=comp, pages=st["pages"], M=M, P=P)
            lsa.lsa_topk(comp, K, pages=st["pages"], P=P, idx=idx_hi)
        t2 = time_on_stream(stage2, steps, warmup)
        del comp
        scores = torch.empty((q_len, L), dtype=torch.float32, device="cuda")
        idx_flat = torch.empty((q_len, K), dtype=torch.int32, device="cuda")

        def flat():
            lsa.lsa_index_score(rows, x["q_idx"], x["w"], x["k_idx"], bud, scores=scores)
            lsa.lsa_topk(scores, K, idx=idx_flat)
        tf = time_on_stream(flat, steps, warmup)
        res[str(L)] = dict(stage1_ms=t1 * 1e3, stage2_ms=t2 * 1e3, hi_total_ms=(t1 + t2) * 1e3, flat_ms=tf * 1e3,
                           speedup=tf / (t1 + t2), page_means_build_ms=t_means * 1e3,
                           same_sets_rows=int((idx_hi == idx_flat).all(1).sum().item()))
        log(f"[bench] HI prefill L={L}: stage 1 {t1 * 1e3:.3f} ms, stage 2 {t2 * 1e3:.3f} ms, HI "
            f"{(t1 + t2) * 1e3:.3f} ms, flat {tf * 1e3:.3f} ms ({tf / (t1 + t2):.2f}x), mean build "
            f"{t_means * 1e3:.2f} ms")
        del x, km, ps, scores, st
        torch.cuda.empty_cache()
    return res


def bench_prefill(steps, warmup):
    """Chunked prefill: 8192 causal rows over a 131072-token prefix; owner layer and CLI reuse layer."""
    import torch

    import long_context_sparse_weighted_amd as lsa
    import synth
    x = synth.chunked_prefill_cli(device="cuda")
    c = x["cfg"]
    (q1, kv1), (q2, kv2) = x["layers"]
    t_own, idx = time_layer(x, c, steps, warmup, q=q1, kv=kv1)
    t_reuse, _ = time_layer(x, dict(c, is_owner=0), steps, warmup, q=q2, kv=kv2, idx=idx)
    rows = lsa.RowsDesc(x["kv_off"], x["row_seq"], x["row_pos"], x["max_len"])
    scores = torch.empty((8192, x["max_len"]), dtype=torch.float32, device="cuda")
    t_idx = time_on_stream(lambda: lsa.lsa_index_score(rows, x["q_idx"], x["w"], x["k_idx"], (16, 1024, 1024),
                                                       scores=scores), steps, warmup)
    t_attn = time_on_stream(lambda: lsa.lsa_hybrid_attn(rows, q2, kv2, 512, c["scale"], (16, 1024, 1024), idx),
                            steps, warmup)
    n_keys = sum(int(t) - 1040 + 1 for t in x["row_pos_host"].tolist())
    idx_flops = n_keys * 64 * 128 * 2
    attn_flops = 8192 * 2064 * 128 * (576 + 512) * 2
    res = dict(owner_us=t_own * 1e6, reuse_us=t_reuse * 1e6, index_score_us=t_idx * 1e6, attention_us=t_attn * 1e6,
               index_flops=idx_flops, index_mfma_frac=idx_flops / t_idx / BF16_PEAK,
               attention_mfma_frac=attn_flops / t_attn / BF16_PEAK)
    log(f"[bench] prefill: owner {t_own * 1e3:.2f} ms, reuse {t_reuse * 1e3:.2f} ms, indexer scoring "
        f"{t_idx * 1e3:.2f} ms ({res['index_mfma_frac'] * 100:.1f}% MFMA), attention {t_attn * 1e3:.2f} ms "
        f"({res['attention_mfma_frac'] * 100:.1f}% MFMA)")
    return res


def ragged_alg_bytes(lengths, drafts=3, hi_min_len=262144, P=128, B=128, M=1024, k_sink=16, k_swa=1024,
                     k_sparse=1024):
    """The method's own HBM bytes for one ragged MTP layer call: indexer keys of each flat owner row
    (256 B per middle token), under HI the sub-block means of the causal pages and the keys of the M
    recalled pages, the selected latent rows once per sequence (its drafts share them), and per row q,
    out and lse (plus q_idx, w and idx per owner)."""
    total = 0
    for L in lengths:
        mid = max(0, L - k_sink - k_swa)
        if L >= hi_min_len:
            total += (L + B - 1) // B * 256 + min(M * P, mid) * 256
        else:
            total += mid * 256
        total += min(L, k_sink + k_swa + k_sparse) * 1152
        total += drafts * (128 * 576 * 2 + 128 * 512 * 2 + 128 * 4) + 64 * 128 * 2 + 64 * 4 + k_sparse * 4
    return total


def bench_ragged(steps, warmup):
    """64 ragged sequences (4K-512K), 3 MTP drafts each sharing the first draft's index; HI for L >= 256K."""
    import torch

    import long_context_sparse_weighted_amd as lsa
    import synth
    x = synth.ragged_mtp(device="cuda")
    c = x["cfg"]
    sb_off = lsa.sb_offsets(x["lengths"], 128).to("cuda")
    km = lsa.lsa_page_means(x["kv_off"], sb_off, x["k_idx"], 128, x["max_len"])
    t, _ = time_layer(x, c, steps, warmup, idx_row=x["idx_row"], sb_off=sb_off, k_mean=km)
    n_hi = sum(1 for L in x["lengths"] if L >= 262144)
    alg = ragged_alg_bytes(x["lengths"])
    log(f"[bench] ragged MTP: {t * 1e6:.1f} us for 64 sequences (sum L = {sum(x['lengths'])}, {n_hi} on HI), "
        f"{alg / 1e6:.1f} MB algorithmic = {alg / t / HBM_PEAK * 100:.1f}% of HBM peak")
    return dict(latency_us=t * 1e6, sum_len=sum(x["lengths"]), hi_sequences=n_hi, queries_per_s=192 / t,
                alg_bytes=alg, hbm_frac=alg / t / HBM_PEAK, hbm_bound_us=alg / HBM_PEAK * 1e6)


def bench_tiny(steps, warmup):
    import torch

    import synth
    x = synth.tiny_prefill(device="cuda")
    t, _ = time_layer_fp32(x, steps, warmup)
    log(f"[bench] tiny fp32 prefill: {t * 1e6:.1f} us")
    return dict(latency_us=t * 1e6)


def time_layer_fp32(x, steps, warmup):
    import torch

    import long_context_sparse_weighted_amd as lsa
    c = x["cfg"]
    rows = lsa.RowsDesc(x["kv_off"], x["row_seq"], x["row_pos"], x["max_len"])
    layer = lsa.Layer(c, rows, torch.float32, "cuda")
    n = x["row_pos"].numel()
    idx = torch.full((n, c["k_sparse"]), -1, dtype=torch.int32, device="cuda")
    out = torch.empty((n, c["H"], c["Dv"]), dtype=torch.float32, device="cuda")
    lse = torch.empty((n, c["H"]), dtype=torch.float32, device="cuda")
    return time_on_stream(lambda: layer(x["q"], x["kv"], idx, out, lse, q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"]),
                          steps, warmup), idx


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device copy of known size (for scaling the FETCH_SIZE / WRITE_SIZE counters)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(7)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} copies of {nbytes} bytes")
    del a, b


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=32)
    ap.add_argument("--lengths", default="131072,1048576")
    ap.add_argument("--hi-lengths", default="262144,524288,1048576", help="KV lengths of the HI workload")
    ap.add_argument("--hi-prefill-lengths", default="32768,65536,131072,262144,524288,1048576",
                    help="KV lengths of the HI chunked-prefill workload")
    ap.add_argument("--fp8-lengths", default="131072,1048576", help="KV lengths of the FP8 indexer workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="decode", choices=["decode", "hi", "hi_prefill", "fp8", "prefill", "ragged", "tiny", "all"],
                    help="decode prints the metric line; the others print their own figures as one JSON line")
    ap.add_argument("--copy-calibration", action="store_true", help="run a 1 GiB device copy first (PMC scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
    if args.workload != "decode":
        extra = {}
        if args.workload in ("hi", "all"):
            hl = [int(v) for v in args.hi_lengths.split(",")]
            extra["hi_decode_batch8"] = bench_hi(args.steps, args.warmup, lengths=hl)
            extra["hi_decode_batch8_B8"] = bench_hi(args.steps, args.warmup, lengths=hl, B=8)
        if args.workload in ("fp8", "all"):
            extra["fp8_indexer_decode"] = bench_fp8(args.steps, args.warmup,
                                                    lengths=[int(v) for v in args.fp8_lengths.split(",")])
        if args.workload in ("hi_prefill", "all"):
            extra["hi_prefill_qlen2048_B8"] = bench_hi_prefill(
                args.steps, args.warmup, lengths=[int(v) for v in args.hi_prefill_lengths.split(",")])
        if args.workload in ("prefill", "all"):
            extra["chunked_prefill_cli"] = bench_prefill(args.steps, args.warmup)
        if args.workload in ("ragged", "all"):
            extra["ragged_mtp"] = bench_ragged(args.steps, args.warmup)
        if args.workload in ("tiny", "all"):
            extra["tiny_fp32_prefill"] = bench_tiny(args.steps, args.warmup)
        if args.workload == "all":
            extra["decode_sweep"] = {str(L): run_length(L, args.batch, args.steps, args.warmup)
                                     for L in (4096, 16384, 65536, 131072, 262144, 1048576)}
        print(json.dumps(extra), flush=True)
        return
    lengths = [int(v) for v in args.lengths.split(",")]
    legs = [run_length(L, args.batch, args.steps, args.warmup) for L in lengths]
    head = legs[-1]
    cpu = None if args.no_cpu_baseline else cpu_baseline(L=head["L"], batch=args.batch)
    line = {
        "metric": "LSA layer fwd latency (us) at 128K/1M decode; % HBM peak and % MFMA peak",
        "value": round(head["latency_us"], 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["latency_us"] / 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode batch {args.batch} x 1 query, KV {head['L']}, bf16, HI=64 dI=128, "
                               f"H=128 latent 576/512, K=16+1024+1024, flat indexer, 64 needles/seq",
                   "global_batch": args.batch, "seq_len": head["L"], "parallelism": "single GPU"},
        "legs": {str(r["L"]): {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()} for r in legs},
        "queries_per_s": round(args.batch / (head["latency_us"] * 1e-6), 1),
        "hbm_frac_layer": round(head["hbm_frac_layer"], 4),
        "mfma_frac_layer": round(head["flops"] / (head["latency_us"] * 1e-6) / BF16_PEAK, 4),
        "roofline": {"kernel": "lsa_index_topk: score_stream_kernel<Flat, 5, 16384> (indexer scoring fused with "
                               "the first top-K level) + topk_level_kernel over the candidate lists",
                     "bound": "hbm", "achieved": round(head["select_gbs"], 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(head["select_gbs"] * 1e9 / HBM_PEAK, 4),
                     "traffic": measured_traffic() if head["L"] == TRAFFIC_L else None,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
