"""Parity at the workloads' full sizes, in the launch configuration the benchmark times.

The oracle cannot redo whole 1M-key rows in seconds, so these tests check sampled outputs it can
compute one by one (scores at sampled positions, whole rows at 128K, page scores and HI selection of
one sequence, attention of sampled rows) and properties that hold at any size (every planted needle
is picked; no sampled unpicked position beats a picked one beyond the near-tie band; idx ascending,
unique, inside mid(t)).  Oracle inputs are host copies of the generated inputs, never GPU results.
"""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_weighted_amd as lsa
import oracle as ref
import synth
from parity_util import (assert_attn_close, assert_idx_sets_match, assert_scores_close, f64, host, kth_best, log,
                         near_tie, rows_of)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_layer(x, idx_row=None, sb_off=None, k_mean=None, q=None, kv=None, idx=None, cfg=None):
    """One lsa_layer_fwd exactly as bench.py launches it (a configured Layer with its workspace)."""
    c = dict(x["cfg"]) if cfg is None else cfg
    n = x["row_pos"].numel()
    layer = lsa.Layer(c, rows_of(x), torch.bfloat16, DEV, use_hi=k_mean is not None)
    if idx is None:
        idx = torch.full((n, c["k_sparse"]), -1, dtype=torch.int32, device=DEV)
    out = torch.empty((n, c["H"], c["Dv"]), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((n, c["H"]), dtype=torch.float32, device=DEV)
    layer(x["q"] if q is None else q, x["kv"] if kv is None else kv, idx, out, lse, q_idx=x["q_idx"], w=x["w"],
          k_idx=x["k_idx"], idx_row=idx_row, sb_off=sb_off, k_mean=k_mean)
    torch.cuda.synchronize()
    return idx, out, lse


def seq_host(x, b, name):
    lo, hi = int(x["kv_off_host"][b]), int(x["kv_off_host"][b + 1])
    return host(x[name][lo:hi])


def one_row_oracle(x, r, b):
    """Oracle-convention inputs for a single row r of sequence b (sequence rebased to offset 0)."""
    L = x["lengths"][b]
    return dict(kv_off=np.array([0, L], np.int64), row_seq=np.zeros(1, np.int32),
                row_pos=np.array([int(x["row_pos_host"][r])], np.int32), q_idx=host(x["q_idx"][r:r + 1]),
                w=host(x["w"][r:r + 1]))


def check_idx_properties(g_idx, x, c):
    for r in range(g_idx.shape[0]):
        b = int(x["row_seq_host"][r])
        t = int(x["row_pos_host"][r])
        picks = g_idx[r][g_idx[r] >= 0]
        assert np.all(np.diff(picks) > 0)
        assert picks.size == 0 or (picks[0] >= c["k_sink"] and picks[-1] <= t - c["k_swa"])
        assert picks.size == min(c["k_sparse"], max(0, t - c["k_sink"] - c["k_swa"] + 1))


def check_sampled_selection(x, c, r, b, g_idx_row, rng, n_sample=4096):
    """Oracle scores of the picks and of random unpicked middle positions: no unpicked one may beat the
    weakest pick beyond the near-tie band (a property of any exact top-K of the oracle's scores)."""
    o = one_row_oracle(x, r, b)
    k_seq = seq_host(x, b, "k_idx")
    t = int(o["row_pos"][0])
    picks = g_idx_row[g_idx_row >= 0]
    mid = np.arange(c["k_sink"], t - c["k_swa"] + 1)
    others = np.setdiff1d(rng.choice(mid, min(n_sample, mid.size), replace=False), picks)
    sc = lambda pos: np.array([ref.score_one(o["q_idx"][0], o["w"][0], k_seq[s]) for s in pos])
    pick_sc = sc(picks)
    other_sc = sc(others)
    weakest = float(pick_sc.min())
    assert np.all(other_sc <= weakest + 1e-3 * abs(weakest)), (float(other_sc.max()), weakest)
    return weakest


# --------------------------------------------------------------------------------------------- decode


@pytest.mark.parametrize("L", [131072, 1048576])
def test_decode_batch32_full_size(L):
    log(f"decode batch 32 at L={L}")
    x = synth.decode_sweep(L, device=DEV)
    c = x["cfg"]
    idx, out, lse = run_layer(x)
    g_idx = host(idx)
    check_idx_properties(g_idx, x, c)
    for b, picks in enumerate(x["needles"]):
        assert set(picks) <= set(g_idx[b].tolist()), f"needles of sequence {b} not all picked"
    rng = np.random.default_rng(L)
    # scores at sampled positions of two rows (the same scoring launch the layer makes)
    scores = lsa.lsa_index_score(rows_of(x), x["q_idx"], x["w"], x["k_idx"], (16, 1024, 1024))
    for r in (0, 31):
        o = one_row_oracle(x, r, r)
        k_seq = seq_host(x, r, "k_idx")
        # mid(t) for t = L - 1 is [16, L - 1025]: sample it and its edges on both sides
        pos = np.concatenate([rng.integers(0, L, 2048), [0, 15, 16, L - 1026, L - 1025, L - 1024, L - 1]])
        got = host(scores[r])[pos]
        want = np.array([ref.score_one(o["q_idx"][0], o["w"][0], k_seq[s]) if 16 <= s <= L - 1025 else -np.inf
                         for s in pos], np.float32)
        assert_scores_close(got[None], want[None], f"scores row {r}")
    del scores
    # whole-row oracle selection for two rows, in the launch the benchmark times (at 1M the fused
    # scoring + first top-K level on 16384-column chunks; at 128K on 8192-column chunks): the oracle
    # scores every middle key of the two rows (two threads, one row each) and takes its own top-K
    two = (3, 17)
    k_two = np.concatenate([seq_host(x, r, "k_idx") for r in two])
    two_scores = ref.index_score(np.array([0, L, 2 * L], np.int64), np.array([0, 1], np.int32),
                                 np.array([L - 1, L - 1], np.int32), host(x["q_idx"][list(two)]),
                                 host(x["w"][list(two)]), k_two, 16, 1024, ld=L, threads=2)
    del k_two
    w_two = ref.topk(two_scores, 1024, threads=2)
    for i, r in enumerate(two):
        th = kth_best(two_scores[i], 1024)
        n_diff = assert_idx_sets_match(g_idx[r:r + 1], w_two[i:i + 1],
                                       lambda _, d: near_tie(two_scores[i][d], th))
        log(f"row {r}: whole-row oracle selection, {n_diff} rows with near-tie differences")
    del two_scores
    if L > 131072:
        for r in (5, 30):
            check_sampled_selection(x, c, r, r, g_idx[r], rng)
    # end-to-end attention of the layer call above: the oracle's attention on the GPU's own index rows
    for r in (0, 31):
        kv_seq = seq_host(x, r, "kv")
        wo, wl = ref.hybrid_attn(np.array([0, L], np.int64), [0], [L - 1], host(x["q"][r:r + 1]), kv_seq, 512,
                                 c["scale"], 16, 1024, g_idx[r:r + 1])
        assert_attn_close(host(out[r:r + 1]), wo, host(lse[r:r + 1]), wl, 2e-2, f"layer attention row {r}")
        del kv_seq
    # attention of two rows fed the same pick lists on both sides, in the 32-row launch
    picks = np.full((32, 1024), -1, np.int32)
    for r in range(32):
        picks[r] = np.sort(rng.choice(np.arange(16, L - 1040), 1024, replace=False))
    out2, lse2 = lsa.lsa_hybrid_attn(rows_of(x), x["q"], x["kv"], 512, c["scale"], (16, 1024, 1024),
                                     torch.from_numpy(picks).to(DEV))
    for r in (0, 19):
        kv_seq = seq_host(x, r, "kv")
        wo, wl = ref.hybrid_attn(np.array([0, L], np.int64), [0], [L - 1], host(x["q"][r:r + 1]), kv_seq, 512,
                                 c["scale"], 16, 1024, picks[r:r + 1])
        assert_attn_close(host(out2[r:r + 1]), wo, host(lse2[r:r + 1]), wl, 2e-2, f"attention row {r}")


@pytest.mark.parametrize("L", [131072, 1048576])
def test_fp8_decode_batch32_full_size(L):
    # The FP8 indexer on the decode batch as bench.py runs it: quantizer codes of sampled keys and of
    # whole query rows bit for bit, scores at sampled positions, and the selection built on them.
    from oracle import fp8
    log(f"FP8 decode batch 32 at L={L}")
    x = synth.decode_sweep(L, device=DEV)
    c = x["cfg"]
    rows = rows_of(x)
    k8, ks = lsa.lsa_quantize_fp8(x["k_idx"])
    q8, qs = lsa.lsa_quantize_fp8(x["q_idx"])
    rng = np.random.default_rng(L + 8)
    keys = rng.integers(0, 32 * L, 65536)
    wc, wsc = fp8.quantize(f64(host(x["k_idx"][torch.from_numpy(keys).to(DEV)])))
    assert np.array_equal(host(k8[torch.from_numpy(keys).to(DEV)]), wc)
    assert np.array_equal(host(ks[torch.from_numpy(keys).to(DEV)]), wsc)
    qc, qsc = fp8.quantize(f64(host(x["q_idx"])))
    assert np.array_equal(host(q8), qc) and np.array_equal(host(qs), qsc)
    scores = lsa.lsa_index_score_fp8(rows, q8, qs, x["w"], k8, ks, (16, 1024, 1024))
    for r in (0, 31):
        k_seq = seq_host(x, r, "k_idx")
        pos = np.concatenate([rng.integers(0, L, 2048), [0, 15, 16, L - 1026, L - 1025, L - 1024, L - 1]])
        kc, ksc = fp8.quantize(f64(k_seq[pos]))
        kd = fp8.dequantize(kc, ksc)
        qd = fp8.dequantize(qc[r], qsc[r])
        want = np.array([ref.score_one(qd, host(x["w"][r]), kd[i]) if 16 <= s <= L - 1025 else -np.inf
                         for i, s in enumerate(pos)], np.float32)
        assert_scores_close(host(scores[r])[pos][None], want[None], f"FP8 scores row {r}")
    g_idx = host(lsa.lsa_topk(scores, c["k_sparse"]))
    check_idx_properties(g_idx, x, c)
    for b, picks in enumerate(x["needles"]):
        assert set(picks) <= set(g_idx[b].tolist()), f"needles of sequence {b} not all picked under FP8"
    if L <= 131072:
        r = 9
        o = one_row_oracle(x, r, r)
        kc, ksc = fp8.quantize(f64(seq_host(x, r, "k_idx")))
        row_scores = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], fp8.dequantize(qc[r:r + 1], qsc[r:r + 1]),
                                     o["w"], fp8.dequantize(kc, ksc), 16, 1024, ld=L)
        w_idx = ref.topk(row_scores, 1024)
        th = kth_best(row_scores[0], 1024)
        assert_idx_sets_match(g_idx[r:r + 1], w_idx, lambda _, d: near_tie(row_scores[0][d], th))


def check_hi_row_against_oracle(x, r, b, g_idx_row, P=128, B=128, M=1024):
    """The oracle's own HI selection for row r (its own sub-block means, page recall, stage-2 scores,
    top-K) against the GPU's picks; differences only at token- or page-level near-ties."""
    L = x["lengths"][b]
    k_seq = seq_host(x, b, "k_idx")
    o = one_row_oracle(x, r, b)
    nsb = (L + B - 1) // B
    km_o = ref.page_means(np.array([0, L], np.int64), np.array([0, nsb], np.int64), k_seq, B)
    pages, ps = ref.page_recall(o["kv_off"], np.array([0, nsb], np.int64), o["row_seq"], o["row_pos"], o["q_idx"],
                                o["w"], km_o, P, B, M, ld=(L + P - 1) // P)
    comp = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], k_seq, 16, 1024, ld=M * P,
                           pages=pages, P=P)
    w_idx = ref.topk(comp, 1024, pages=pages, P=P)
    th, th_p = kth_best(comp[0], 1024), kth_best(ps[0], M)

    def accept(_, d):
        ok = near_tie(ps[0][d // P], th_p)
        sc = np.array([ref.score_one(o["q_idx"][0], o["w"][0], k_seq[s]) for s in d])
        return ok | near_tie(sc, th)
    return assert_idx_sets_match(g_idx_row[None], w_idx, accept), km_o


def test_hi_decode_1m_full_size():
    log("HI decode batch 8 at L=1M")
    x = synth.hi_decode(device=DEV)
    c = x["cfg"]
    L, P, B, M = 1 << 20, 128, 128, 1024
    sb_off = lsa.sb_offsets(x["lengths"], B)
    km = lsa.lsa_page_means(x["kv_off"], sb_off.to(DEV), x["k_idx"], B, L)
    idx, out, lse = run_layer(x, sb_off=sb_off.to(DEV), k_mean=km)
    g_idx = host(idx)
    check_idx_properties(g_idx, x, c)
    rng = np.random.default_rng(3)
    b = 2
    k_seq = seq_host(x, b, "k_idx")
    # sub-block means of sequence b: bit-exact at sampled sub-blocks
    km_b = host(km[int(sb_off[b]):int(sb_off[b + 1])])
    for n_sb in rng.integers(0, L // B, 64):
        want = ref.page_means(np.array([0, B], np.int64), np.array([0, 1], np.int64), k_seq[n_sb * B:(n_sb + 1) * B],
                              B)
        assert np.array_equal(km_b[n_sb], want[0])
    # the oracle's own HI selection for row b, from its own means
    n_diff, km_o = check_hi_row_against_oracle(x, b, b, g_idx[b])
    assert np.array_equal(km_o, km_b)
    log(f"HI row {b}: {'differs only at near-ties' if n_diff else 'identical to the oracle'}")
    hits = sum(len(set(p) & set(g_idx[i].tolist())) for i, p in enumerate(x["needles"]))
    log(f"HI needle recall {hits}/{sum(len(p) for p in x['needles'])}")


# --------------------------------------------------------------------------------------------- prefill + CLI


def test_chunked_prefill_cli_full_size():
    log("chunked prefill 8192 x 139264 with a CLI reuse layer")
    x = synth.chunked_prefill_cli(device=DEV)
    c = x["cfg"]
    (q1, kv1), (q2, kv2) = x["layers"]
    idx, out, lse = run_layer(x, q=q1, kv=kv1)
    _, out_r, lse_r = run_layer(x, q=q2, kv=kv2, idx=idx.clone(), cfg=dict(c, is_owner=0))
    g_idx = host(idx)
    L = x["max_len"]
    rows = [0, 1, 4095, 8191]
    k_all = host(x["k_idx"])
    w_sets = {}
    for r in rows:
        o = dict(kv_off=np.array([0, L], np.int64), row_seq=np.zeros(1, np.int32),
                 row_pos=np.array([int(x["row_pos_host"][r])], np.int32), q_idx=host(x["q_idx"][r:r + 1]),
                 w=host(x["w"][r:r + 1]))
        row_scores = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], k_all, 16, 1024,
                                     ld=L)
        w_idx = ref.topk(row_scores, 1024)
        th = kth_best(row_scores[0], 1024)
        assert_idx_sets_match(g_idx[r:r + 1], w_idx, lambda _, d: near_tie(row_scores[0][d], th))
        w_sets[r] = w_idx[0]
    # attention (owner and reuse) of the sampled rows with the oracle's sets, in the 8192-row launch
    picks = g_idx.copy()
    for r in rows:
        picks[r] = w_sets[r]
    pk = torch.from_numpy(picks).to(DEV)
    kv1_h, kv2_h = host(kv1), host(kv2)
    for q_l, kv_l, kv_h in ((q1, kv1, kv1_h), (q2, kv2, kv2_h)):
        o2, l2 = lsa.lsa_hybrid_attn(rows_of(x), q_l, kv_l, 512, c["scale"], (16, 1024, 1024), pk)
        for r in rows:
            wo, wl = ref.hybrid_attn(np.array([0, L], np.int64), [0], [int(x["row_pos_host"][r])],
                                     host(q_l[r:r + 1]), kv_h, 512, c["scale"], 16, 1024, picks[r:r + 1])
            assert_attn_close(host(o2[r:r + 1]), wo, host(l2[r:r + 1]), wl, 2e-2, f"prefill attention row {r}")
    # the reuse layer with the owner's index set equals a direct attention call with it
    o3, l3 = lsa.lsa_hybrid_attn(rows_of(x), q2, kv2, 512, c["scale"], (16, 1024, 1024), idx)
    assert torch.equal(o3.view(torch.int16), out_r.view(torch.int16)) and torch.equal(l3, lse_r)


# --------------------------------------------------------------------------------------------- ragged MTP


def test_ragged_mtp_full_size():
    log("ragged MTP decode, 64 sequences x 3 drafts")
    x = synth.ragged_mtp(device=DEV)
    c = x["cfg"]
    lengths = x["lengths"]
    sb_off = lsa.sb_offsets(lengths, 128)
    km = lsa.lsa_page_means(x["kv_off"], sb_off.to(DEV), x["k_idx"], 128, x["max_len"])
    idx, out, lse = run_layer(x, idx_row=x["idx_row"], sb_off=sb_off.to(DEV), k_mean=km)
    g_idx = host(idx)
    owners = np.arange(0, 192, 3)
    check_idx_properties(g_idx[owners], dict(x, row_seq_host=x["row_seq_host"][owners],
                                              row_pos_host=x["row_pos_host"][owners]), c)
    assert np.all(g_idx[np.setdiff1d(np.arange(192), owners)] == -1)
    rng = np.random.default_rng(11)
    flat_b = [b for b in range(64) if lengths[b] < 262144]
    hi_b = [b for b in range(64) if lengths[b] >= 262144]
    log(f"{len(hi_b)} sequences take the HI path")
    for b in flat_b[:2]:
        r = 3 * b
        o = one_row_oracle(x, r, b)
        k_seq = seq_host(x, b, "k_idx")
        row_scores = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], k_seq, 16, 1024,
                                     ld=lengths[b])
        w_idx = ref.topk(row_scores, 1024)
        th = kth_best(row_scores[0], 1024)
        assert_idx_sets_match(g_idx[r:r + 1], w_idx, lambda _, d: near_tie(row_scores[0][d], th))
    for b in hi_b[:1]:
        check_hi_row_against_oracle(x, 3 * b, b, g_idx[3 * b])
    # drafts attend with their owner's set: a seeded pick list per owner row, given to both sides, in
    # the 192-row launch with idx_row mapping every draft to its owner
    picks = np.full((192, 1024), -1, np.int32)
    for b in range(64):
        L = lengths[b]
        picks[3 * b] = np.sort(rng.choice(np.arange(16, L - 1040), 1024, replace=False))
    o2, l2 = lsa.lsa_hybrid_attn(rows_of(x), x["q"], x["kv"], 512, c["scale"], (16, 1024, 1024),
                                 torch.from_numpy(picks).to(DEV), idx_row=x["idx_row"])
    for b in (flat_b[0], (hi_b or flat_b)[0]):
        L = lengths[b]
        kv_seq = seq_host(x, b, "kv")
        for r in (3 * b, 3 * b + 2):
            wo, wl = ref.hybrid_attn(np.array([0, L], np.int64), [0], [L - 1], host(x["q"][r:r + 1]), kv_seq, 512,
                                     c["scale"], 16, 1024, picks[3 * b:3 * b + 1])
            assert_attn_close(host(o2[r:r + 1]), wo, host(l2[r:r + 1]), wl, 2e-2, f"draft row {r}")
    # and the layer's drafts equal a direct attention call on the layer's own index sets
    o3, l3 = lsa.lsa_hybrid_attn(rows_of(x), x["q"], x["kv"], 512, c["scale"], (16, 1024, 1024), idx,
                                 idx_row=x["idx_row"])
    assert torch.equal(o3.view(torch.int16), out.view(torch.int16)) and torch.equal(l3, lse)


# --------------------------------------------------------------------------------------------- HI prefill


def test_hi_prefill_stage2_256k_full_size():
    # HI stage 2 of the 2048-row prefill chunk at 256K as the benchmark times it (M = 1024 recalled pages
    # of 128 tokens per row: the multi-row kernel over recalled pages).  The recall lists are seeded on
    # the host, overlapping within each 16-row group as a chunk's lists do (1024 of a pool of 1536 of the
    # row's middle pages); the oracle scores sampled rows on the same lists, then the token top-K of those
    # rows is checked against the oracle's whole-row selection.
    L, q_len, P, M, K = 262144, 2048, 128, 1024, 1024
    x = synth.hi_prefill(L, device=DEV)
    c = x["cfg"]
    rows = lsa.RowsDesc(x["kv_off"], x["row_seq"], x["row_pos"], x["max_len"], L)
    rng = np.random.default_rng(21)
    pos = host(x["row_pos"]).astype(np.int64)
    pages = np.empty((q_len, M), np.int32)
    for g0 in range(0, q_len, 16):
        last = (pos[g0] - c["k_swa"]) // P  # pages with middle tokens for every row of the group
        pool = rng.choice(np.arange(0, last + 1), 1536, replace=False)
        for r in range(g0, g0 + 16):
            pages[r] = np.sort(rng.choice(pool, M, replace=False))  # (lsa_topk takes ascending lists)
    pg = torch.from_numpy(pages).to(DEV)
    bud = (c["k_sink"], c["k_swa"], K)
    comp = lsa.lsa_index_score(rows, x["q_idx"], x["w"], x["k_idx"], bud, pages=pg, M=M, P=P)
    idx = lsa.lsa_topk(comp, K, pages=pg, P=P)
    torch.cuda.synchronize()
    sample = [0, 777, 1500, 2047]
    k_seq = seq_host(x, 0, "k_idx")
    o = dict(kv_off=np.array([0, L], np.int64), row_seq=np.zeros(len(sample), np.int32),
             row_pos=pos[sample].astype(np.int32), q_idx=host(x["q_idx"][sample]), w=host(x["w"][sample]))
    want = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], k_seq, c["k_sink"],
                           c["k_swa"], ld=M * P, pages=pages[sample], P=P)
    got = host(comp)[sample]
    log("HI stage-2 scores (sampled rows) worst err/tol", assert_scores_close(got, want))
    w_idx = ref.topk(want, K, pages=pages[sample], P=P)
    g_idx = host(idx)[sample]
    for i in range(len(sample)):
        th = kth_best(want[i], K)
        slot = np.full(-(-L // P), -1, np.int64)
        slot[pages[sample[i]]] = np.arange(M)
        score_at = lambda d: want[i][slot[d // P] * P + d % P]  # oracle score of token position d
        assert_idx_sets_match(g_idx[i:i + 1], w_idx[i:i + 1], lambda _, d: near_tie(score_at(np.asarray(d)), th))
