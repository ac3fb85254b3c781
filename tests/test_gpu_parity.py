"""GPU parity of every hot-path step against the CPU oracle, through the C ABI (small and ragged
shapes that still span several tiles, plus the edge cases of the method)."""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_weighted_amd as lsa
import oracle as ref
import synth
from parity_util import (assert_attn_close, assert_idx_sets_match, assert_scores_close, budget_of, f64, host,
                         kth_best, log, near_tie, oracle_inputs, rows_of)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def custom_rows(lengths, rows, *, HI=64, dI=128, H=128, dtype=torch.bfloat16, seed=0, k_sink=16, k_swa=1024,
                k_sparse=1024, attn=True):
    """Sequences of the given lengths and explicit query rows (seq, t) with seeded Gaussian inputs."""
    g = synth.generator(seed, DEV)
    kv_off = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64)
    tot = int(kv_off[-1])
    n = len(rows)
    row_seq = torch.tensor([r[0] for r in rows], dtype=torch.int32)
    row_pos = torch.tensor([r[1] for r in rows], dtype=torch.int32)
    x = dict(kv_off=kv_off.to(DEV), kv_off_host=kv_off, row_seq=row_seq.to(DEV), row_seq_host=row_seq,
             row_pos=row_pos.to(DEV), row_pos_host=row_pos, max_len=max(lengths), lengths=list(lengths))
    x["q_idx"] = synth.normal((n, HI, dI), 1 / math.sqrt(dI), g, DEV, dtype)
    x["w"] = synth.softplus_normal((n, HI), g, DEV)
    x["k_idx"] = synth.normal((max(tot, 1), dI), 1 / math.sqrt(dI), g, DEV, dtype)
    if attn:
        x["q"] = synth.normal((n, H, 576), 1.0, g, DEV, dtype)
        x["kv"] = synth.normal((max(tot, 1), 576), 1.0, g, DEV, dtype)
    x["cfg"] = dict(HI=HI, dI=dI, H=H, Dqk=576, Dv=512, scale=1 / math.sqrt(576), k_sink=k_sink, k_swa=k_swa,
                    k_sparse=k_sparse, P=128, B=128, M=1024, hi_min_len=1 << 62, is_owner=1)
    return x


RAGGED_LENGTHS = [1, 17, 1041, 1042, 3001, 6000]
RAGGED_ROWS = [(0, 0), (1, 16), (1, 5), (2, 1040), (2, 1039), (3, 1041), (3, 1000), (4, 3000), (4, 2048),
               (5, 5999), (5, 4321), (5, 6000)]  # the last row is outside its sequence (t == L)


# --------------------------------------------------------------------------------------------- a2 scores


def test_index_score_fp32_tiny_prefill():
    x = synth.tiny_prefill(device=DEV)
    o = oracle_inputs(x)
    c = x["cfg"]
    g = lsa.lsa_index_score(rows_of(x), x["q_idx"], x["w"], x["k_idx"], budget_of(c))
    want = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"], c["k_sink"],
                           c["k_swa"], ld=2048)
    log("fp32 scores worst err/tol", assert_scores_close(host(g), want))


def test_index_score_bf16_ragged_and_edges():
    x = custom_rows(RAGGED_LENGTHS, RAGGED_ROWS, attn=False)
    o = oracle_inputs(x)
    c = x["cfg"]
    ld = x["max_len"] + 37
    g = lsa.lsa_index_score(rows_of(x), x["q_idx"], x["w"], x["k_idx"], budget_of(c), ld=ld)
    want = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"], c["k_sink"],
                           c["k_swa"], ld=ld)
    log("bf16 scores worst err/tol", assert_scores_close(host(g), want))
    assert np.all(np.isneginf(host(g)[-1]))  # a row outside its sequence scores nothing


# Rows that exercise the multi-row (prefill) scoring kernel: groups of 16 rows of one sequence are
# scored together, other groups row by row.  Groups: 0 uniform; 1 uniform with empty and edge mid
# regions; 2 alternating sequences; 3 uniform in the second sequence; 4 uniform in a sequence too
# short for any mid region; 5 with one row outside its sequence; 6 whose first row lies outside another
# sequence; 7 with every row outside its sequence; then a partial group of 5 rows.
GROUPED_LENGTHS = [6000, 3000, 700]
GROUPED_ROWS = ([(0, t) for t in range(5984, 6000)]
                + [(0, t) for t in (0, 1, 15, 16, 1039, 1040, 1041, 1042, 2000, 2001, 3000, 4500, 5999, 5998, 100,
                                    3333)]
                + [((0, 5000 + i) if i % 2 == 0 else (1, 2900 - 7 * i)) for i in range(16)]
                + [(1, t) for t in range(2984, 3000)]
                + [(2, t) for t in range(684, 700)]
                + [(0, t) for t in range(3000, 3015)] + [(0, 6000)]
                + [(1, 3000)] + [(0, t) for t in range(4100, 4115)]
                + [(2, 700 + 3 * i) for i in range(16)]
                + [(0, t) for t in range(4000, 4005)])
# One sequence in whole groups (every group is scored by the multi-row kernel, no per-row launch), with
# rows outside the sequence (t >= L) inside the groups and a group of them only.
SINGLE_SEQ_ROWS = ([(0, t) for t in range(4900, 4916)] + [(0, 5000 + t if t % 5 == 0 else 4800 + t) for t in range(16)]
                   + [(0, 5000 + t) for t in range(16)] + [(0, t) for t in range(1030, 1046)])


def test_index_score_bf16_grouped_rows():
    x = custom_rows(GROUPED_LENGTHS, GROUPED_ROWS, attn=False, seed=31)
    o = oracle_inputs(x)
    c = x["cfg"]
    ld = x["max_len"] + 37
    g = lsa.lsa_index_score(rows_of(x), x["q_idx"], x["w"], x["k_idx"], budget_of(c), ld=ld)
    want = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"], c["k_sink"],
                           c["k_swa"], ld=ld)
    log("grouped bf16 scores worst err/tol", assert_scores_close(host(g), want))
    assert np.all(np.isneginf(host(g)[64:80]))   # L = 700: no mid region anywhere


def test_index_score_bf16_single_sequence_groups():
    x = custom_rows([5000], SINGLE_SEQ_ROWS, attn=False, seed=33)
    o = oracle_inputs(x)
    c = x["cfg"]
    g = lsa.lsa_index_score(rows_of(x), x["q_idx"], x["w"], x["k_idx"], budget_of(c))
    want = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"], c["k_sink"],
                           c["k_swa"], ld=5000)
    log("single-sequence groups worst err/tol", assert_scores_close(host(g), want))
    assert np.all(np.isneginf(host(g)[32:48]))   # rows past the sequence: no scores


def test_layer_bf16_grouped_rows():
    x = custom_rows(GROUPED_LENGTHS, GROUPED_ROWS, seed=32)
    o = oracle_inputs(x)
    c = x["cfg"]
    idx, out, lse = lsa.lsa_layer_fwd(c, rows_of(x), x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"])
    w_idx, w_out, w_lse = ref.layer_fwd(c, o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"],
                                        o["q"], o["kv"])
    _compare_layer(o, c, host(idx), host(out), host(lse), w_idx, w_out, w_lse, 2e-2, OracleRanking(o, c))


@pytest.mark.parametrize("P", [128, 48])  # 48: a page size that is not a power of two (division path)
def test_index_score_bf16_page_mapped(P):
    L = 9000
    x = custom_rows([L, 4000], [(0, L - 1), (0, 5000), (1, 3999)], attn=False)
    o = oracle_inputs(x)
    c = x["cfg"]
    M = 12
    pages = np.full((3, M), -1, np.int32)
    # (for P = 128: 70 is the partial last page of L = 9000, 31 straddles the end of mid(5000), 39 lies
    # beyond t = 5000 and 31 beyond L = 4000; for P = 48 the same page numbers cover other tokens)
    pages[0, :10] = [0, 1, 7, 8, 30, 31, 55, 60, 69, 70]
    pages[1, :6] = [3, 9, 20, 30, 31, 39]
    pages[2, :5] = [0, 5, 10, 23, 31]
    pg = torch.from_numpy(pages).to(DEV)
    g = lsa.lsa_index_score(rows_of(x), x["q_idx"], x["w"], x["k_idx"], budget_of(c), pages=pg, P=P, ld=M * P + 5)
    want = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"], c["k_sink"],
                           c["k_swa"], ld=M * P + 5, pages=pages, P=P)
    log("paged scores worst err/tol", assert_scores_close(host(g), want))


@pytest.mark.parametrize("tail", [False, True])
def test_index_score_bf16_page_mapped_grouped_rows(tail):
    # Prefill-like batches (at least 16 rows per sequence) take the multi-row kernel over recalled pages:
    # a group's recalled pages are streamed once and each row scores its own.  The lists overlap
    # heavily (drawn from a small pool) and hold -1 padding, a page listed twice, pages past the
    # sequence, the partial last page and pages straddling the end of mid(t); sequence 0 spans two
    # page ranges of the kernel (266 pages).  Row 3 lies outside its sequence (t = L), and the rows
    # of one group mix the two sequences, so the per-row kernel scores that group.  With a tail the
    # batch is not whole groups (the last 8 rows go to the per-row kernel too).
    rng = np.random.default_rng(5)
    L0, L1 = 34000, 9000
    t0 = sorted(rng.integers(26000, L0, 39).tolist())
    t1 = sorted(rng.integers(3000, L1, 32 if tail else 40).tolist())
    rows = [(0, t) for t in t0[:3]] + [(0, L0)] + [(0, t) for t in t0[3:]] + [(1, t) for t in t1]
    x = custom_rows([L0, L1], rows, attn=False, seed=3)
    o = oracle_inputs(x)
    c = x["cfg"]
    P, M = 128, 48  # (the multi-row kernel takes recall lists covering at least a sixth of the sequence)
    n = len(rows)
    pages = np.full((n, M), -1, np.int32)
    for i, (sq, t) in enumerate(rows):
        n_pages = -(-(L0 if sq == 0 else L1) // P)
        pool = rng.choice(n_pages, 70, replace=False)
        k = int(rng.integers(M - 6, M + 1))
        pick = rng.choice(pool, k, replace=False)
        pages[i, :k] = pick
        if i % 5 == 0:
            pages[i, M - 1] = pages[i, 0]        # listed twice
        if i % 7 == 0:
            pages[i, M - 2] = n_pages + 2        # past the sequence
        if i % 3 == 0:
            pages[i, 1] = n_pages - 1            # the partial last page
            pages[i, 2] = (t - 1024) // P        # straddles the end of mid(t)
    pg = torch.from_numpy(pages).to(DEV)
    ld = M * P + 5
    g = lsa.lsa_index_score(rows_of(x), x["q_idx"], x["w"], x["k_idx"], budget_of(c), pages=pg, P=P, ld=ld)
    want = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"], c["k_sink"],
                           c["k_swa"], ld=ld, pages=pages, P=P)
    log("grouped paged scores worst err/tol", assert_scores_close(host(g), want))


def test_index_score_bf16_page_mapped_grouped_short_rows():
    # Four short sequences of 16 rows each (every group uniform): rows with an empty middle range
    # (t < k_sink + k_swa), rows just past it, a row outside its sequence, M = 4 recalled pages of 128
    # (lists of -1 only, pages past the sequence, the same page twice), ld = M P exactly.
    rng = np.random.default_rng(8)
    lengths = [1100, 2000, 2900, 3000]
    rows = []
    for b, L in enumerate(lengths):
        ts = [0, 15, 16, 1039, 1040, 1041, L - 1, L] + sorted(rng.integers(1, L, 8).tolist())
        rows += [(b, int(t)) for t in ts]
    x = custom_rows(lengths, rows, attn=False, seed=6)
    o = oracle_inputs(x)
    c = x["cfg"]
    P, M = 128, 4
    pages = np.full((len(rows), M), -1, np.int32)
    for i, (b, t) in enumerate(rows):
        n_pages = -(-lengths[b] // P)
        if i % 9 == 4:
            continue  # an empty list
        pages[i] = rng.choice(n_pages + 2, M, replace=False)
        if i % 5 == 1:
            pages[i, 3] = pages[i, 0]
    pg = torch.from_numpy(pages).to(DEV)
    g = lsa.lsa_index_score(rows_of(x), x["q_idx"], x["w"], x["k_idx"], budget_of(c), pages=pg, P=P, ld=M * P)
    want = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"], c["k_sink"],
                           c["k_swa"], ld=M * P, pages=pages, P=P)
    log("grouped paged scores, short rows: worst err/tol", assert_scores_close(host(g), want))


# --------------------------------------------------------------------------------------------- a7 top-K


def _score_rows(rng, n_rows, n_cols, kind):
    if kind == "gauss":
        s = rng.standard_normal((n_rows, n_cols)).astype(np.float32)
    elif kind == "ties":
        s = rng.choice(np.array([-2.0, -0.0, 0.0, 0.5, 1.0, 3.0, np.inf], np.float32), (n_rows, n_cols))
    elif kind == "equal":
        s = np.full((n_rows, n_cols), 0.75, np.float32)
    elif kind.startswith("pos"):  # positive, over two binades like indexer scores (optionally quantised):
        # the first digit pass leaves a small bin of several values, with ties when quantised
        s = (1.0 + 3.0 * rng.random((n_rows, n_cols))).astype(np.float32)
        if kind != "pos":
            step = int(kind[3:])
            s = (np.round(s * step) / step).astype(np.float32)
    elif kind.startswith("fine"):  # finely quantised: a few equal keys per value, also near the threshold
        step = int(kind[4:])
        s = (np.round(rng.standard_normal((n_rows, n_cols)) * step) / step).astype(np.float32)
    else:  # coarse quantised values: many ties at the threshold
        s = (rng.integers(-50, 50, (n_rows, n_cols)) / 8.0).astype(np.float32)
    s[rng.random((n_rows, n_cols)) < 0.1] = -np.inf
    return s


@pytest.mark.parametrize("n_rows,n_cols,K,kind", [
    (3, 1, 1, "gauss"), (5, 100, 7, "gauss"), (4, 100, 200, "ties"), (4, 5000, 1024, "gauss"),
    (4, 5000, 1024, "ties"), (3, 20000, 1024, "quant"), (2, 70000, 1024, "equal"), (1, 4096, 4096, "quant"),
    (64, 3000, 112, "gauss"), (2, 300000, 1024, "quant"), (3, 8192, 1024, "quant"), (2, 8193, 1024, "gauss"),
    (2, 8192, 4096, "ties"), (4, 16384, 1024, "fine256"), (4, 16384, 1024, "fine2048"), (2, 70000, 1024, "fine256"),
    (3, 5000, 100, "fine2048"), (2, 300000, 1024, "fine4096"), (6, 16384, 1024, "pos"), (6, 16384, 1024, "pos4096"),
    (4, 8192, 1024, "pos8192"), (3, 70000, 1024, "pos4096"), (2, 300000, 1024, "pos8192"), (4, 5000, 37, "pos4096")])
def test_topk_bit_exact_on_oracle_style_scores(n_rows, n_cols, K, kind):
    rng = np.random.default_rng(n_rows * 7919 + n_cols + K)
    s = _score_rows(rng, n_rows, n_cols, kind)
    s[0, : min(5, n_cols)] = -np.inf
    want = ref.topk(s, K)
    got = host(lsa.lsa_topk(torch.from_numpy(s).to(DEV), K))
    assert np.array_equal(got, want), f"first differing row {np.argwhere((got != want).any(1))[:3].ravel()}"


def test_topk_negative_zero_and_all_neg_inf_rows():
    s = np.array([[0.0, -0.0, 0.0, -0.0, -1.0], [-np.inf] * 5, [-0.0, -np.inf, 0.0, -np.inf, -0.0]], np.float32)
    got = host(lsa.lsa_topk(torch.from_numpy(s).to(DEV), 3))
    assert np.array_equal(got, ref.topk(s, 3))
    assert list(got[1]) == [-1, -1, -1]


@pytest.mark.parametrize("P", [128, 48])
def test_topk_page_mapped_bit_exact(P):
    rng = np.random.default_rng(5)
    M = 40
    s = _score_rows(rng, 6, M * P, "quant")
    pages = np.sort(rng.choice(5000, (6, M), replace=False), axis=1).astype(np.int32)
    pages[:, -3:] = -1
    s[:, -3 * P:] = -np.inf
    s[2, 5 * P:6 * P] = 1.0   # a filled slot of a valid page with ties
    want = ref.topk(s, 1024, pages=pages, P=P)
    got = host(lsa.lsa_topk(torch.from_numpy(s).to(DEV), 1024, pages=torch.from_numpy(pages).to(DEV), P=P))
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------------------------- a3 means


@pytest.mark.parametrize("dtype,B", [(torch.bfloat16, 128), (torch.bfloat16, 8), (torch.float32, 16)])
def test_page_means_bit_exact(dtype, B):
    lengths = [1, 127, 128, 129, 5000]
    g = synth.generator(3, DEV)
    kv_off = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64)
    k = synth.normal((int(kv_off[-1]), 128), 1 / math.sqrt(128), g, DEV, dtype)
    sb_off = lsa.sb_offsets(lengths, B)
    got = lsa.lsa_page_means(kv_off.to(DEV), sb_off.to(DEV), k, B, max(lengths))
    want = ref.page_means(kv_off.numpy(), sb_off.numpy(), host(k), B)
    assert np.array_equal(host(got), want)
    # incremental rebuild from token 4000 on: the rows it touches equal a full rebuild
    k[kv_off[4] + 4000:] *= 2
    got2 = lsa.lsa_page_means(kv_off.to(DEV), sb_off.to(DEV), k, B, max(lengths), k_mean=got.clone(),
                              first_token=4000)
    want2 = ref.page_means(kv_off.numpy(), sb_off.numpy(), host(k), B)
    assert np.array_equal(host(got2), want2)


@pytest.mark.parametrize("dtype,B,n_new", [(torch.bfloat16, 8, 1), (torch.bfloat16, 8, 20), (torch.bfloat16, 128, 1),
                                           (torch.float32, 16, 3)])
def test_page_means_append_bit_exact(dtype, B, n_new):
    # A decode step appended n_new tokens to every sequence: the sub-blocks holding them are rebuilt to
    # the oracle's full-cache means; every other row of the cache is left as it was (here a sentinel).
    lengths = [1, 8, 9, 127, 128, 129, 4999, 70000]
    g = synth.generator(5, DEV)
    kv_off = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64)
    k = synth.normal((int(kv_off[-1]), 128), 1 / math.sqrt(128), g, DEV, dtype)
    sb_off = lsa.sb_offsets(lengths, B)
    want = ref.page_means(kv_off.numpy(), sb_off.numpy(), host(k), B)
    touched = np.zeros(len(want), bool)
    for b, L in enumerate(lengths):
        first = max(L - n_new, 0)
        touched[int(sb_off[b]) + first // B:int(sb_off[b + 1])] = True
    stale = np.where(touched[:, None], np.zeros_like(want) + 7, np.zeros_like(want)).astype(want.dtype)
    km = (synth.bits_to_bf16(stale) if dtype == torch.bfloat16 else torch.from_numpy(stale)).to(DEV)
    lsa.lsa_page_means_append(kv_off.to(DEV), sb_off.to(DEV), k, B, km, n_new=n_new)
    got = host(km)
    assert np.array_equal(got[touched], want[touched])
    assert np.array_equal(got[~touched], stale[~touched])


# --------------------------------------------------------------------------------------------- a4/a5 HI


@pytest.mark.parametrize("B", [128, 8])
def test_page_recall_scores_and_pages(B):
    lengths = [70000, 20000, 130]
    rows = [(0, 69999), (1, 19999), (0, 40000), (2, 129)]
    x = custom_rows(lengths, rows, attn=False, seed=11)
    o = oracle_inputs(x)
    P, M = 128, 64
    sb_off = lsa.sb_offsets(lengths, B)
    km_o = ref.page_means(o["kv_off"], sb_off.numpy(), o["k_idx"], B)
    km = synth.bits_to_bf16(km_o).to(DEV)             # both sides read the oracle's cache
    ld = (max(lengths) + P - 1) // P
    ps = torch.empty((len(rows), ld), dtype=torch.float32, device=DEV)
    pages, _ = lsa.lsa_page_recall(rows_of(x), sb_off.to(DEV), x["q_idx"], x["w"], km, P, B, M, page_scores=ps)
    want_ps = ref.page_scores(o["kv_off"], sb_off.numpy(), o["row_seq"], o["row_pos"], o["q_idx"], o["w"], km_o, P,
                              B, ld)
    log("page scores worst err/tol", assert_scores_close(host(ps), want_ps, "page scores"))
    want_pages = ref.topk(want_ps, M)

    assert_idx_sets_match(host(pages), want_pages, lambda r, d: near_tie(want_ps[r, d], kth_best(want_ps[r], M)),
                          what="pages")
    # fed the oracle's page scores, the selection is bit-exact
    got = host(lsa.lsa_topk(torch.from_numpy(want_ps).to(DEV), M))
    assert np.array_equal(got, want_pages)


# Rows for the multi-row page scoring: groups of 16 rows of one sequence (a prefill chunk crossing
# page edges, one group straddling the end of a partial last page), then rows scored one by one.
PM_LENGTHS = [20100, 9000]
PM_ROWS = ([(0, t) for t in range(19940, 20004)]          # 4 uniform groups over the page edge at 19968
           + [(0, t) for t in range(20084, 20100)]        # a group ending in the partial last page
           + [(1, 9000)] + [(0, t) for t in range(20000, 20015)]  # first row outside its (other) sequence
           + [(1, 8999), (0, 5000), (1, 4000), (0, 20099), (1, 127), (0, 0), (1, 200)])


@pytest.mark.parametrize("B", [8, 128])
def test_page_scores_single_sequence_groups(B):
    # one sequence in whole groups: no per-row launch; rows past the sequence come out all -inf
    L = 20100
    rows = [(0, t) for t in range(19940, 19988)] + [(0, L + t if t % 4 == 0 else 19900 + t) for t in range(16)]
    x = custom_rows([L], rows, attn=False, seed=14)
    o = oracle_inputs(x)
    P, M = 128, 40
    sb_off = lsa.sb_offsets([L], B)
    km_o = ref.page_means(o["kv_off"], sb_off.numpy(), o["k_idx"], B)
    km = synth.bits_to_bf16(km_o).to(DEV)
    ld = (L + P - 1) // P + 3
    ps = torch.empty((len(rows), ld), dtype=torch.float32, device=DEV)
    lsa.lsa_page_recall(rows_of(x), sb_off.to(DEV), x["q_idx"], x["w"], km, P, B, M, page_scores=ps)
    want_ps = ref.page_scores(o["kv_off"], sb_off.numpy(), o["row_seq"], o["row_pos"], o["q_idx"], o["w"], km_o, P,
                              B, ld)
    log("single-sequence page scores worst err/tol", assert_scores_close(host(ps), want_ps, "page scores"))


@pytest.mark.parametrize("B", [8, 128, 32])
def test_page_scores_grouped_rows(B):
    x = custom_rows(PM_LENGTHS, PM_ROWS, attn=False, seed=13)
    o = oracle_inputs(x)
    P, M = 128, 40
    sb_off = lsa.sb_offsets(PM_LENGTHS, B)
    km_o = ref.page_means(o["kv_off"], sb_off.numpy(), o["k_idx"], B)
    km = synth.bits_to_bf16(km_o).to(DEV)
    ld = (max(PM_LENGTHS) + P - 1) // P + 3
    ps = torch.empty((len(PM_ROWS), ld), dtype=torch.float32, device=DEV)
    pages, _ = lsa.lsa_page_recall(rows_of(x), sb_off.to(DEV), x["q_idx"], x["w"], km, P, B, M, page_scores=ps)
    want_ps = ref.page_scores(o["kv_off"], sb_off.numpy(), o["row_seq"], o["row_pos"], o["q_idx"], o["w"], km_o, P,
                              B, ld)
    log("grouped page scores worst err/tol", assert_scores_close(host(ps), want_ps, "page scores"))
    want_pages = ref.topk(want_ps, M)
    assert_idx_sets_match(host(pages), want_pages, lambda r, d: near_tie(want_ps[r, d], kth_best(want_ps[r], M)),
                          what="pages")


# --------------------------------------------------------------------------------------------- a8-a10 attention


def _oracle_idx_for(x, k_sparse, rng):
    """A valid ascending pick list per row drawn from mid(t) (what an indexer could return)."""
    c = x["cfg"]
    out = np.full((len(x["row_pos_host"]), k_sparse), -1, np.int32)
    for r, (b, t) in enumerate(zip(x["row_seq_host"].tolist(), x["row_pos_host"].tolist())):
        L = x["lengths"][b]
        if t < 0 or t >= L:
            continue
        lo, hi = c["k_sink"], t - c["k_swa"] + 1
        if hi > lo:
            pick = np.sort(rng.choice(np.arange(lo, hi), min(k_sparse, hi - lo), replace=False))
            out[r, :len(pick)] = pick
    return out


def test_attention_fp32_tiny_prefill_shape():
    x = synth.tiny_prefill(device=DEV)
    o = oracle_inputs(x)
    c = x["cfg"]
    rng = np.random.default_rng(1)
    rows_sel = np.array([0, 1, 15, 16, 143, 144, 145, 300, 1023, 2047])
    sub = {k: x[k][rows_sel] for k in ("q",)}
    rs = torch.from_numpy(np.zeros(len(rows_sel), np.int32)).to(DEV)
    rp = torch.from_numpy(rows_sel.astype(np.int32)).to(DEV)
    rows = lsa.RowsDesc(x["kv_off"], rs, rp, 2048)
    xs = dict(cfg=c, row_seq_host=torch.zeros(len(rows_sel), dtype=torch.int32),
              row_pos_host=torch.from_numpy(rows_sel.astype(np.int32)), lengths=[2048])
    idx = _oracle_idx_for(xs, c["k_sparse"], rng)
    out, lse = lsa.lsa_hybrid_attn(rows, sub["q"], x["kv"], 512, c["scale"], budget_of(c),
                                   torch.from_numpy(idx).to(DEV))
    want_o, want_l = ref.hybrid_attn(o["kv_off"], np.zeros(len(rows_sel)), rows_sel, o["q"][rows_sel], o["kv"], 512,
                                     c["scale"], c["k_sink"], c["k_swa"], idx)
    log("fp32 attn max err", assert_attn_close(host(out), want_o, host(lse), want_l, 1e-4))


@pytest.mark.parametrize("budget", [(16, 1024, 1024), (16, 32, 64), (4, 100, 300)])
def test_attention_bf16_vs_oracle(budget):
    ks, kw, kp = budget
    x = custom_rows(RAGGED_LENGTHS, RAGGED_ROWS, k_sink=ks, k_swa=kw, k_sparse=kp, seed=21)
    o = oracle_inputs(x)
    c = x["cfg"]
    rng = np.random.default_rng(2)
    idx = _oracle_idx_for(x, kp, rng)
    idx[3, 1:4] = idx[3, 0]            # repeats are ignored
    out, lse = lsa.lsa_hybrid_attn(rows_of(x), x["q"], x["kv"], 512, c["scale"], budget,
                                   torch.from_numpy(idx).to(DEV))
    want_o, want_l = ref.hybrid_attn(o["kv_off"], o["row_seq"], o["row_pos"], o["q"], o["kv"], 512, c["scale"], ks,
                                     kw, idx)
    log("bf16 attn max err", assert_attn_close(host(out), want_o, host(lse), want_l, 2e-2))
    assert np.all(f64(host(out))[-1] == 0) and np.all(np.isneginf(host(lse)[-1]))


@pytest.mark.parametrize("heads", [16, 48, 256])
def test_attention_bf16_head_counts(heads):
    # 16 and 48 heads take the 16-heads-per-wave kernel, 256 two blocks of the 128-head kernel
    x = custom_rows(RAGGED_LENGTHS, RAGGED_ROWS, H=heads, seed=23)
    o = oracle_inputs(x)
    c = x["cfg"]
    idx = _oracle_idx_for(x, c["k_sparse"], np.random.default_rng(4))
    out, lse = lsa.lsa_hybrid_attn(rows_of(x), x["q"], x["kv"], 512, c["scale"], budget_of(c),
                                   torch.from_numpy(idx).to(DEV))
    want_o, want_l = ref.hybrid_attn(o["kv_off"], o["row_seq"], o["row_pos"], o["q"], o["kv"], 512, c["scale"],
                                     c["k_sink"], c["k_swa"], idx)
    log(f"bf16 attn H={heads} max err", assert_attn_close(host(out), want_o, host(lse), want_l, 2e-2))


def test_attention_bf16_many_rows_single_split():
    # enough rows that each row runs in one block (no split partials)
    lengths = [3000] * 4
    rows = [(b, t) for b in range(4) for t in (1100, 2999, 2000, 1500)] * 20
    x = custom_rows(lengths, rows, seed=5)
    o = oracle_inputs(x)
    c = x["cfg"]
    idx = _oracle_idx_for(x, 1024, np.random.default_rng(3))
    out, lse = lsa.lsa_hybrid_attn(rows_of(x), x["q"], x["kv"], 512, c["scale"], budget_of(c),
                                   torch.from_numpy(idx).to(DEV))
    sel = np.arange(0, len(rows), 9)
    want_o, want_l = ref.hybrid_attn(o["kv_off"], o["row_seq"][sel], o["row_pos"][sel], o["q"][sel], o["kv"], 512,
                                     c["scale"], 16, 1024, idx[sel])
    assert_attn_close(host(out)[sel], want_o, host(lse)[sel], want_l, 2e-2)


def test_attention_bf16_ragged_batch_192_rows():
    # 192 rows of 128 heads (the ragged MTP batch's count: one block per row, more than half the CUs):
    # rows of every list length, down to rows near the start of their sequence that hold almost no
    # list (the positions repeat, each row with its own query and picks)
    lengths = [3000, 6000, 700, 60]
    base = [(0, 2999), (1, 5999), (1, 4000), (0, 1500), (2, 699), (2, 100), (3, 0), (3, 59), (1, 1039),
            (1, 1040), (1, 2064), (0, 2200)]
    rows = base * 16
    x = custom_rows(lengths, rows, seed=9)
    o = oracle_inputs(x)
    c = x["cfg"]
    idx = _oracle_idx_for(x, 1024, np.random.default_rng(6))
    out, lse = lsa.lsa_hybrid_attn(rows_of(x), x["q"], x["kv"], 512, c["scale"], budget_of(c),
                                   torch.from_numpy(idx).to(DEV))
    sel = np.concatenate([np.arange(12), np.arange(12, len(rows), 13)])
    want_o, want_l = ref.hybrid_attn(o["kv_off"], o["row_seq"][sel], o["row_pos"][sel], o["q"][sel], o["kv"], 512,
                                     c["scale"], 16, 1024, idx[sel])
    log("192-row attn max err", assert_attn_close(host(out)[sel], want_o, host(lse)[sel], want_l, 2e-2))


@pytest.mark.parametrize("repeat", [1, 40])
def test_attention_bf16_late_dominant_logit(repeat):
    # Latent rows whose last 64 dims (outside the value part) align with head 0's query give that head a
    # logit ~100 nats (over 140 in log2 units) above everything in the first tile of each split: the
    # softmax must still be exact.
    lengths = [3000, 6000]
    rows = [(0, 2999), (1, 5999), (1, 4000), (0, 1500)] * repeat
    x = custom_rows(lengths, rows, seed=8)
    q0 = x["q"][:, 0].float()
    for r, (b, t) in enumerate(rows[:4]):
        base = int(x["kv_off_host"][b])
        for d in (0, 33, 70, 500):
            x["kv"][base + t - d, 512:] = (48.0 * torch.sign(q0[r, 512:])).to(x["kv"].dtype)
    o = oracle_inputs(x)
    c = x["cfg"]
    idx = _oracle_idx_for(x, 1024, np.random.default_rng(4))
    out, lse = lsa.lsa_hybrid_attn(rows_of(x), x["q"], x["kv"], 512, c["scale"], budget_of(c),
                                   torch.from_numpy(idx).to(DEV))
    sel = np.arange(0, len(rows), 7) if repeat > 1 else np.arange(len(rows))
    want_o, want_l = ref.hybrid_attn(o["kv_off"], o["row_seq"][sel], o["row_pos"][sel], o["q"][sel], o["kv"], 512,
                                     c["scale"], 16, 1024, idx[sel])
    assert np.max(want_l[:, 0]) > 80.0
    log("dominant-logit attn max err", assert_attn_close(host(out)[sel], want_o, host(lse)[sel], want_l, 2e-2))


# --------------------------------------------------------------------------------------------- layer


class OracleRanking:
    """The oracle's own scores, to decide where GPU and oracle index sets may differ: a position is a
    near-tie when its Eq. 1 score is within 1e-3 of the row's K-th best; under HI also when its page
    score is within 1e-3 of the M-th best page score (the page ranking itself tied)."""

    def __init__(self, o, c, sb_off=None, k_mean=None):
        self.o, self.c = o, c
        self.lengths = np.diff(o["kv_off"])
        self.sb_off, self.k_mean = sb_off, k_mean
        self.cache = {}

    def _row(self, r):
        if r not in self.cache:
            o, c = self.o, self.c
            sl = slice(r, r + 1)
            flat = ref.index_score(o["kv_off"], o["row_seq"][sl], o["row_pos"][sl], o["q_idx"][sl], o["w"][sl],
                                   o["k_idx"], c["k_sink"], c["k_swa"], ld=int(self.lengths.max()))[0]
            b = int(o["row_seq"][r])
            hi = self.k_mean is not None and self.lengths[b] >= c["hi_min_len"]
            if not hi:
                self.cache[r] = (flat, kth_best(flat, c["k_sparse"]), None, None)
            else:
                P, M = c["P"], c["M"]
                ld = int((self.lengths.max() + P - 1) // P)
                pages, ps = ref.page_recall(o["kv_off"], self.sb_off, o["row_seq"][sl], o["row_pos"][sl],
                                            o["q_idx"][sl], o["w"][sl], self.k_mean, P, c["B"], M, ld=ld)
                comp = ref.index_score(o["kv_off"], o["row_seq"][sl], o["row_pos"][sl], o["q_idx"][sl], o["w"][sl],
                                       o["k_idx"], c["k_sink"], c["k_swa"], ld=M * P, pages=pages, P=P)[0]
                self.cache[r] = (flat, kth_best(comp, c["k_sparse"]), ps[0], kth_best(ps[0], M))
        return self.cache[r]

    def accept(self, r, diff):
        flat, theta, ps, theta_p = self._row(r)
        ok = near_tie(flat[diff], theta)
        if ps is not None:
            ok |= near_tie(ps[diff // self.c["P"]], theta_p)
        return ok


def _compare_layer(o, c, g_idx, g_out, g_lse, w_idx, w_out, w_lse, tol, ranking, idx_row=None):
    """Index sets equal up to near-ties of the oracle's ranking; then EVERY row's attention against the
    oracle's attention run on the GPU's own index set (the same selected set on both sides), and the
    rows whose index set is the oracle's also against the oracle's whole layer."""
    n_diff = assert_idx_sets_match(g_idx, w_idx, ranking.accept)
    a_out, a_lse = ref.hybrid_attn(o["kv_off"], o["row_seq"], o["row_pos"], o["q"], o["kv"], int(c["Dv"]),
                                   c["scale"], int(c["k_sink"]), int(c["k_swa"]), g_idx, idx_row=idx_row)
    err = assert_attn_close(g_out, a_out, g_lse, a_lse, tol, "attention on the GPU's index sets")
    same = np.all(g_idx == w_idx, axis=1)
    if idx_row is not None:
        same = same[np.asarray(idx_row)]
    if same.any():
        assert_attn_close(g_out[same], w_out[same], g_lse[same], w_lse[same], tol, "layer output")
    log(f"layer: {n_diff} rows with near-tie index differences; attention of all {len(g_out)} rows within "
        f"{err:.2e}; {int(same.sum())} rows equal the oracle's whole layer")


def test_layer_tiny_prefill_fp32():
    x = synth.tiny_prefill(device=DEV)
    o = oracle_inputs(x)
    c = x["cfg"]
    idx, out, lse = lsa.lsa_layer_fwd(c, rows_of(x), x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"])
    w_idx, w_out, w_lse = ref.layer_fwd(c, o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"],
                                        o["q"], o["kv"])
    _compare_layer(o, c, host(idx), host(out), host(lse), w_idx, w_out, w_lse, 1e-4, OracleRanking(o, c))
    # needles: every planted key is picked by the row it was planted for
    g_idx = host(idx)
    for r, s in x["needles"]:
        assert s in set(g_idx[r].tolist()), (r, s)


def test_layer_bf16_decode_ragged():
    lengths = [1040, 1041, 2000, 9000, 17000]
    x = synth.decode_batch(lengths, device=DEV, seed=4, needles=8)
    o = oracle_inputs(x)
    c = x["cfg"]
    idx, out, lse = lsa.lsa_layer_fwd(c, rows_of(x), x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"])
    w_idx, w_out, w_lse = ref.layer_fwd(c, o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"],
                                        o["q"], o["kv"])
    _compare_layer(o, c, host(idx), host(out), host(lse), w_idx, w_out, w_lse, 2e-2, OracleRanking(o, c))
    g_idx = host(idx)
    for b, picks in enumerate(x["needles"]):
        assert set(picks) <= set(g_idx[b].tolist())


FUSED_LENGTHS = [1, 17, 1041, 1042, 3001, 8192, 8193, 20000, 40000, 200001]
# (the last two rows sit at t = L_b: rows outside their sequence, which select nothing)
FUSED_ROWS = [(b, L - 1) for b, L in enumerate(FUSED_LENGTHS)] + [(8, 9000), (9, 8192 + 1040), (6, 8193), (5, 8192)]
# 42 rows x 13 chunks of 16384 columns (546 blocks): the bf16 fused pass on 16384-column chunks, two
# 4-wave blocks per CU
WIDE_FUSED_ROWS = FUSED_ROWS + [(9, 200000 - 4001 * i) for i in range(1, 29)]
# 24 rows x 13 chunks (312 blocks, one round): 16384-column chunks, one 8-wave block per CU
MID_FUSED_ROWS = FUSED_ROWS + [(9, 200000 - 9001 * i) for i in range(1, 11)]
# 60 rows x 19 chunks of 16384 columns (1140 blocks): more than two rounds of two 4-wave blocks per CU,
# rows ending all along the sequence
TAIL_FUSED_LENGTHS = FUSED_LENGTHS + [300000]
TAIL_FUSED_ROWS = FUSED_ROWS + [(10, 299999 - 6001 * i) for i in range(46)]


@pytest.mark.parametrize("distinct", [1, 3, 40, 4096])
def test_index_topk_fused_ties(distinct):
    # keys drawn from a few distinct vectors, so every row's scores tie in long runs and the picks at the
    # threshold are decided by position (1: all candidates equal; 4096: a few equal scores per value, so
    # the threshold's digit bin is small but holds ties); the fused pass (14 rows x 25 segments) must
    # match scoring then selecting bit for bit
    rows = {3: WIDE_FUSED_ROWS, 40: MID_FUSED_ROWS, 4096: MID_FUSED_ROWS}.get(distinct, FUSED_ROWS)
    x = custom_rows(FUSED_LENGTHS, rows, attn=False, seed=46)
    n_tok = x["k_idx"].shape[0]
    pick = torch.randint(0, distinct, (n_tok,), generator=synth.generator(47, DEV), device=DEV)
    x["k_idx"] = x["k_idx"][:distinct].clone()[pick].contiguous()
    c = x["cfg"]
    for k in (1, 1024):
        bud = (c["k_sink"], c["k_swa"], k)
        log(f"index_topk ties distinct={distinct} k={k}")
        got = lsa.lsa_index_topk(rows_of(x), x["q_idx"], x["w"], x["k_idx"], bud)
        sc = lsa.lsa_index_score(rows_of(x), x["q_idx"], x["w"], x["k_idx"], bud)
        assert torch.equal(got, lsa.lsa_topk(sc, k))


@pytest.mark.parametrize("form", ["8192", "16384x8w", "16384"])
def test_index_topk_fused_vs_oracle(form):
    # The fused scoring + first top-K level against the oracle's whole-row selection (Eq. 1 over mid(t),
    # then Eq. 2): 14 rows x 25 chunks take the 8192-column kernel, 24 rows x 13 chunks the 16384-column
    # 8-wave kernel that the 128K decode runs, 42 rows x 13 chunks the 16384-column 4-wave kernel that the
    # 1M decode runs.  Index sets must agree except at near-ties of the oracle's ranking.
    rows = {"8192": FUSED_ROWS, "16384x8w": MID_FUSED_ROWS, "16384": WIDE_FUSED_ROWS}[form]
    x = custom_rows(FUSED_LENGTHS, rows, attn=False, seed=61)
    o = oracle_inputs(x)
    c = x["cfg"]
    sc = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"], c["k_sink"],
                         c["k_swa"], ld=x["max_len"])
    for k in (1, 1024, 4096):
        got = host(lsa.lsa_index_topk(rows_of(x), x["q_idx"], x["w"], x["k_idx"], (c["k_sink"], c["k_swa"], k)))
        want = ref.topk(sc, k)
        theta = [kth_best(sc[r], k) for r in range(len(rows))]
        n_diff = assert_idx_sets_match(got, want, lambda r, d: near_tie(sc[r][d], theta[r]), f"fused k={k}")
        log(f"fused selection ({form}) k={k}: {n_diff} rows with near-tie differences")


def test_layer_fused_first_level_equals_separate_passes():
    # Rows scored one by one go through the fused scoring + first top-K level (segments of 8192
    # columns; used when rows x segments >= 256, here 14 x 25); the index sets must be bit-identical to
    # scoring everything and then selecting.
    x = custom_rows(FUSED_LENGTHS, FUSED_ROWS, seed=41)
    c = x["cfg"]
    idx_layer = lsa.lsa_layer_fwd(c, rows_of(x), x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"])[0]
    sc = lsa.lsa_index_score(rows_of(x), x["q_idx"], x["w"], x["k_idx"], budget_of(c))
    idx_sep = lsa.lsa_topk(sc, c["k_sparse"])
    assert torch.equal(idx_layer, idx_sep)
    assert (host(idx_layer)[0] == -1).all()       # L = 1: no mid region


@pytest.mark.parametrize("k", [1, 1024, 4096])
def test_index_topk_equals_score_then_topk(k):
    # lsa_index_topk on the fused pass (14 rows x 25 segments of 8192 columns) and on the separate
    # passes (2 rows) against scoring everything and then selecting: bit-identical index sets
    for lengths, rows, seed in ((FUSED_LENGTHS, FUSED_ROWS, 42), (FUSED_LENGTHS, WIDE_FUSED_ROWS, 51),
                                (FUSED_LENGTHS, MID_FUSED_ROWS, 52), (TAIL_FUSED_LENGTHS, TAIL_FUSED_ROWS, 54),
                                ([20000, 9000], [(0, 19999), (1, 8999)], 43)):
        x = custom_rows(lengths, rows, attn=False, seed=seed)
        c = x["cfg"]
        bud = (c["k_sink"], c["k_swa"], k)
        log(f"index_topk k={k} rows={len(rows)} max_len={x['max_len']}")
        got = lsa.lsa_index_topk(rows_of(x), x["q_idx"], x["w"], x["k_idx"], bud)
        sc = lsa.lsa_index_score(rows_of(x), x["q_idx"], x["w"], x["k_idx"], bud)
        assert torch.equal(got, lsa.lsa_topk(sc, k))
        # a reused workspace and output give the same answer
        ws = lsa.lsa_index_topk_workspace(rows_of(x), x["q_idx"], k)
        again = torch.full_like(got, 7)
        lsa.lsa_index_topk(rows_of(x), x["q_idx"], x["w"], x["k_idx"], bud, idx=again, ws=ws)
        lsa.lsa_index_topk(rows_of(x), x["q_idx"], x["w"], x["k_idx"], bud, idx=again, ws=ws)
        assert torch.equal(got, again)


def test_layer_deterministic():
    x = synth.decode_batch([5000, 12000], device=DEV, seed=6, needles=4)
    c = x["cfg"]
    a = lsa.lsa_layer_fwd(c, rows_of(x), x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"])
    b = lsa.lsa_layer_fwd(c, rows_of(x), x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"])
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.uint8) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.uint8) if v.dtype == torch.bfloat16 else v)


def _hi_setup(lengths, M, B=128, seed=8, drafts=1, hi_min_len=0):
    x = synth.decode_batch(lengths, device=DEV, seed=seed, needles=0, needle_pages=8, M=M, B=B, drafts=drafts,
                           hi_min_len=hi_min_len)
    sb_off = lsa.sb_offsets(lengths, B)
    km = lsa.lsa_page_means(x["kv_off"], sb_off.to(DEV), x["k_idx"], B, x["max_len"])
    return x, sb_off, km


def test_layer_hi_full_recall_equals_flat_on_gpu():
    # M * P >= L: every causal page is recalled, so HI picks exactly what the flat indexer picks
    lengths = [6000, 3000, 1500]
    x, sb_off, km = _hi_setup(lengths, M=64)
    c = x["cfg"]
    flat = lsa.lsa_layer_fwd(c, rows_of(x), x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"])
    hi = lsa.lsa_layer_fwd(c, rows_of(x), x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"],
                           sb_off=sb_off.to(DEV), k_mean=km)
    assert torch.equal(flat[0], hi[0])
    assert torch.equal(flat[1].view(torch.int16), hi[1].view(torch.int16))


@pytest.mark.parametrize("B", [128, 16])
def test_layer_hi_vs_oracle(B):
    lengths = [40000, 25000, 9000]
    x, sb_off, km = _hi_setup(lengths, M=24, B=B, hi_min_len=20000)
    o = oracle_inputs(x)
    c = x["cfg"]
    km_o = ref.page_means(o["kv_off"], sb_off.numpy(), o["k_idx"], B)
    assert np.array_equal(host(km), km_o)
    idx, out, lse = lsa.lsa_layer_fwd(c, rows_of(x), x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"],
                                      sb_off=sb_off.to(DEV), k_mean=km)
    w_idx, w_out, w_lse = ref.layer_fwd(c, o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"],
                                        o["q"], o["kv"], sb_off=sb_off.numpy(), k_mean=km_o)
    _compare_layer(o, c, host(idx), host(out), host(lse), w_idx, w_out, w_lse, 2e-2,
                   OracleRanking(o, c, sb_off.numpy(), km_o))
    # diagnostic only: with one needle per page, a page mean can dilute it below the recall cut
    # (the coarse stage cannot recover what it misses), so needle recall under HI is reported.
    g_idx = host(idx)
    hits = sum(len(set(p) & set(g_idx[b].tolist())) for b, p in enumerate(x["needles"]))
    log(f"HI B={B}: needles picked {hits}/{sum(len(p) for p in x['needles'])}")


@pytest.mark.parametrize("M", [24, 64])  # 64: recall lists long enough for the multi-row stage-2 kernel
def test_layer_hi_chunked_prefill_vs_oracle(M):
    # HI on the rows of a prefill chunk with sub-blocks of 8: the page of row t also holds tokens after
    # t, which lie in the window or in the future and never yield candidates.  The oracle runs on rows
    # on both sides of the page edges crossed by the chunk (t = 38016 and 38144 start pages).
    x = synth.prefill_chunk(38000, 160, device=DEV, seed=11, B=8, M=M, hi_min_len=0)
    c = x["cfg"]
    sb_off = lsa.sb_offsets(x["lengths"], c["B"])
    km = lsa.lsa_page_means(x["kv_off"], sb_off.to(DEV), x["k_idx"], c["B"], x["max_len"])
    o = oracle_inputs(x)
    km_o = ref.page_means(o["kv_off"], sb_off.numpy(), o["k_idx"], c["B"])
    assert np.array_equal(host(km), km_o)
    idx, out, lse = lsa.lsa_layer_fwd(c, rows_of(x), x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"],
                                      sb_off=sb_off.to(DEV), k_mean=km)
    sel = np.array([0, 15, 16, 17, 80, 143, 144, 159])
    os_ = dict(o)
    for k in ("row_seq", "row_pos", "q_idx", "w", "q"):
        os_[k] = o[k][sel]
    w_idx, w_out, w_lse = ref.layer_fwd(c, os_["kv_off"], os_["row_seq"], os_["row_pos"], os_["q_idx"], os_["w"],
                                        o["k_idx"], os_["q"], o["kv"], sb_off=sb_off.numpy(), k_mean=km_o)
    _compare_layer(os_, c, host(idx)[sel], host(out)[sel], host(lse)[sel], w_idx, w_out, w_lse, 2e-2,
                   OracleRanking(os_, c, sb_off.numpy(), km_o))
    # the recall restricts the candidates: the flat indexer picks differently on most rows
    flat = lsa.lsa_layer_fwd(dict(c, hi_min_len=1 << 62), rows_of(x), x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"],
                             k_idx=x["k_idx"])[0]
    assert (host(flat) != host(idx)).any(axis=1).mean() > 0.5


def test_layer_hi_all_rows_bound():
    # min_kv_len >= hi_min_len lets the layer skip the flat passes and the row-role pass; the result is
    # bit for bit that of the gated run (min_kv_len = 0)
    lengths = [40000, 25000]
    x, sb_off, km = _hi_setup(lengths, M=24, B=128, hi_min_len=20000)
    c = x["cfg"]
    r0 = rows_of(x)
    r1 = lsa.RowsDesc(r0.kv_off, r0.row_seq, r0.row_pos, r0.max_kv_len, min(lengths))
    a = lsa.lsa_layer_fwd(c, r0, x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"], sb_off=sb_off.to(DEV),
                          k_mean=km)
    b = lsa.lsa_layer_fwd(c, r1, x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"], sb_off=sb_off.to(DEV),
                          k_mean=km)
    assert torch.equal(a[0], b[0])
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16)) and torch.equal(a[2], b[2])


def test_cli_reuse_layer():
    x = synth.decode_batch([7000, 3000], device=DEV, seed=9, needles=4)
    c = x["cfg"]
    o = oracle_inputs(x)
    idx, out, lse = lsa.lsa_layer_fwd(c, rows_of(x), x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"])
    reuse = dict(c, is_owner=0)
    # with the owner's own q / kv the reuse layer reproduces the owner's output bit for bit
    _, out2, lse2 = lsa.lsa_layer_fwd(reuse, rows_of(x), x["q"], x["kv"], idx=idx.clone())
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse, lse2)
    # with its own q / kv and the oracle's index set it matches the oracle's reuse layer
    g = synth.generator(99, DEV)
    q2 = synth.normal(tuple(x["q"].shape), 1.0, g, DEV, torch.bfloat16)
    kv2 = synth.normal(tuple(x["kv"].shape), 1.0, g, DEV, torch.bfloat16)
    w_idx, _, _ = ref.layer_fwd(c, o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"], o["q"],
                                o["kv"])
    _, out3, lse3 = lsa.lsa_layer_fwd(reuse, rows_of(x), q2, kv2, idx=torch.from_numpy(w_idx).to(DEV))
    _, w_out3, w_lse3 = ref.layer_fwd(reuse, o["kv_off"], o["row_seq"], o["row_pos"], None, None, None, host(q2),
                                      host(kv2), idx=w_idx)
    assert_attn_close(host(out3), w_out3, host(lse3), w_lse3, 2e-2)


def test_mtp_drafts_share_index_and_hi_gate():
    lengths = [5000, 30000, 2000]
    x, sb_off, km = _hi_setup(lengths, M=16, drafts=3, hi_min_len=20000)
    c = x["cfg"]
    o = oracle_inputs(x)
    km_o = ref.page_means(o["kv_off"], sb_off.numpy(), o["k_idx"], 128)
    idx, out, lse = lsa.lsa_layer_fwd(c, rows_of(x), x["q"], x["kv"], q_idx=x["q_idx"], w=x["w"], k_idx=x["k_idx"],
                                      idx_row=x["idx_row"], sb_off=sb_off.to(DEV), k_mean=km)
    g_idx = host(idx)
    w_idx, w_out, w_lse = ref.layer_fwd(c, o["kv_off"], o["row_seq"], o["row_pos"], o["q_idx"], o["w"], o["k_idx"],
                                        o["q"], o["kv"], idx_row=x["idx_row_host"].numpy(), sb_off=sb_off.numpy(),
                                        k_mean=km_o)
    assert np.all(g_idx[x["idx_row_host"].numpy() != np.arange(9)] == -1)   # drafts own no index row
    # every draft attends with its sequence's index set (the oracle runs on the GPU's index rows)
    _compare_layer(o, c, g_idx, host(out), host(lse), w_idx, w_out, w_lse, 2e-2,
                   OracleRanking(o, c, sb_off.numpy(), km_o), idx_row=x["idx_row_host"].numpy())
    for r in range(9):
        if r % 3:
            assert not torch.equal(out[r].view(torch.int16), out[r - r % 3].view(torch.int16))  # own q per draft
