"""GPU parity of the FP8 indexer path against the oracle: the quantizer bit for bit, the scores within
the indexer tolerance (Eq. 1 on the oracle's own dequantized inputs), and the selection built on them."""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_weighted_amd as lsa
import oracle as ref
import synth
from oracle import fp8
from parity_util import (assert_idx_sets_match, assert_scores_close, budget_of, f64, host, kth_best, log, near_tie,
                         oracle_inputs, rows_of)
from test_gpu_parity import (FUSED_LENGTHS, FUSED_ROWS, MID_FUSED_ROWS, RAGGED_LENGTHS, RAGGED_ROWS, TAIL_FUSED_LENGTHS,
                             TAIL_FUSED_ROWS, WIDE_FUSED_ROWS, custom_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _oracle_deq(a):
    """The oracle's quantize-then-dequantize of host values (bf16 bits or fp32), as fp32."""
    codes, scale = fp8.quantize(f64(a))
    return fp8.dequantize(codes, scale)


def _gpu_fp8(x):
    q8, qs = lsa.lsa_quantize_fp8(x["q_idx"])
    k8, ks = lsa.lsa_quantize_fp8(x["k_idx"])
    return q8, qs, k8, ks


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_fp8_bit_exact(dtype):
    g = synth.generator(21, DEV)
    x = synth.normal((3000, 128), 1 / math.sqrt(128), g, DEV, dtype)
    x[0] = 0.0                                      # all zero: scale 1, codes 0
    x[1] = x[1] * 1e-30                             # tiny vector: a large negative exponent
    x[2, 5] = 56.0                                  # max exactly 448 * 2^-3
    x[3, :4] = torch.tensor([448.0, 1.0625, 17.0, 3 * 2.0 ** -10], dtype=dtype)   # ties at scale 1
    x[4] = -x[4]
    codes, scale = lsa.lsa_quantize_fp8(x)
    want_c, want_s = fp8.quantize(f64(host(x)))
    assert np.array_equal(host(codes), want_c)
    assert np.array_equal(host(scale), want_s)
    assert host(codes)[3, :4].tolist() == [0x7E, 0x38, 0x58, 0x02]
    # query heads (3-D) and a vector length that is not a multiple of the wave
    q = synth.normal((7, 64, 100), 0.3, g, DEV, dtype)
    qc, qsc = lsa.lsa_quantize_fp8(q)
    wc, wsc = fp8.quantize(f64(host(q)))
    assert np.array_equal(host(qc), wc) and np.array_equal(host(qsc), wsc)


def test_index_score_fp8_ragged_and_edges():
    x = custom_rows(RAGGED_LENGTHS, RAGGED_ROWS, attn=False, seed=22)
    o = oracle_inputs(x)
    c = x["cfg"]
    ld = x["max_len"] + 37
    q8, qs, k8, ks = _gpu_fp8(x)
    g = lsa.lsa_index_score_fp8(rows_of(x), q8, qs, x["w"], k8, ks, budget_of(c), ld=ld)
    want = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], _oracle_deq(o["q_idx"]), o["w"],
                           _oracle_deq(o["k_idx"]), c["k_sink"], c["k_swa"], ld=ld)
    log("fp8 scores worst err/tol", assert_scores_close(host(g), want))
    assert np.all(np.isneginf(host(g)[-1]))


def test_index_score_fp8_multi_chunk_decode():
    # rows spanning several 16384-column chunks and a ragged tail, plus interior rows
    lengths = [40000, 21000, 1100]
    rows = [(0, 39999), (0, 17000), (1, 20999), (1, 1040), (2, 1099)]
    x = custom_rows(lengths, rows, attn=False, seed=23)
    o = oracle_inputs(x)
    c = x["cfg"]
    q8, qs, k8, ks = _gpu_fp8(x)
    g = lsa.lsa_index_score_fp8(rows_of(x), q8, qs, x["w"], k8, ks, budget_of(c))
    want = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], _oracle_deq(o["q_idx"]), o["w"],
                           _oracle_deq(o["k_idx"]), c["k_sink"], c["k_swa"], ld=x["max_len"])
    log("fp8 multi-chunk scores worst err/tol", assert_scores_close(host(g), want))


@pytest.mark.parametrize("P", [128, 48])
def test_index_score_fp8_page_mapped(P):
    L = 9000
    x = custom_rows([L, 4000], [(0, L - 1), (0, 5000), (1, 3999)], attn=False, seed=24)
    o = oracle_inputs(x)
    c = x["cfg"]
    M = 12
    pages = np.full((3, M), -1, np.int32)
    pages[0, :10] = [0, 1, 7, 8, 30, 31, 55, 60, 69, 70]
    pages[1, :6] = [3, 9, 20, 30, 31, 39]
    pages[2, :5] = [0, 5, 10, 23, 31]
    pg = torch.from_numpy(pages).to(DEV)
    q8, qs, k8, ks = _gpu_fp8(x)
    g = lsa.lsa_index_score_fp8(rows_of(x), q8, qs, x["w"], k8, ks, budget_of(c), pages=pg, P=P, ld=M * P + 5)
    want = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], _oracle_deq(o["q_idx"]), o["w"],
                           _oracle_deq(o["k_idx"]), c["k_sink"], c["k_swa"], ld=M * P + 5, pages=pages, P=P)
    log("fp8 paged scores worst err/tol", assert_scores_close(host(g), want))


def test_fp8_selection_vs_oracle():
    # FP8 scores -> top-K on the GPU against the oracle's top-K of its own FP8 scores: equal sets
    # except near-ties; the planted needles (bf16 keys, then quantized) are still picked
    x = synth.decode_batch([30000, 12000, 5000], device=DEV, seed=25, needles=16, with_attn=False)
    o = oracle_inputs(x)
    c = x["cfg"]
    q8, qs, k8, ks = _gpu_fp8(x)
    g = lsa.lsa_index_score_fp8(rows_of(x), q8, qs, x["w"], k8, ks, budget_of(c))
    g_idx = host(lsa.lsa_topk(g, c["k_sparse"]))
    want = ref.index_score(o["kv_off"], o["row_seq"], o["row_pos"], _oracle_deq(o["q_idx"]), o["w"],
                           _oracle_deq(o["k_idx"]), c["k_sink"], c["k_swa"], ld=x["max_len"])
    w_idx = ref.topk(want, c["k_sparse"])
    theta = [kth_best(want[r], c["k_sparse"]) for r in range(len(w_idx))]
    n = assert_idx_sets_match(g_idx, w_idx, lambda r, d: near_tie(want[r][d], theta[r]))
    log(f"fp8 selection: {n} rows with near-tie differences")
    for b, picks in enumerate(x["needles"]):
        assert set(picks) <= set(g_idx[b].tolist())


FP8_FUSED_ROWS = WIDE_FUSED_ROWS  # a larger fused batch: 42 rows x 25 segments of 8192 columns


@pytest.mark.parametrize("k", [1, 1024, 4096])
def test_index_topk_fp8_equals_score_then_topk(k):
    # the fused FP8 pass (42 and 14 rows x 25 segments of 8192 columns) and the separate passes (2 rows)
    # against FP8 scores then top-K: bit-identical index sets
    for lengths, rows, seed in ((FUSED_LENGTHS, FP8_FUSED_ROWS, 44), (FUSED_LENGTHS, FUSED_ROWS, 50),
                                (FUSED_LENGTHS, MID_FUSED_ROWS, 53), (TAIL_FUSED_LENGTHS, TAIL_FUSED_ROWS, 55),
                                ([20000, 9000], [(0, 19999), (1, 8999)], 45)):
        x = custom_rows(lengths, rows, attn=False, seed=seed)
        c = x["cfg"]
        bud = (c["k_sink"], c["k_swa"], k)
        log(f"index_topk_fp8 k={k} rows={len(rows)} max_len={x['max_len']}")
        q8, qs, k8, ks = _gpu_fp8(x)
        got = lsa.lsa_index_topk_fp8(rows_of(x), q8, qs, x["w"], k8, ks, bud)
        sc = lsa.lsa_index_score_fp8(rows_of(x), q8, qs, x["w"], k8, ks, bud)
        assert torch.equal(got, lsa.lsa_topk(sc, k))


def test_index_topk_fp8_fused_ties():
    # keys from 3 distinct vectors: long runs of equal FP8 scores, picks at the threshold by position
    x = custom_rows(FUSED_LENGTHS, FP8_FUSED_ROWS, attn=False, seed=48)
    n_tok = x["k_idx"].shape[0]
    pick = torch.randint(0, 3, (n_tok,), generator=synth.generator(49, DEV), device=DEV)
    x["k_idx"] = x["k_idx"][:3].clone()[pick].contiguous()
    c = x["cfg"]
    bud = (c["k_sink"], c["k_swa"], c["k_sparse"])
    q8, qs, k8, ks = _gpu_fp8(x)
    got = lsa.lsa_index_topk_fp8(rows_of(x), q8, qs, x["w"], k8, ks, bud)
    sc = lsa.lsa_index_score_fp8(rows_of(x), q8, qs, x["w"], k8, ks, bud)
    assert torch.equal(got, lsa.lsa_topk(sc, c["k_sparse"]))
