"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every check here is a closed form, an invariant the pages state, a special case that reduces to a
textbook or library routine (a dot product, a full sort, dense softmax attention), or brute force
on tiny inputs.  Each is chosen so that a plausible slip in the oracle (a dropped term, a wrong
sign or index, a transposed operand, an off-by-one range) makes one of them fail.
"""
import math

import numpy as np
import pytest
import torch

from synth import bf16_to_bits

# -------------------------------------------------------------------------------- helpers


def bf16(a):
    """float array -> bf16 raw bits (round to nearest even, by torch)."""
    return bf16_to_bits(torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16))


def dec(ref, a):
    return ref.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def one_seq(L):
    return np.array([0, L], np.int64)


# -------------------------------------------------------------------------------- bf16 rounding


def test_bf16_rounding_ties_and_edges(ref):
    # exact values and ties to even, by hand
    assert ref.double_to_bf16(1.0) == 0x3F80
    assert ref.double_to_bf16(1.0 + 2.0 ** -8) == 0x3F80          # tie -> even (1.0)
    assert ref.double_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even (1 + 2^-6)
    assert ref.double_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # just above the tie
    assert ref.double_to_bf16(-2.5) == 0xC020
    assert ref.double_to_bf16(0.0) == 0x0000
    assert ref.double_to_bf16(-0.0) == 0x8000
    assert ref.double_to_bf16(3.5e38) == 0x7F80                     # overflow -> inf
    assert ref.double_to_bf16(2.0 ** -133) == 0x0001                # smallest subnormal
    assert ref.double_to_bf16(2.0 ** -135) == 0x0000                # rounds to zero


def test_bf16_rounding_matches_torch_on_fp32_values(ref):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(4000) * np.exp(rng.uniform(-30, 30, 4000))).astype(np.float32)
    want = bf16(x)  # torch: fp32 -> bf16, nearest-even; the fp32 values are exact doubles
    got = np.array([ref.double_to_bf16(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, want)


# -------------------------------------------------------------------------------- a1: SI ranges


@pytest.mark.parametrize("k_sink,k_swa", [(16, 1024), (16, 128), (0, 8), (4, 0), (1, 1)])
def test_ranges_partition_the_prefix(ref, k_sink, k_swa):
    L = 1300
    for t in list(range(0, 40)) + list(range(k_sink + k_swa - 3, k_sink + k_swa + 4)) + [L - 1]:
        if t < 0 or t >= L:
            continue
        (a0, a1), (b0, b1), (c0, c1) = ref.ranges(t, L, k_sink, k_swa)
        sets = [set(range(a0, a1)), set(range(b0, b1)), set(range(c0, c1))]
        assert not (sets[0] & sets[1]) and not (sets[0] & sets[2]) and not (sets[1] & sets[2])
        assert sets[0] | sets[1] | sets[2] == set(range(t + 1))          # they tile [0, t]
        assert sets[0] == set(range(min(k_sink, t + 1)))                  # the first Ksink tokens
        assert sets[1] == set(range(max(0, t - k_swa + 1), t + 1)) - sets[0]  # the last Kswa, minus sink
        assert len(sets[2]) == max(0, t - k_sink - k_swa + 1)


def test_ranges_invalid_row_is_empty(ref):
    for t in (-1, 50, 51):
        r = ref.ranges(t, 50, 16, 8)
        if t < 0 or t >= 50:
            assert r == ((0, 0), (0, 0), (0, 0))


# -------------------------------------------------------------------------------- a2: Eq. 1 score


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_score_one_hot_closed_form(ref, dt):
    """q_j = a_j e_{pi(j)}  =>  I = sum_j w_j ReLU(a_j k[pi(j)]); exercises head/dim indexing and signs."""
    rng = np.random.default_rng(2)
    HI, dI = 8, 16
    pi = rng.permutation(dI)[:HI]
    a = rng.choice([-2.0, -0.5, 0.25, 1.0, 3.0], HI)
    q = np.zeros((HI, dI), np.float32)
    q[np.arange(HI), pi] = a
    k = rng.choice([-1.5, -0.25, 0.5, 2.0], dI).astype(np.float32)
    w = rng.choice([0.5, 1.0, 2.0, -1.0], HI).astype(np.float32)
    want = float(sum(w[j] * max(a[j] * k[pi[j]], 0.0) for j in range(HI)))
    if dt == "bf16":
        got = ref.score_one(bf16(q), w, bf16(k))
    else:
        got = ref.score_one(q, w, k)
    assert got == want  # every value above is exact in both dtypes


def test_score_single_head_is_relu_of_dot(ref):
    rng = np.random.default_rng(3)
    for _ in range(20):
        q = rng.standard_normal((1, 128)).astype(np.float32)
        k = rng.standard_normal(128).astype(np.float32)
        d = float(np.dot(q[0].astype(np.float64), k.astype(np.float64)))
        assert ref.score_one(q, np.ones(1, np.float32), k) == pytest.approx(max(d, 0.0), rel=1e-13, abs=1e-13)


def test_score_homogeneity_and_weight_sign(ref):
    rng = np.random.default_rng(4)
    q = rng.standard_normal((6, 32)).astype(np.float32)
    k = rng.standard_normal(32).astype(np.float32)
    w = np.abs(rng.standard_normal(6)).astype(np.float32)
    base = ref.score_one(q, w, k)
    assert ref.score_one(q, w, 4.0 * k) == pytest.approx(4.0 * base, rel=1e-14)   # ReLU(c x) = c ReLU(x), c > 0
    assert ref.score_one(q, -w, k) == pytest.approx(-base, rel=1e-14)
    assert ref.score_one(-np.abs(q), w, np.abs(k)) == 0.0                         # every dot < 0 -> 0
    perm = rng.permutation(6)
    assert ref.score_one(q[perm], w[perm], k) == pytest.approx(base, rel=1e-14)   # heads commute


def test_index_score_flat_masks_exactly_outside_mid(ref):
    rng = np.random.default_rng(5)
    L, HI, dI, k_sink, k_swa = 90, 3, 8, 5, 20
    rows = np.array([0, 4, 5, 24, 25, 26, 60, 89], np.int32)
    q = rng.standard_normal((len(rows), HI, dI)).astype(np.float32)
    w = rng.uniform(0.1, 2, (len(rows), HI)).astype(np.float32)
    k = rng.standard_normal((L, dI)).astype(np.float32)
    sc = ref.index_score(one_seq(L), np.zeros(len(rows)), rows, q, w, k, k_sink, k_swa, ld=L + 7)
    for i, t in enumerate(rows):
        lo, hi = k_sink, t - k_swa + 1
        for s in range(L + 7):
            if lo <= s < hi:
                want = sum(float(w[i, j]) * max(float(np.dot(q[i, j].astype(np.float64), k[s].astype(np.float64))), 0.0)
                           for j in range(HI))
                assert sc[i, s] == np.float32(want) or abs(sc[i, s] - want) <= 1e-6 * abs(want) + 1e-7
            else:
                assert sc[i, s] == -np.inf


def test_index_score_page_mapped_equals_flat_gather(ref):
    rng = np.random.default_rng(6)
    L, P, M = 700, 16, 9
    q = rng.standard_normal((2, 4, 8)).astype(np.float32)
    w = rng.uniform(0.1, 2, (2, 4)).astype(np.float32)
    k = rng.standard_normal((L, 8)).astype(np.float32)
    rows = np.array([699, 650], np.int32)
    flat = ref.index_score(one_seq(L), [0, 0], rows, q, w, k, 4, 50, ld=L)
    pages = np.full((2, M), -1, np.int32)
    pages[0, :7] = [0, 3, 10, 20, 40, 41, 43]          # 43 is the last, partial page (L = 700)
    pages[1, :4] = [1, 2, 39, 40]                      # page 40 holds t - Kswa + 1 .. : masked part
    comp = ref.index_score(one_seq(L), [0, 0], rows, q, w, k, 4, 50, ld=M * P, pages=pages, P=P)
    for r in range(2):
        for u in range(M * P):
            pg = pages[r, u // P]
            pos = pg * P + u % P if pg >= 0 else -1
            want = flat[r, pos] if 0 <= pos < L else -np.inf
            assert comp[r, u] == want


# -------------------------------------------------------------------------------- a7: top-K


def _sort_topk(scores, K):
    """Full sort by (score desc, position asc) with numpy's lexsort; finite entries only."""
    out = np.full((scores.shape[0], K), -1, np.int32)
    for r, row in enumerate(scores):
        pos = np.nonzero(np.isfinite(row))[0]
        order = np.lexsort((pos, -row[pos].astype(np.float64)))
        pick = np.sort(pos[order[:K]])
        out[r, :len(pick)] = pick
    return out


def test_topk_equals_full_sort(ref):
    rng = np.random.default_rng(7)
    for trial in range(30):
        n = int(rng.integers(1, 300))
        K = int(rng.integers(1, 64))
        s = rng.choice([-1.0, 0.0, -0.0, 0.5, 0.5, 2.0, 3.25], (4, n)).astype(np.float32) if trial % 2 else \
            rng.standard_normal((4, n)).astype(np.float32)
        s[rng.random((4, n)) < 0.2] = -np.inf
        assert np.array_equal(ref.topk(s, K), _sort_topk(s, K))


def test_topk_rank_count_brute_force(ref):
    """Selected  <=>  fewer than K entries are strictly better under (score desc, position asc)."""
    rng = np.random.default_rng(8)
    s = rng.integers(-3, 4, (3, 60)).astype(np.float32)
    s[:, ::7] = -np.inf
    K = 13
    got = ref.topk(s, K)
    for r in range(3):
        sel = set(int(x) for x in got[r] if x >= 0)
        for p in range(60):
            if not np.isfinite(s[r, p]):
                assert p not in sel
                continue
            better = sum(1 for o in range(60) if np.isfinite(s[r, o]) and
                         (s[r, o] > s[r, p] or (s[r, o] == s[r, p] and o < p)))
            assert (p in sel) == (better < K)


def test_topk_special_cases(ref):
    # all equal -> the K lowest positions
    assert np.array_equal(ref.topk(np.full((1, 50), 1.5, np.float32), 8)[0], np.arange(8))
    # -0.0 and +0.0 are equal: the lower position wins either way round
    assert ref.topk(np.array([[-0.0, 0.0]], np.float32), 1)[0, 0] == 0
    assert ref.topk(np.array([[0.0, -0.0]], np.float32), 1)[0, 0] == 0
    # -inf is never chosen; fewer candidates than K -> pad with -1
    got = ref.topk(np.array([[-np.inf, 1.0, -np.inf, -5.0]], np.float32), 4)[0]
    assert list(got) == [1, 3, -1, -1]
    # empty row
    assert list(ref.topk(np.full((1, 5), -np.inf, np.float32), 3)[0]) == [-1, -1, -1]
    # NaN is rejected
    with pytest.raises(ValueError):
        ref.topk(np.array([[1.0, np.nan]], np.float32), 1)
    # negative scores order correctly
    assert list(ref.topk(np.array([[-3.0, -1.0, -2.0, -1.0]], np.float32), 2)[0]) == [1, 3]


def test_topk_page_map(ref):
    s = np.array([[5.0, 1.0, 7.0, 7.0, 2.0, 9.0]], np.float32)     # 3 pages of P = 2
    pages = np.array([[4, 9, -1]], np.int32)                        # columns 4, 5 sit in an empty slot
    got = ref.topk(s, 3, pages=pages, P=2)
    # page 4 -> positions 8, 9; page 9 -> 18, 19.  Best three: 7 (pos 18), 7 (pos 19), 5 (pos 8)
    assert list(got[0]) == [8, 18, 19]


# -------------------------------------------------------------------------------- a3: sub-block means


def test_page_means_closed_forms(ref):
    lens = [37, 16, 5]
    kv_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    B, dI = 8, 4
    sb_off = np.concatenate([[0], np.cumsum([(L + B - 1) // B for L in lens])]).astype(np.int64)
    tot = int(kv_off[-1])
    k = np.zeros((tot, dI), np.float32)
    for b, L in enumerate(lens):
        pos = np.arange(L, dtype=np.float32)
        k[kv_off[b]:kv_off[b + 1], 0] = pos                 # mean = middle position of the block
        k[kv_off[b]:kv_off[b + 1], 1] = -2.0                # constant
        k[kv_off[b]:kv_off[b + 1], 2] = (pos % 2) * 4.0     # alternating 0, 4
        k[kv_off[b]:kv_off[b + 1], 3] = b + 1
    for dt in ("f32", "bf16"):
        kk = k if dt == "f32" else bf16(k)
        m = dec(ref, ref.page_means(kv_off, sb_off, kk, B))
        for b, L in enumerate(lens):
            for n in range((L + B - 1) // B):
                lo, hi = n * B, min((n + 1) * B, L)
                row = m[sb_off[b] + n]
                want0 = (lo + hi - 1) / 2.0
                assert row[0] == (want0 if dt == "f32" else ref.bf16_bits_to_f64(bf16([want0]))[0])
                assert row[1] == -2.0
                cnt_odd = sum(1 for s in range(lo, hi) if s % 2)
                want2 = 4.0 * cnt_odd / (hi - lo)
                got2 = row[2]
                assert abs(got2 - want2) <= (2 ** -8 if dt == "bf16" else 1e-7) * max(1, want2)
                assert row[3] == b + 1
    with pytest.raises(ValueError):
        ref.page_means(kv_off, sb_off + np.array([0, 1, 1, 1]), k, B)


def test_page_means_rounds_once(ref):
    # mean of bf16 values whose exact mean lies between two bf16 values: one rounding of the exact mean
    k = bf16(np.array([[1.0], [1.0 + 2 ** -7], [1.0 + 2 ** -7]], np.float32))
    m = ref.page_means(np.array([0, 3], np.int64), np.array([0, 1], np.int64), k, 4)
    exact = (1.0 + 2 * (1.0 + 2 ** -7)) / 3
    assert m[0, 0] == ref.double_to_bf16(exact)


# -------------------------------------------------------------------------------- a4/a5: HI


def test_page_score_with_unit_subblocks_sums_token_scores(ref):
    """B = 1: the page score is the sum of Eq. 1 over every token of the page (ties Eq. 9 to Eq. 1)."""
    rng = np.random.default_rng(9)
    L, P, HI, dI = 200, 16, 4, 8
    k = rng.standard_normal((L, dI)).astype(np.float32)
    q = rng.standard_normal((2, HI, dI)).astype(np.float32)
    w = rng.uniform(-0.5, 2, (2, HI)).astype(np.float32)
    rows = np.array([199, 100], np.int32)
    kv_off = one_seq(L)
    sb_off = np.array([0, L], np.int64)
    km = ref.page_means(kv_off, sb_off, k, 1)
    assert np.array_equal(km, k)
    ps = ref.page_scores(kv_off, sb_off, [0, 0], rows, q, w, km, P, 1, ld=15)
    for r, t in enumerate(rows):
        for p in range(15):
            if p > t // P or p >= (L + P - 1) // P:
                assert ps[r, p] == -np.inf
                continue
            want = sum(ref.score_one(q[r], w[r], k[s]) for s in range(p * P, min((p + 1) * P, L)))
            assert abs(ps[r, p] - want) <= 1e-6 * abs(want) + 1e-6


def test_page_score_constant_page_equals_token_score(ref):
    """B = P and every key of a page equal to c_p: page score = Eq. 1 at key c_p."""
    rng = np.random.default_rng(10)
    L, P, dI = 8 * 32, 32, 16
    c = rng.standard_normal((8, dI)).astype(np.float32)
    k = bf16(np.repeat(c, P, axis=0))
    q = bf16(rng.standard_normal((1, 4, dI)))
    w = rng.uniform(0.1, 2, (1, 4)).astype(np.float32)
    kv_off, sb_off = one_seq(L), np.array([0, 8], np.int64)
    km = ref.page_means(kv_off, sb_off, k, P)
    assert np.array_equal(km, k[::P])
    ps = ref.page_scores(kv_off, sb_off, [0], [L - 1], q, w, km, P, P, ld=8)
    for p in range(8):
        assert ps[0, p] == np.float32(ref.score_one(q[0], w[0], k[p * P]))


def test_page_recall_is_topM_of_page_scores(ref):
    rng = np.random.default_rng(11)
    L, P, B, M = 1000, 16, 4, 7
    k = rng.standard_normal((L, 8)).astype(np.float32)
    q = rng.standard_normal((3, 2, 8)).astype(np.float32)
    w = rng.uniform(0.1, 2, (3, 2)).astype(np.float32)
    rows = np.array([999, 500, 40], np.int32)
    kv_off = one_seq(L)
    sb_off = np.array([0, (L + B - 1) // B], np.int64)
    km = ref.page_means(kv_off, sb_off, k, B)
    pages, ps = ref.page_recall(kv_off, sb_off, [0, 0, 0], rows, q, w, km, P, B, M)
    assert np.array_equal(pages, _sort_topk(ps, M))
    assert list(pages[2]) == [0, 1, 2, -1, -1, -1, -1]            # t = 40: only pages 0..2 are causal


# -------------------------------------------------------------------------------- a8-a10: attention


def _dense_attn(q, kv, t, Dv, scale):
    """Textbook causal softmax attention of one query over keys 0..t (scipy's logsumexp)."""
    from scipy.special import logsumexp
    z = scale * (kv[:t + 1] @ q)
    lse = logsumexp(z)
    return np.exp(z - lse) @ kv[:t + 1, :Dv], lse


def test_attention_dense_when_budget_covers_prefix(ref):
    rng = np.random.default_rng(12)
    L, H, Dqk, Dv = 64, 3, 24, 16
    ks, kw = 4, 8
    kv = rng.standard_normal((L, Dqk)).astype(np.float32)
    rows = np.array([0, 3, 4, 11, 12, 13, 40, 63], np.int32)
    q = rng.standard_normal((len(rows), H, Dqk)).astype(np.float32)
    idx = np.full((len(rows), L), -1, np.int32)
    for i, t in enumerate(rows):
        mid = np.arange(ks, t - kw + 1)
        idx[i, :len(mid)] = rng.permutation(mid)                  # unsorted on purpose
    scale = 0.37
    out, lse = ref.hybrid_attn(one_seq(L), np.zeros(len(rows)), rows, q, kv, Dv, scale, ks, kw, idx)
    for i, t in enumerate(rows):
        for h in range(H):
            o, l = _dense_attn(q[i, h].astype(np.float64), kv.astype(np.float64), t, Dv, scale)
            assert np.allclose(out[i, h], o, rtol=1e-6, atol=1e-6)
            assert lse[i, h] == pytest.approx(l, rel=1e-6)


def test_attention_single_key_and_zero_query(ref):
    rng = np.random.default_rng(13)
    L, Dqk, Dv = 30, 12, 8
    kv = rng.standard_normal((L, Dqk)).astype(np.float32)
    q = rng.standard_normal((2, 2, Dqk)).astype(np.float32)
    q[1] = 0.0
    idx = np.full((2, 4), -1, np.int32)
    idx[1] = [7, 9, -1, 3]
    out, lse = ref.hybrid_attn(one_seq(L), [0, 0], [0, 25], q, kv, Dv, 0.5, 4, 10, idx)
    # row 0: t = 0 -> S = {0}: out = V row 0, lse = the single logit
    for h in range(2):
        assert np.allclose(out[0, h], kv[0, :Dv], rtol=1e-7)
        assert lse[0, h] == pytest.approx(0.5 * float(np.dot(q[0, h].astype(np.float64), kv[0].astype(np.float64))),
                                          rel=1e-6)
    # row 1: q = 0 -> uniform weights over S = sink 0..3, window 16..25, picks 7, 9 (3 is in the sink)
    S = [0, 1, 2, 3, 7, 9] + list(range(16, 26))
    for h in range(2):
        assert np.allclose(out[1, h], kv[S, :Dv].astype(np.float64).mean(0), rtol=1e-6, atol=1e-7)
        assert lse[1, h] == pytest.approx(math.log(len(S)), rel=1e-7)


def test_attention_split_merge_identity(ref):
    """Online-softmax merge of two disjoint parts of S equals attention over the union."""
    rng = np.random.default_rng(14)
    L, H, Dqk, Dv = 300, 2, 20, 12
    kv = rng.standard_normal((L, Dqk)).astype(np.float32)
    q = rng.standard_normal((1, H, Dqk)).astype(np.float32)
    t = 299
    picks = np.sort(rng.choice(np.arange(8, t - 16 + 1), 40, replace=False)).astype(np.int32)
    full_o, full_l = ref.hybrid_attn(one_seq(L), [0], [t], q, kv, Dv, 0.3, 8, 16, picks[None])
    # part A: sink + window only (no picks); part B: picks only (no sink, no window)
    a_o, a_l = ref.hybrid_attn(one_seq(L), [0], [t], q, kv, Dv, 0.3, 8, 16, np.full((1, 1), -1, np.int32))
    b_o, b_l = ref.hybrid_attn(one_seq(L), [0], [t], q, kv, Dv, 0.3, 0, 0, picks[None])
    m = np.maximum(a_l, b_l).astype(np.float64)
    wa, wb = np.exp(a_l - m), np.exp(b_l - m)
    merged = (wa[..., None] * a_o + wb[..., None] * b_o) / (wa + wb)[..., None]
    assert np.allclose(merged, full_o, rtol=1e-5, atol=1e-6)
    assert np.allclose(m + np.log(wa + wb), full_l, rtol=1e-6)


def test_attention_ignores_picks_outside_mid_and_repeats(ref):
    rng = np.random.default_rng(15)
    L = 200
    kv = rng.standard_normal((L, 16)).astype(np.float32)
    q = rng.standard_normal((1, 2, 16)).astype(np.float32)
    clean = np.array([[20, 50, 77, -1, -1, -1, -1, -1]], np.int32)
    noisy = np.array([[77, 2, 50, 190, 20, 50, 500, -7]], np.int32)   # sink, window, beyond, repeats
    o1, l1 = ref.hybrid_attn(one_seq(L), [0], [199], q, kv, 8, 0.25, 4, 16, clean)
    o2, l2 = ref.hybrid_attn(one_seq(L), [0], [199], q, kv, 8, 0.25, 4, 16, noisy)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_attention_bf16_output_is_rounded_fp64_result(ref):
    rng = np.random.default_rng(16)
    L = 40
    kv32 = rng.standard_normal((L, 16)).astype(np.float32)
    q32 = rng.standard_normal((1, 1, 16)).astype(np.float32)
    kv, q = bf16(kv32), bf16(q32)
    o, _ = ref.hybrid_attn(one_seq(L), [0], [39], q, kv, 8, 0.5, 40, 0, np.full((1, 1), -1, np.int32))
    of, _ = ref.hybrid_attn(one_seq(L), [0], [39], dec(ref, q).astype(np.float32), dec(ref, kv).astype(np.float32),
                            8, 0.5, 40, 0, np.full((1, 1), -1, np.int32))
    # the fp32 result is the same fp64 value rounded to fp32; bf16 rounding of it is within half a bf16 ulp
    got = dec(ref, o)[0, 0]
    assert np.all(np.abs(got - of[0, 0]) <= np.abs(of[0, 0]) * 2 ** -8 + 1e-30)


# -------------------------------------------------------------------------------- selected set


def test_selected_set_invariants(ref):
    rng = np.random.default_rng(17)
    L, ks, kw, kp = 3000, 16, 1024, 64
    rows = np.array([0, 5, 15, 16, 500, 1039, 1040, 1041, 1100, 2999], np.int32)
    k = rng.standard_normal((L, 8)).astype(np.float32)
    q = rng.standard_normal((len(rows), 2, 8)).astype(np.float32)
    w = np.ones((len(rows), 2), np.float32)
    sc = ref.index_score(one_seq(L), np.zeros(len(rows)), rows, q, w, k, ks, kw, ld=L)
    idx = ref.topk(sc, kp)
    for r, t in enumerate(rows):
        S = ref.selected_set(one_seq(L), np.zeros(len(rows)), rows, ks, kw, idx, r)
        (a0, a1), (b0, b1), (c0, c1) = ref.ranges(t, L, ks, kw)
        assert len(S) == min(ks + kw + kp, t + 1)                 # |S_t| = min(K, t + 1)
        assert len(set(S.tolist())) == len(S)
        assert set(range(a0, a1)) <= set(S.tolist())              # sink always present
        assert set(range(b0, b1)) <= set(S.tolist())              # window always present
        sparse = set(S.tolist()) - set(range(a0, a1)) - set(range(b0, b1))
        assert sparse <= set(range(c0, c1))                        # sparse picks only from mid(t)


# -------------------------------------------------------------------------------- layer: HI, CLI, MTP


def _layer_inputs(rng, lens, HI=2, dI=8, H=2, Dqk=16):
    kv_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    tot = int(kv_off[-1])
    n = len(lens)
    return dict(kv_off=kv_off, row_seq=np.arange(n, dtype=np.int32),
                row_pos=np.array([L - 1 for L in lens], np.int32),
                q_idx=bf16(rng.standard_normal((n, HI, dI)) / math.sqrt(dI)),
                w=rng.uniform(0.1, 2, (n, HI)).astype(np.float32),
                k_idx=bf16(rng.standard_normal((tot, dI)) / math.sqrt(dI)),
                q=bf16(rng.standard_normal((n, H, Dqk))), kv=bf16(rng.standard_normal((tot, Dqk))))


def _cfg(**kw):
    c = dict(HI=2, dI=8, H=2, Dqk=16, Dv=8, scale=0.25, k_sink=4, k_swa=16, k_sparse=12, P=16, B=16, M=64,
             hi_min_len=1 << 62, is_owner=1)
    c.update(kw)
    return c


def test_hi_with_full_recall_equals_flat(ref):
    """M*P >= L: every causal page is recalled, so HI selects exactly what the flat indexer selects."""
    rng = np.random.default_rng(18)
    lens = [500, 733, 64, 1000]
    x = _layer_inputs(rng, lens)
    for B in (16, 4, 1):
        sb_off = np.concatenate([[0], np.cumsum([(L + B - 1) // B for L in lens])]).astype(np.int64)
        km = ref.page_means(x["kv_off"], sb_off, x["k_idx"], B)
        flat = ref.layer_fwd(_cfg(B=B), **x)
        hi = ref.layer_fwd(_cfg(B=B, hi_min_len=0), sb_off=sb_off, k_mean=km, **x)
        assert np.array_equal(flat[0], hi[0])
        assert np.array_equal(flat[1], hi[1]) and np.array_equal(flat[2], hi[2])


def test_hi_gate_by_length(ref):
    """Only sequences with L >= hi_min_len take the HI path (M small, so HI can differ from flat)."""
    rng = np.random.default_rng(19)
    lens = [900, 300]
    x = _layer_inputs(rng, lens)
    sb_off = np.concatenate([[0], np.cumsum([(L + 15) // 16 for L in lens])]).astype(np.int64)
    km = ref.page_means(x["kv_off"], sb_off, x["k_idx"], 16)
    flat = ref.layer_fwd(_cfg(M=2), **x)
    gated = ref.layer_fwd(_cfg(M=2, hi_min_len=800), sb_off=sb_off, k_mean=km, **x)
    assert np.array_equal(flat[0][1], gated[0][1])                    # L = 300 < 800: flat
    all_hi = ref.layer_fwd(_cfg(M=2, hi_min_len=0), sb_off=sb_off, k_mean=km, **x)
    assert np.array_equal(all_hi[0][0], gated[0][0])                  # L = 900: HI
    # HI picks only from the 2 recalled pages (tokens of at most 2 pages of 16)
    pages = set(int(s) // 16 for s in gated[0][0] if s >= 0)
    assert len(pages) <= 2


def test_cli_reuse_with_owner_inputs_is_identical(ref):
    rng = np.random.default_rng(20)
    x = _layer_inputs(rng, [400, 130])
    idx, out, lse = ref.layer_fwd(_cfg(), **x)
    r_idx, r_out, r_lse = ref.layer_fwd(_cfg(is_owner=0), idx=idx, **x)
    assert np.array_equal(r_idx, idx) and np.array_equal(r_out, out) and np.array_equal(r_lse, lse)


def test_mtp_drafts_share_the_first_drafts_index(ref):
    rng = np.random.default_rng(21)
    lens = [300, 260]
    x = _layer_inputs(rng, lens)
    # three drafts per sequence, all at t = L - 1; drafts 1, 2 reuse draft 0's index row
    rep = lambda a: np.repeat(a, 3, axis=0)
    y = dict(kv_off=x["kv_off"], row_seq=rep(x["row_seq"]), row_pos=rep(x["row_pos"]), q_idx=rep(x["q_idx"]),
             w=rep(x["w"]), k_idx=x["k_idx"], q=rep(x["q"]), kv=x["kv"])
    y["q_idx"][1] = bf16(rng.standard_normal((2, 8)))      # a draft's own indexer query must be ignored
    idx_row = np.array([0, 0, 0, 3, 3, 3], np.int32)
    idx, out, lse = ref.layer_fwd(_cfg(), idx_row=idx_row, **y)
    base = ref.layer_fwd(_cfg(), **x)
    assert np.array_equal(idx[0], base[0][0]) and np.array_equal(idx[3], base[0][1])
    for r in range(6):
        assert np.array_equal(out[r], base[1][r // 3]) and np.array_equal(lse[r], base[2][r // 3])
