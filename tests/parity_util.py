"""Helpers of the GPU parity tests: comparisons at the tolerances the acceptance criteria fix.

  * indexer / page scores: |g - o| <= 1e-4 + 2e-3 |o| elementwise, -inf at identical positions
  * top-K fed the oracle's scores: bit-exact indices
  * attention fed the oracle's indices: max |g - o| <= 2e-2 (bf16) or 1e-4 (fp32); lse within
    1e-4 * max(1, |lse|)
  * end-to-end index sets: equal, except positions whose oracle score lies within 1e-3 (relative)
    of the oracle's K-th best score (a near-tie the two sides may order differently)
"""
import sys

import numpy as np
import torch

import long_context_sparse_weighted_amd as lsa
import synth


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return synth.to_host(t)


def rows_of(x):
    return lsa.RowsDesc(x["kv_off"], x["row_seq"], x["row_pos"], x["max_len"])


def f64(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def assert_scores_close(g, o, what="scores"):
    g = np.asarray(g, np.float32)
    o = np.asarray(o, np.float32)
    assert g.shape == o.shape, (g.shape, o.shape)
    gi, oi = np.isneginf(g), np.isneginf(o)
    bad = np.argwhere(gi != oi)
    assert bad.size == 0, f"{what}: -inf pattern differs at {bad[:5].tolist()}"
    fin = ~oi
    err = np.abs(g[fin].astype(np.float64) - o[fin])
    tol = 1e-4 + 2e-3 * np.abs(o[fin].astype(np.float64))
    worst = float((err / tol).max()) if err.size else 0.0
    assert worst <= 1.0, f"{what}: max err/tol = {worst:.3f}"
    return worst


def assert_idx_sets_match(g_idx, o_idx, accept_fn, what="idx"):
    """g_idx / o_idx [n_rows, K], ascending with -1 padding.  Rows must agree except at positions
    accept_fn(r, positions) -> bool array marks as near-ties of the oracle's ranking."""
    n_diff_rows = 0
    for r in range(o_idx.shape[0]):
        g = g_idx[r][g_idx[r] >= 0]
        o = o_idx[r][o_idx[r] >= 0]
        assert np.all(np.diff(g) > 0), f"{what}: row {r} not strictly ascending"
        if np.array_equal(g, o):
            continue
        n_diff_rows += 1
        assert len(g) == len(o), f"{what}: row {r} sizes {len(g)} vs {len(o)}"
        diff = np.setxor1d(g, o)
        ok = np.asarray(accept_fn(r, diff), bool)
        assert ok.all(), f"{what}: row {r} differs at {diff[~ok][:8].tolist()} beyond the near-tie band"
    return n_diff_rows


def near_tie(scores, theta, rel=1e-3):
    return np.abs(np.asarray(scores, np.float64) - theta) <= rel * abs(theta)


def kth_best(row_scores, K):
    fin = row_scores[np.isfinite(row_scores)]
    if len(fin) == 0:
        return np.nan
    K = min(K, len(fin))
    return float(np.partition(fin.astype(np.float64), len(fin) - K)[len(fin) - K])


def assert_attn_close(g_out, o_out, g_lse, o_lse, tol, what="attn"):
    go, oo = f64(g_out), f64(o_out)
    err = float(np.abs(go - oo).max()) if go.size else 0.0
    assert err <= tol, f"{what}: max |out err| = {err:.3e} > {tol}"
    gl, ol = np.asarray(g_lse, np.float64), np.asarray(o_lse, np.float64)
    both_inf = np.isneginf(gl) & np.isneginf(ol)
    gl0, ol0 = np.where(both_inf, 0.0, gl), np.where(both_inf, 0.0, ol)  # (-inf on both sides agrees)
    lerr = np.abs(gl0 - ol0)
    ltol = 1e-4 * np.maximum(1.0, np.abs(ol0))
    worst = float((lerr / ltol).max()) if lerr.size else 0.0
    assert worst <= 1.0, f"{what}: lse err/tol = {worst:.3f}"
    return err


def budget_of(cfg):
    return (int(cfg["k_sink"]), int(cfg["k_swa"]), int(cfg["k_sparse"]))


def oracle_inputs(x):
    """Host copies (oracle convention) of a synth workload."""
    out = {k: host(x[k]) for k in ("q_idx", "w", "k_idx", "q", "kv") if x.get(k) is not None}
    out["kv_off"] = x["kv_off_host"].numpy()
    out["row_seq"] = x["row_seq_host"].numpy()
    out["row_pos"] = x["row_pos_host"].numpy()
    return out


def torch_sync():
    torch.cuda.synchronize()
