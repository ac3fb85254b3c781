"""CPU oracle for one LongCat Sparse Attention layer forward (TEST INFRASTRUCTURE ONLY).

Thin ctypes wrapper around ``oracle/liblsa_ref.so`` (plain C, fp64), built by ``oracle/build.py``.
Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this module.
The HIP library never imports it, and it never imports the HIP library.

Array conventions: numpy, C-contiguous.  bf16 tensors travel as ``np.uint16`` raw bits
(dtype code 1); fp32 tensors as ``np.float32`` (dtype code 0).  Positions are 0-indexed.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32 = 0
BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib():
    global _lib
    if _lib is None:
        # LSA_ORACLE_LIB: another build of the same source (the sanitizer build of build.py --sanitize)
        path = os.environ.get("LSA_ORACLE_LIB") or os.path.join(_HERE, "liblsa_ref.so")
        if not os.path.exists(path):
            _build.build()
        _lib = ctypes.CDLL(path)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_D = ctypes.c_double


def _declare(L):
    L.lsa_ref_double_to_bf16.argtypes = [_D]
    L.lsa_ref_double_to_bf16.restype = ctypes.c_uint16
    L.lsa_ref_ranges.argtypes = [_L, _L, _L, _L, _P]
    L.lsa_ref_ranges.restype = None
    L.lsa_ref_score_one.argtypes = [_I, _P, _P, _P, _I, _I]
    L.lsa_ref_score_one.restype = _D
    L.lsa_ref_index_score.argtypes = [_I, _P, _I, _P, _P, _P, _P, _P, _I, _I, _L, _L, _P, _L, _L, _P, _L,
                                      _P, _I]
    L.lsa_ref_index_score.restype = None
    L.lsa_ref_topk.argtypes = [_P, _I, _L, _L, _P, _L, _L, _L, _P, _P, _I]
    L.lsa_ref_topk.restype = _I
    L.lsa_ref_page_means.argtypes = [_I, _I, _P, _P, _P, _I, _L, _P]
    L.lsa_ref_page_means.restype = _I
    L.lsa_ref_page_scores.argtypes = [_I, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _L, _L, _P, _L, _P, _I]
    L.lsa_ref_page_scores.restype = None
    L.lsa_ref_page_recall.argtypes = [_I, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _L, _L, _L, _P, _L, _P,
                                      _P, _I]
    L.lsa_ref_page_recall.restype = _I
    L.lsa_ref_hybrid_attn.argtypes = [_I, _P, _I, _P, _P, _P, _P, _I, _I, _I, _D, _L, _L, _L, _P, _P, _P,
                                      _P, _I]
    L.lsa_ref_hybrid_attn.restype = _I
    L.lsa_ref_selected_set.argtypes = [_P, _P, _P, _L, _L, _L, _P, _P, _L, _P]
    L.lsa_ref_selected_set.restype = _L
    L.lsa_ref_layer_fwd.argtypes = ([_I] * 6 + [_D] + [_L] * 7 + [_I, _I, _P, _I] + [_P] * 14 + [_L, _P, _L,
                                    _P, _P, _I])
    L.lsa_ref_layer_fwd.restype = _I


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def _dt(a):
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle takes bf16 bits (uint16) or float32, got {a.dtype}")


def default_threads():
    return max(1, min(16, os.cpu_count() or 1))


# ------------------------------------------------------------------------------------ scalars

def double_to_bf16(x: float) -> int:
    return int(lib().lsa_ref_double_to_bf16(float(x)))


def ranges(t, L, k_sink, k_swa):
    """(sink, swa, mid) half-open ranges of a row at position t in a sequence of L tokens."""
    out = np.zeros(6, np.int64)
    lib().lsa_ref_ranges(int(t), int(L), int(k_sink), int(k_swa), _ptr(out))
    return (int(out[0]), int(out[1])), (int(out[2]), int(out[3])), (int(out[4]), int(out[5]))


def score_one(q_row, w_row, k_vec):
    """Eq. 1 for one (query row, key): q_row [HI, dI], w_row [HI] fp32, k_vec [dI]; returns float64."""
    q_row = np.ascontiguousarray(q_row)
    k_vec = np.ascontiguousarray(k_vec, dtype=q_row.dtype)
    w_row = _c(w_row, np.float32)
    HI, dI = q_row.shape
    return float(lib().lsa_ref_score_one(_dt(q_row), _ptr(q_row), _ptr(w_row), _ptr(k_vec), HI, dI))


# ------------------------------------------------------------------------------------ path steps

def index_score(kv_off, row_seq, row_pos, q_idx, w, k_idx, k_sink, k_swa, ld, pages=None, P=1,
                only=None, threads=None):
    """scores [n_rows, ld] fp32 (flat, or page-mapped when ``pages`` [n_rows, M] is given)."""
    kv_off = _c(kv_off, np.int64)
    row_seq = _c(row_seq, np.int32)
    row_pos = _c(row_pos, np.int32)
    q_idx = np.ascontiguousarray(q_idx)
    k_idx = np.ascontiguousarray(k_idx, dtype=q_idx.dtype)
    w = _c(w, np.float32)
    n_rows, HI, dI = q_idx.shape
    pages = _c(pages, np.int32)
    M = 0 if pages is None else pages.shape[1]
    only = _c(only, np.int32)
    out = np.empty((n_rows, ld), np.float32)
    lib().lsa_ref_index_score(_dt(q_idx), _ptr(kv_off), n_rows, _ptr(row_seq), _ptr(row_pos), _ptr(q_idx),
                              _ptr(w), _ptr(k_idx), HI, dI, int(k_sink), int(k_swa), _ptr(pages), M, int(P),
                              _ptr(out), int(ld), _ptr(only), threads or default_threads())
    return out


def topk(scores, K, pages=None, P=1, n_cols=None, threads=None):
    """idx [n_rows, K] int32: ascending positions of the K best finite scores (-1 padded)."""
    scores = _c(scores, np.float32)
    n_rows, ld = scores.shape
    n_cols = ld if n_cols is None else n_cols
    pages = _c(pages, np.int32)
    M = 0 if pages is None else pages.shape[1]
    idx = np.empty((n_rows, K), np.int32)
    st = lib().lsa_ref_topk(_ptr(scores), n_rows, ld, int(n_cols), _ptr(pages), M, int(P), int(K), _ptr(idx),
                            None, threads or default_threads())
    if st != 0:
        raise ValueError("oracle topk: NaN score or allocation failure")
    return idx


def page_means(kv_off, sb_off, k_idx, B):
    kv_off = _c(kv_off, np.int64)
    sb_off = _c(sb_off, np.int64)
    k_idx = np.ascontiguousarray(k_idx)
    dI = k_idx.shape[1]
    out = np.empty((int(sb_off[-1]), dI), k_idx.dtype)
    st = lib().lsa_ref_page_means(_dt(k_idx), len(kv_off) - 1, _ptr(kv_off), _ptr(sb_off), _ptr(k_idx), dI,
                                  int(B), _ptr(out))
    if st != 0:
        raise ValueError("oracle page_means: sb_off does not match ceil(L/B)")
    return out


def page_scores(kv_off, sb_off, row_seq, row_pos, q_idx, w, k_mean, P, B, ld, threads=None):
    kv_off, sb_off = _c(kv_off, np.int64), _c(sb_off, np.int64)
    row_seq, row_pos = _c(row_seq, np.int32), _c(row_pos, np.int32)
    q_idx = np.ascontiguousarray(q_idx)
    k_mean = np.ascontiguousarray(k_mean, dtype=q_idx.dtype)
    w = _c(w, np.float32)
    n_rows, HI, dI = q_idx.shape
    out = np.empty((n_rows, ld), np.float32)
    lib().lsa_ref_page_scores(_dt(q_idx), _ptr(kv_off), _ptr(sb_off), n_rows, _ptr(row_seq), _ptr(row_pos),
                              _ptr(q_idx), _ptr(w), _ptr(k_mean), HI, dI, int(P), int(B), _ptr(out), int(ld),
                              None, threads or default_threads())
    return out


def page_recall(kv_off, sb_off, row_seq, row_pos, q_idx, w, k_mean, P, B, M, ld=None, threads=None):
    """pages [n_rows, M] int32 (ascending, -1 padded) and the page scores [n_rows, ld]."""
    kv_off, sb_off = _c(kv_off, np.int64), _c(sb_off, np.int64)
    row_seq, row_pos = _c(row_seq, np.int32), _c(row_pos, np.int32)
    q_idx = np.ascontiguousarray(q_idx)
    k_mean = np.ascontiguousarray(k_mean, dtype=q_idx.dtype)
    w = _c(w, np.float32)
    n_rows, HI, dI = q_idx.shape
    if ld is None:
        ld = int(max((kv_off[b + 1] - kv_off[b] + P - 1) // P for b in range(len(kv_off) - 1)))
    ws = np.empty((n_rows, ld), np.float32)
    pages = np.empty((n_rows, M), np.int32)
    st = lib().lsa_ref_page_recall(_dt(q_idx), _ptr(kv_off), _ptr(sb_off), n_rows, _ptr(row_seq),
                                   _ptr(row_pos), _ptr(q_idx), _ptr(w), _ptr(k_mean), HI, dI, int(P), int(B),
                                   int(M), _ptr(ws), int(ld), _ptr(pages), None, threads or default_threads())
    if st != 0:
        raise ValueError("oracle page_recall failed")
    return pages, ws


def hybrid_attn(kv_off, row_seq, row_pos, q, kv, Dv, scale, k_sink, k_swa, idx, idx_row=None,
                threads=None):
    """(out [n_rows, H, Dv] in q's dtype, lse [n_rows, H] fp32)."""
    kv_off = _c(kv_off, np.int64)
    row_seq, row_pos = _c(row_seq, np.int32), _c(row_pos, np.int32)
    q = np.ascontiguousarray(q)
    kv = np.ascontiguousarray(kv, dtype=q.dtype)
    idx = _c(idx, np.int32)
    idx_row = _c(idx_row, np.int32)
    n_rows, H, Dqk = q.shape
    k_sparse = idx.shape[1]
    out = np.empty((n_rows, H, Dv), q.dtype)
    lse = np.empty((n_rows, H), np.float32)
    st = lib().lsa_ref_hybrid_attn(_dt(q), _ptr(kv_off), n_rows, _ptr(row_seq), _ptr(row_pos), _ptr(q),
                                   _ptr(kv), H, Dqk, int(Dv), float(scale), int(k_sink), int(k_swa),
                                   int(k_sparse), _ptr(idx), _ptr(idx_row), _ptr(out), _ptr(lse),
                                   threads or default_threads())
    if st != 0:
        raise MemoryError("oracle hybrid_attn allocation failure")
    return out, lse


def selected_set(kv_off, row_seq, row_pos, k_sink, k_swa, idx, r, idx_row=None):
    kv_off = _c(kv_off, np.int64)
    row_seq, row_pos = _c(row_seq, np.int32), _c(row_pos, np.int32)
    idx = _c(idx, np.int32)
    idx_row = _c(idx_row, np.int32)
    k_sparse = idx.shape[1]
    buf = np.empty(k_sink + k_swa + k_sparse + 1, np.int64)
    n = lib().lsa_ref_selected_set(_ptr(kv_off), _ptr(row_seq), _ptr(row_pos), int(k_sink), int(k_swa),
                                   int(k_sparse), _ptr(idx), _ptr(idx_row), int(r), _ptr(buf))
    return buf[:n].copy()


def layer_fwd(cfg, kv_off, row_seq, row_pos, q_idx, w, k_idx, q, kv, idx=None, idx_row=None, sb_off=None,
              k_mean=None, threads=None):
    """One layer: returns (idx [n_rows, Ksparse], out, lse).

    cfg keys: HI, dI, H, Dqk, Dv, scale, k_sink, k_swa, k_sparse, P, B, M, hi_min_len, is_owner.
    """
    kv_off = _c(kv_off, np.int64)
    row_seq, row_pos = _c(row_seq, np.int32), _c(row_pos, np.int32)
    q = np.ascontiguousarray(q)
    kv = np.ascontiguousarray(kv, dtype=q.dtype)
    n_rows = q.shape[0]
    H, Dqk = q.shape[1], q.shape[2]
    dt = _dt(q)
    owner = int(cfg["is_owner"])
    k_sparse = int(cfg["k_sparse"])
    if owner:
        q_idx = np.ascontiguousarray(q_idx, dtype=q.dtype)
        k_idx = np.ascontiguousarray(k_idx, dtype=q.dtype)
        w = _c(w, np.float32)
        idx = np.full((n_rows, k_sparse), -1, np.int32) if idx is None else _c(idx, np.int32).copy()
    else:
        idx = _c(idx, np.int32)
    idx_row = _c(idx_row, np.int32)
    lens = np.diff(kv_off)
    max_len = int(lens.max())
    P, B, M = int(cfg.get("P", 128)), int(cfg.get("B", 128)), int(cfg.get("M", 1024))
    use_hi = owner and k_mean is not None
    flat_ws = np.empty((n_rows, max_len), np.float32) if owner else None
    max_pages = int((max_len + P - 1) // P)
    page_ws = np.empty((n_rows, max_pages), np.float32) if use_hi else None
    pages_ws = np.empty((n_rows, M), np.int32) if use_hi else None
    comp_ws = np.empty((n_rows, M * P), np.float32) if use_hi else None
    if use_hi:
        sb_off = _c(sb_off, np.int64)
        k_mean = np.ascontiguousarray(k_mean, dtype=q.dtype)
    out = np.empty((n_rows, H, int(cfg["Dv"])), q.dtype)
    lse = np.empty((n_rows, H), np.float32)
    st = lib().lsa_ref_layer_fwd(
        dt, int(cfg.get("HI", 0)), int(cfg.get("dI", 0)), H, Dqk, int(cfg["Dv"]), float(cfg["scale"]),
        int(cfg["k_sink"]), int(cfg["k_swa"]), k_sparse, P, B, M, int(cfg.get("hi_min_len", 1 << 62)), owner,
        len(kv_off) - 1, _ptr(kv_off), n_rows, _ptr(row_seq), _ptr(row_pos), _ptr(idx_row),
        _ptr(q_idx) if owner else None, _ptr(w) if owner else None, _ptr(k_idx) if owner else None,
        _ptr(sb_off) if use_hi else None, _ptr(k_mean) if use_hi else None, _ptr(q), _ptr(kv), _ptr(idx),
        _ptr(out), _ptr(lse), _ptr(flat_ws), max_len, _ptr(page_ws), max_pages, _ptr(pages_ws), _ptr(comp_ws),
        threads or default_threads())
    if st != 0:
        raise ValueError(f"oracle layer_fwd failed ({st})")
    return idx, out, lse


# ------------------------------------------------------------------------------------ bf16 helpers

def bf16_bits_to_f64(a):
    """Exact decode of bf16 raw bits (uint16) to float64."""
    a = np.asarray(a, np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
