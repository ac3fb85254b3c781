"""Python binding of liblsa (include/lsa.h): the MI355X LongCat Sparse Attention layer forward.

Argument marshalling only: every step runs in the HIP kernels of liblsa.so.  Tensors are torch
tensors on the GPU (bf16 or fp32 as documented in lsa.h); work is enqueued on torch's current
stream.  Importing this module fails loudly when liblsa.so has not been built; no CPU fallback
exists.
"""
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LSA_LIB: another build of the same sources (e.g. the host-sanitizer build of the CPU tests)
LIB_PATH = os.environ.get("LSA_LIB") or os.path.join(_HERE, "liblsa.so")

LSA_OK, LSA_ERR_INVALID, LSA_ERR_UNSUPPORTED, LSA_ERR_WORKSPACE, LSA_ERR_HIP = range(5)
LSA_F32, LSA_BF16 = 0, 1

SYMBOLS = ("lsa_index_score", "lsa_quantize_fp8", "lsa_index_score_fp8", "lsa_page_means", "lsa_page_means_append", "lsa_page_recall", "lsa_page_recall_workspace_size", "lsa_topk",
           "lsa_topk_workspace_size", "lsa_index_topk", "lsa_index_topk_workspace_size", "lsa_index_topk_noalloc",
           "lsa_index_topk_fp8", "lsa_index_topk_fp8_workspace_size", "lsa_hybrid_attn", "lsa_hybrid_attn_workspace_size", "lsa_layer_fwd",
           "lsa_layer_workspace_size", "lsa_status_string", "lsa_last_error")


class LsaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (status {code})")
        self.code = code


class Rows(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("n_rows", ctypes.c_int32), ("kv_off", ctypes.c_void_p),
                ("row_seq", ctypes.c_void_p), ("row_pos", ctypes.c_void_p), ("max_kv_len", ctypes.c_int64),
                ("min_kv_len", ctypes.c_int64)]


class Budget(ctypes.Structure):
    _fields_ = [("k_sink", ctypes.c_int32), ("k_swa", ctypes.c_int32), ("k_sparse", ctypes.c_int32)]


class LayerCfg(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("n_heads_idx", ctypes.c_int32), ("head_dim_idx", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("scale", ctypes.c_float), ("budget", Budget), ("P", ctypes.c_int32), ("B", ctypes.c_int32),
                ("M", ctypes.c_int32), ("hi_min_len", ctypes.c_int64), ("is_owner", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded liblsa.so (raises if it is missing: build it with __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        RP = ctypes.POINTER(Rows)
        L.lsa_index_score.argtypes = [ctypes.c_int, RP, P, P, P, I32, I32, Budget, P, I32, I32, P, I64, P]
        L.lsa_page_means.argtypes = [ctypes.c_int, I32, P, P, P, I32, I32, I64, I64, P, P]
        L.lsa_quantize_fp8.argtypes = [ctypes.c_int, I64, I32, P, P, P, P]
        L.lsa_index_score_fp8.argtypes = [RP, P, P, P, P, P, I32, I32, Budget, P, I32, I32, P, I64, P]
        L.lsa_page_means_append.argtypes = [ctypes.c_int, I32, P, P, P, I32, I32, I64, P, P]
        L.lsa_page_recall.argtypes = [ctypes.c_int, RP, P, P, P, P, I32, I32, I32, I32, I32, P, I64, P, P, SZ, P]
        L.lsa_page_recall_workspace_size.argtypes = [RP, I32, I32, ctypes.POINTER(SZ)]
        L.lsa_topk.argtypes = [I32, P, I64, I64, P, I32, I32, I32, P, P, SZ, P]
        L.lsa_topk_workspace_size.argtypes = [I32, I64, I32, ctypes.POINTER(SZ)]
        L.lsa_index_topk.argtypes = [ctypes.c_int, RP, P, P, P, I32, I32, Budget, P, P, SZ, P]
        L.lsa_index_topk_workspace_size.argtypes = [ctypes.c_int, RP, I32, I32, I32, ctypes.POINTER(SZ)]
        L.lsa_index_topk_noalloc.argtypes = [ctypes.c_int, RP, P, P, P, I32, I32, Budget, P, P]
        L.lsa_index_topk_fp8.argtypes = [RP, P, P, P, P, P, I32, I32, Budget, P, P, SZ, P]
        L.lsa_index_topk_fp8_workspace_size.argtypes = [RP, I32, I32, I32, ctypes.POINTER(SZ)]
        L.lsa_hybrid_attn.argtypes = [ctypes.c_int, RP, P, P, I32, I32, I32, F, Budget, P, P, P, P, P, SZ, P]
        L.lsa_hybrid_attn_workspace_size.argtypes = [ctypes.c_int, RP, I32, I32, Budget, ctypes.POINTER(SZ)]
        L.lsa_layer_fwd.argtypes = [ctypes.POINTER(LayerCfg), RP, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.lsa_layer_workspace_size.argtypes = [ctypes.POINTER(LayerCfg), RP, I32, ctypes.POINTER(SZ)]
        for name in SYMBOLS:
            if name not in ("lsa_status_string", "lsa_last_error"):
                getattr(L, name).restype = ctypes.c_int
        L.lsa_status_string.argtypes = [ctypes.c_int]
        L.lsa_status_string.restype = ctypes.c_char_p
        L.lsa_last_error.argtypes = []
        L.lsa_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(code):
    if code != LSA_OK:
        L = lib()
        raise LsaError(code, f"{L.lsa_status_string(code).decode()}: {L.lsa_last_error().decode()}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t):
    if t.dtype == torch.bfloat16:
        return LSA_BF16
    if t.dtype == torch.float32:
        return LSA_F32
    raise TypeError(f"expected bf16 or fp32, got {t.dtype}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name):
    if t is None:
        return
    if not t.is_cuda or not t.is_contiguous() or t.dtype != dtype:
        raise ValueError(f"{name} must be a contiguous CUDA tensor of {dtype}")


@dataclass
class RowsDesc:
    """Rows of a batch: device tensors kv_off (int64 [n_seq+1]), row_seq / row_pos (int32 [n_rows]);
    max_kv_len bounds every sequence length from above, min_kv_len (0: not known) from below."""
    kv_off: torch.Tensor
    row_seq: torch.Tensor
    row_pos: torch.Tensor
    max_kv_len: int
    min_kv_len: int = 0

    def c(self):
        _need(self.kv_off, torch.int64, "kv_off")
        _need(self.row_seq, torch.int32, "row_seq")
        _need(self.row_pos, torch.int32, "row_pos")
        return Rows(self.kv_off.numel() - 1, self.row_pos.numel(), _p(self.kv_off), _p(self.row_seq),
                    _p(self.row_pos), int(self.max_kv_len), int(self.min_kv_len))


def _workspace(nbytes, device):
    n = max(int(nbytes), 1)
    return torch.empty(n + 256, dtype=torch.uint8, device=device)


def _aligned(ws):
    p = ws.data_ptr()
    return ctypes.c_void_p((p + 255) & ~255), ws.numel() - ((-p) & 255)


# ----------------------------------------------------------------------------------------- entry points


def lsa_index_score(rows: RowsDesc, q_idx, w, k_idx, budget, scores=None, pages=None, M=0, P=0, ld=None):
    """Indexer scores [n_rows, ld] fp32 (flat over positions, or page-mapped when ``pages`` is given)."""
    n_rows, HI, dI = q_idx.shape
    dt = _dt(q_idx)
    _need(k_idx, q_idx.dtype, "k_idx")
    _need(w, torch.float32, "w")
    if pages is not None:
        _need(pages, torch.int32, "pages")
        M = pages.shape[1]
        ld = ld or M * P
    else:
        ld = ld or max(int(rows.max_kv_len), 1)
    if scores is None:
        scores = torch.empty((n_rows, ld), dtype=torch.float32, device=q_idx.device)
    _check(lib().lsa_index_score(dt, ctypes.byref(rows.c()), _p(q_idx), _p(w), _p(k_idx), HI, dI, Budget(*budget),
                                 _p(pages), int(M), int(P), _p(scores), int(ld), _stream()))
    return scores


def lsa_quantize_fp8(x, codes=None, scale=None):
    """x [..., d] bf16 / fp32 -> (codes [..., d] uint8 E4M3, scale [...] fp32 powers of two)."""
    d = x.shape[-1]
    n_vec = x.numel() // d if d else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _check(lib().lsa_quantize_fp8(_dt(x), n_vec, d, _p(x), _p(codes), _p(scale), _stream()))
    return codes, scale


def lsa_index_score_fp8(rows: RowsDesc, q8, q_scale, w, k8, k_scale, budget, scores=None, pages=None, M=0, P=0,
                        ld=None):
    """Eq. 1 scores [n_rows, ld] fp32 from FP8 indexer inputs (flat, or page-mapped with ``pages``)."""
    n_rows, HI, dI = q8.shape
    _need(q8, torch.uint8, "q8")
    _need(k8, torch.uint8, "k8")
    for t, name in ((q_scale, "q_scale"), (k_scale, "k_scale"), (w, "w")):
        _need(t, torch.float32, name)
    if pages is not None:
        _need(pages, torch.int32, "pages")
        M = pages.shape[1]
        ld = ld or M * P
    else:
        ld = ld or max(int(rows.max_kv_len), 1)
    if scores is None:
        scores = torch.empty((n_rows, ld), dtype=torch.float32, device=q8.device)
    rc = rows.c()
    _check(lib().lsa_index_score_fp8(ctypes.byref(rc), _p(q8), _p(q_scale), _p(w), _p(k8), _p(k_scale), HI, dI,
                                     Budget(*budget), _p(pages), int(M), int(P), _p(scores), int(ld), _stream()))
    return scores


def lsa_page_means(kv_off, sb_off, k_idx, B, max_kv_len, k_mean=None, first_token=0):
    """Sub-block mean cache [sb_off[-1], d] of k_idx (bf16 / fp32)."""
    _need(kv_off, torch.int64, "kv_off")
    _need(sb_off, torch.int64, "sb_off")
    if k_mean is None:
        k_mean = torch.empty((int(sb_off[-1].item()), k_idx.shape[1]), dtype=k_idx.dtype, device=k_idx.device)
    _check(lib().lsa_page_means(_dt(k_idx), kv_off.numel() - 1, _p(kv_off), _p(sb_off), _p(k_idx), k_idx.shape[1],
                                int(B), int(max_kv_len), int(first_token), _p(k_mean), _stream()))
    return k_mean


def lsa_page_means_append(kv_off, sb_off, k_idx, B, k_mean, n_new=1):
    """Refresh, in place, the rows of k_mean for the sub-blocks holding each sequence's n_new newest
    tokens (kv_off / sb_off describe the lengths after appending)."""
    _need(kv_off, torch.int64, "kv_off")
    _need(sb_off, torch.int64, "sb_off")
    _check(lib().lsa_page_means_append(_dt(k_idx), kv_off.numel() - 1, _p(kv_off), _p(sb_off), _p(k_idx),
                                       k_idx.shape[1], int(B), int(n_new), _p(k_mean), _stream()))
    return k_mean


def lsa_page_recall(rows: RowsDesc, sb_off, q_idx, w, k_mean, P, B, M, page_scores=None):
    """(pages [n_rows, M] int32 ascending / -1 padded, page_scores [n_rows, ceil(max_len/P)] or None)."""
    n_rows, HI, dI = q_idx.shape
    rc = rows.c()
    sz = ctypes.c_size_t()
    _check(lib().lsa_page_recall_workspace_size(ctypes.byref(rc), int(P), int(M), ctypes.byref(sz)))
    ws = _workspace(sz.value, q_idx.device)
    wp, wn = _aligned(ws)
    pages = torch.empty((n_rows, M), dtype=torch.int32, device=q_idx.device)
    ld = page_scores.shape[1] if page_scores is not None else 0
    _check(lib().lsa_page_recall(_dt(q_idx), ctypes.byref(rc), _p(sb_off), _p(q_idx), _p(w), _p(k_mean), HI, dI,
                                 int(P), int(B), int(M), _p(page_scores), int(ld), _p(pages), wp, wn, _stream()))
    return pages, page_scores


def lsa_topk(scores, k, n_cols=None, pages=None, P=0, idx=None):
    """idx [n_rows, k] int32: ascending positions of the k best candidates of each row."""
    n_rows, ld = scores.shape
    n_cols = ld if n_cols is None else n_cols
    _need(scores, torch.float32, "scores")
    sz = ctypes.c_size_t()
    _check(lib().lsa_topk_workspace_size(n_rows, int(n_cols), int(k), ctypes.byref(sz)))
    ws = _workspace(sz.value, scores.device)
    wp, wn = _aligned(ws)
    if idx is None:
        idx = torch.empty((n_rows, k), dtype=torch.int32, device=scores.device)
    M = 0 if pages is None else pages.shape[1]
    _check(lib().lsa_topk(n_rows, _p(scores), ld, int(n_cols), _p(pages), M, int(P), int(k), _p(idx), wp, wn,
                          _stream()))
    return idx


def lsa_index_topk_workspace(rows: RowsDesc, q_idx, k_sparse):
    """A workspace tensor for lsa_index_topk on these rows (reusable across calls of the same shape)."""
    n_rows, HI, dI = q_idx.shape
    sz = ctypes.c_size_t()
    _check(lib().lsa_index_topk_workspace_size(_dt(q_idx), ctypes.byref(rows.c()), HI, dI, int(k_sparse),
                                               ctypes.byref(sz)))
    return _workspace(sz.value, q_idx.device)


def lsa_index_topk(rows: RowsDesc, q_idx, w, k_idx, budget, idx=None, ws=None):
    """idx [n_rows, k_sparse] int32: the flat token selection (indexer scores and top-K in one call)."""
    n_rows, HI, dI = q_idx.shape
    dt = _dt(q_idx)
    _need(k_idx, q_idx.dtype, "k_idx")
    _need(w, torch.float32, "w")
    bud = Budget(*budget)
    if ws is None:
        ws = lsa_index_topk_workspace(rows, q_idx, bud.k_sparse)
    wp, wn = _aligned(ws)
    if idx is None:
        idx = torch.empty((n_rows, bud.k_sparse), dtype=torch.int32, device=q_idx.device)
    _check(lib().lsa_index_topk(dt, ctypes.byref(rows.c()), _p(q_idx), _p(w), _p(k_idx), HI, dI, bud, _p(idx), wp,
                                wn, _stream()))
    return idx


def lsa_index_topk_noalloc(rows: RowsDesc, q_idx, w, k_idx, budget, idx=None):
    """lsa_index_topk with the library's own device scratch array: no workspace argument, no device
    allocation inside the call (idx must be passed in for that)."""
    n_rows, HI, dI = q_idx.shape
    dt = _dt(q_idx)
    _need(k_idx, q_idx.dtype, "k_idx")
    _need(w, torch.float32, "w")
    bud = Budget(*budget)
    if idx is None:
        idx = torch.empty((n_rows, bud.k_sparse), dtype=torch.int32, device=q_idx.device)
    _check(lib().lsa_index_topk_noalloc(dt, ctypes.byref(rows.c()), _p(q_idx), _p(w), _p(k_idx), HI, dI, bud,
                                        _p(idx), _stream()))
    return idx


def lsa_index_topk_fp8_workspace(rows: RowsDesc, q8, k_sparse):
    """A workspace tensor for lsa_index_topk_fp8 on these rows."""
    n_rows, HI, dI = q8.shape
    sz = ctypes.c_size_t()
    _check(lib().lsa_index_topk_fp8_workspace_size(ctypes.byref(rows.c()), HI, dI, int(k_sparse), ctypes.byref(sz)))
    return _workspace(sz.value, q8.device)


def lsa_index_topk_fp8(rows: RowsDesc, q8, q_scale, w, k8, k_scale, budget, idx=None, ws=None):
    """idx [n_rows, k_sparse] int32: the FP8 flat token selection (scores and top-K in one call)."""
    n_rows, HI, dI = q8.shape
    for t, dt, name in ((q8, torch.uint8, "q8"), (k8, torch.uint8, "k8"), (q_scale, torch.float32, "q_scale"),
                        (k_scale, torch.float32, "k_scale"), (w, torch.float32, "w")):
        _need(t, dt, name)
    bud = Budget(*budget)
    if ws is None:
        ws = lsa_index_topk_fp8_workspace(rows, q8, bud.k_sparse)
    wp, wn = _aligned(ws)
    if idx is None:
        idx = torch.empty((n_rows, bud.k_sparse), dtype=torch.int32, device=q8.device)
    _check(lib().lsa_index_topk_fp8(ctypes.byref(rows.c()), _p(q8), _p(q_scale), _p(w), _p(k8), _p(k_scale), HI, dI,
                                    bud, _p(idx), wp, wn, _stream()))
    return idx


def lsa_hybrid_attn(rows: RowsDesc, q, kv, d_v, scale, budget, idx, idx_row=None, out=None, lse=None):
    """(out [n_rows, H, d_v] in q's dtype, lse [n_rows, H] fp32)."""
    n_rows, H, d_qk = q.shape
    dt = _dt(q)
    _need(kv, q.dtype, "kv")
    _need(idx, torch.int32, "idx")
    rc = rows.c()
    bud = Budget(*budget)
    sz = ctypes.c_size_t()
    _check(lib().lsa_hybrid_attn_workspace_size(dt, ctypes.byref(rc), H, int(d_v), bud, ctypes.byref(sz)))
    ws = _workspace(sz.value, q.device)
    wp, wn = _aligned(ws)
    if out is None:
        out = torch.empty((n_rows, H, d_v), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((n_rows, H), dtype=torch.float32, device=q.device)
    _check(lib().lsa_hybrid_attn(dt, ctypes.byref(rc), _p(q), _p(kv), H, d_qk, int(d_v), float(scale), bud, _p(idx),
                                 _p(idx_row), _p(out), _p(lse), wp, wn, _stream()))
    return out, lse


def layer_cfg(cfg: dict, dtype) -> LayerCfg:
    return LayerCfg(LSA_BF16 if dtype == torch.bfloat16 else LSA_F32, int(cfg.get("HI", 0)), int(cfg.get("dI", 0)),
                    int(cfg["H"]), int(cfg["Dqk"]), int(cfg["Dv"]), float(cfg["scale"]),
                    Budget(int(cfg["k_sink"]), int(cfg["k_swa"]), int(cfg["k_sparse"])), int(cfg.get("P", 128)),
                    int(cfg.get("B", 128)), int(cfg.get("M", 1024)), int(cfg.get("hi_min_len", 1 << 62)),
                    int(cfg.get("is_owner", 1)))


class Layer:
    """A configured layer with a reusable workspace (so repeated calls allocate nothing)."""

    def __init__(self, cfg: dict, rows: RowsDesc, dtype, device, use_hi=False):
        self.cfg = layer_cfg(cfg, dtype)
        self.rows = rows
        self._rc = rows.c()
        sz = ctypes.c_size_t()
        _check(lib().lsa_layer_workspace_size(ctypes.byref(self.cfg), ctypes.byref(self._rc), int(bool(use_hi)),
                                              ctypes.byref(sz)))
        self.ws = _workspace(sz.value, device)
        self.wp, self.wn = _aligned(self.ws)

    def __call__(self, q, kv, idx, out, lse, q_idx=None, w=None, k_idx=None, idx_row=None, sb_off=None, k_mean=None):
        _check(lib().lsa_layer_fwd(ctypes.byref(self.cfg), ctypes.byref(self._rc), _p(idx_row), _p(q_idx), _p(w),
                                   _p(k_idx), _p(sb_off), _p(k_mean), _p(q), _p(kv), _p(idx), _p(out), _p(lse),
                                   self.wp, self.wn, _stream()))
        return idx, out, lse


def lsa_layer_fwd(cfg: dict, rows: RowsDesc, q, kv, q_idx=None, w=None, k_idx=None, idx=None, idx_row=None,
                  sb_off=None, k_mean=None):
    """One layer: (idx [n_rows, k_sparse], out [n_rows, H, Dv], lse [n_rows, H])."""
    n_rows, H, _ = q.shape
    layer = Layer(cfg, rows, q.dtype, q.device, use_hi=k_mean is not None)
    if idx is None:
        idx = torch.full((n_rows, int(cfg["k_sparse"])), -1, dtype=torch.int32, device=q.device)
    out = torch.empty((n_rows, H, int(cfg["Dv"])), dtype=q.dtype, device=q.device)
    lse = torch.empty((n_rows, H), dtype=torch.float32, device=q.device)
    return layer(q, kv, idx, out, lse, q_idx=q_idx, w=w, k_idx=k_idx, idx_row=idx_row, sb_off=sb_off, k_mean=k_mean)


def sb_offsets(lengths, B):
    """Host helper: sb_off (int64 [n_seq+1]) for sub-blocks of B tokens."""
    out = [0]
    for L in lengths:
        out.append(out[-1] + (int(L) + B - 1) // B)
    return torch.tensor(out, dtype=torch.int64)
