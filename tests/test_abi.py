"""The C-ABI library loads, exports every symbol include/lsa.h declares, and rejects bad arguments
before touching the HIP runtime (no GPU needed: validation never reaches a device call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "lsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lsa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    import long_context_sparse_weighted_amd as lsa
    if not os.path.exists(lsa.LIB_PATH):
        pytest.skip("liblsa.so not built")
    return lsa


def test_header_symbols_exported(L):
    names = header_functions()
    assert len(names) >= 12
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SYMBOLS)


def test_status_strings(L):
    lib = L.lib()
    assert lib.lsa_status_string(0) == b"ok"
    assert lib.lsa_status_string(3) == b"workspace too small"
    assert lib.lsa_status_string(99) == b"unknown status"


def _rows(L, n_seq=1, n_rows=2, max_len=100, null=False):
    p = None if null else ctypes.c_void_p(0x1000)
    return L.Rows(n_seq, n_rows, p, p, p, max_len)


def test_index_score_validation(L):
    lib = L.lib()
    b = L.Budget(16, 1024, 1024)
    fake = ctypes.c_void_p(0x1000)
    call = lambda dt, rows, H, D, pages, M, P, ld, bud=b: lib.lsa_index_score(
        dt, rows, fake, fake, fake, H, D, bud, pages, M, P, fake, ld, None)
    r = _rows(L)
    assert call(1, None, 64, 128, None, 0, 0, 100) == L.LSA_ERR_INVALID
    assert call(7, ctypes.byref(r), 64, 128, None, 0, 0, 100) == L.LSA_ERR_INVALID
    assert call(1, ctypes.byref(r), 32, 128, None, 0, 0, 100) == L.LSA_ERR_UNSUPPORTED
    assert call(0, ctypes.byref(r), 4, 96, None, 0, 0, 100) == L.LSA_ERR_UNSUPPORTED
    assert call(1, ctypes.byref(r), 64, 128, None, 0, 0, 99) == L.LSA_ERR_INVALID        # ld < max_kv_len
    assert call(1, ctypes.byref(r), 64, 128, fake, 4, 100, 400) == L.LSA_ERR_UNSUPPORTED  # P % 16
    assert call(1, ctypes.byref(r), 64, 128, fake, 4, 128, 500) == L.LSA_ERR_INVALID      # ld < M*P
    assert call(1, ctypes.byref(r), 64, 128, None, 0, 0, 100, L.Budget(-1, 4, 4)) == L.LSA_ERR_INVALID
    nr = _rows(L, null=True)
    assert call(1, ctypes.byref(nr), 64, 128, None, 0, 0, 100) == L.LSA_ERR_INVALID
    big = _rows(L, n_rows=70000)
    assert call(1, ctypes.byref(big), 64, 128, None, 0, 0, 100) == L.LSA_ERR_UNSUPPORTED
    bad_min = _rows(L)
    bad_min.min_kv_len = 101  # above max_kv_len
    assert call(1, ctypes.byref(bad_min), 64, 128, None, 0, 0, 100) == L.LSA_ERR_INVALID
    bad_min.min_kv_len = -1
    assert call(1, ctypes.byref(bad_min), 64, 128, None, 0, 0, 100) == L.LSA_ERR_INVALID
    assert b"ld_scores" in lib.lsa_last_error() or lib.lsa_last_error()


def test_topk_validation(L):
    lib = L.lib()
    fake = ctypes.c_void_p(0x1000)
    sz = ctypes.c_size_t()
    n = 100000  # several 16384-column segments: the selection needs candidate buffers
    assert lib.lsa_topk_workspace_size(4, n, 0, ctypes.byref(sz)) == L.LSA_ERR_INVALID
    assert lib.lsa_topk_workspace_size(4, 100, 16, ctypes.byref(sz)) == L.LSA_OK and sz.value == 0  # one segment
    assert lib.lsa_topk_workspace_size(4, n, 16, ctypes.byref(sz)) == L.LSA_OK and sz.value > 0
    need = sz.value
    assert lib.lsa_topk(4, fake, n, n, None, 0, 0, 0, fake, fake, need, None) == L.LSA_ERR_UNSUPPORTED
    assert lib.lsa_topk(4, fake, n, n, None, 0, 0, 5000, fake, fake, need, None) == L.LSA_ERR_UNSUPPORTED
    assert lib.lsa_topk(4, fake, n - 1, n, None, 0, 0, 16, fake, fake, need, None) == L.LSA_ERR_INVALID
    assert lib.lsa_topk(4, fake, n, n, None, 0, 0, 16, fake, fake, need - 1, None) == L.LSA_ERR_WORKSPACE
    assert lib.lsa_topk(4, fake, n, n, None, 0, 0, 16, fake, ctypes.c_void_p(0x1010), need, None) == \
        L.LSA_ERR_INVALID                                                                   # misaligned workspace
    assert lib.lsa_topk(4, fake, 100, 100, fake, 2, 16, 16, fake, fake, need, None) == L.LSA_ERR_INVALID  # M*P < n
    assert lib.lsa_topk(4, fake, 100, 100, fake, 10, 24, 16, fake, fake, need, None) == L.LSA_ERR_UNSUPPORTED  # P%16


def test_page_validation(L):
    lib = L.lib()
    fake = ctypes.c_void_p(0x1000)
    r = _rows(L, max_len=4096)
    sz = ctypes.c_size_t()
    assert lib.lsa_page_recall_workspace_size(ctypes.byref(r), 128, 1024, ctypes.byref(sz)) == L.LSA_OK
    call = lambda P, B, M, ws=sz.value: lib.lsa_page_recall(1, ctypes.byref(r), fake, fake, fake, fake, 64, 128, P,
                                                            B, M, None, 0, fake, fake, ws, None)
    assert call(128, 24, 1024) == L.LSA_ERR_INVALID        # B does not divide P
    assert call(128, 4, 1024) == L.LSA_ERR_UNSUPPORTED     # P/B = 32 > 16 on the bf16 path
    assert call(100, 100, 64) == L.LSA_ERR_UNSUPPORTED     # P % 16
    assert call(128, 128, 0) == L.LSA_ERR_INVALID
    assert call(128, 128, 1024, ws=0) == L.LSA_ERR_WORKSPACE
    assert lib.lsa_page_means(1, 1, fake, fake, fake, 128, 0, 100, 0, fake, None) == L.LSA_ERR_INVALID
    assert lib.lsa_page_means(1, 1, fake, fake, fake, 128, 8, 100, -1, fake, None) == L.LSA_ERR_INVALID
    assert lib.lsa_page_means_append(1, 1, fake, fake, fake, 128, 8, 0, fake, None) == L.LSA_ERR_INVALID
    assert lib.lsa_page_means_append(1, 1, fake, fake, fake, 128, 0, 1, fake, None) == L.LSA_ERR_INVALID
    assert lib.lsa_page_means_append(2, 1, fake, fake, fake, 128, 8, 1, fake, None) == L.LSA_ERR_INVALID
    assert lib.lsa_page_means_append(1, 1, None, fake, fake, 128, 8, 1, fake, None) == L.LSA_ERR_INVALID
    assert lib.lsa_page_means_append(1, 0, None, None, None, 128, 8, 1, None, None) == L.LSA_OK  # nothing to do


def test_fp8_validation(L):
    lib = L.lib()
    fake = ctypes.c_void_p(0x1000)
    q = lambda dt, n, d, x=fake: lib.lsa_quantize_fp8(dt, n, d, x, fake, fake, None)
    assert q(2, 10, 128) == L.LSA_ERR_INVALID          # dtype
    assert q(1, 10, 0) == L.LSA_ERR_INVALID            # dim
    assert q(1, -1, 128) == L.LSA_ERR_INVALID
    assert q(1, 10, 300) == L.LSA_ERR_UNSUPPORTED      # dim above 256
    assert q(1, 10, 128, None) == L.LSA_ERR_INVALID    # missing buffer
    assert q(1, 0, 128, None) == L.LSA_OK              # nothing to do
    b = L.Budget(16, 1024, 1024)
    r = _rows(L)
    s = lambda H, D, ld, pages=None, M=0, P=0, k8=fake: lib.lsa_index_score_fp8(
        ctypes.byref(r), fake, fake, fake, k8, fake, H, D, b, pages, M, P, fake, ld, None)
    assert s(32, 128, 100) == L.LSA_ERR_UNSUPPORTED    # 64 heads of dim 128 only
    assert s(64, 64, 100) == L.LSA_ERR_UNSUPPORTED
    assert s(64, 128, 99) == L.LSA_ERR_INVALID         # ld below max_kv_len
    assert s(64, 128, 100, k8=None) == L.LSA_ERR_INVALID
    assert s(64, 128, 2048, fake, 16, 100) == L.LSA_ERR_UNSUPPORTED   # P % 16
    assert s(64, 128, 1000, fake, 16, 128) == L.LSA_ERR_INVALID       # ld < M*P
    assert lib.lsa_index_score_fp8(None, fake, fake, fake, fake, fake, 64, 128, b, None, 0, 0, fake, 100,
                                   None) == L.LSA_ERR_INVALID


def test_index_topk_validation_and_workspace(L):
    lib = L.lib()
    fake = ctypes.c_void_p(0x1000)
    b = L.Budget(16, 1024, 1024)
    sz = ctypes.c_size_t()
    ws_size = lambda dt, r, H=64, D=128, k=1024: lib.lsa_index_topk_workspace_size(dt, ctypes.byref(r), H, D, k,
                                                                                   ctypes.byref(sz))
    # a 32-row bf16 decode batch at 1M tokens takes the fused pass: candidate lists, no score matrix
    big = _rows(L, 32, 32, 1 << 20)
    assert ws_size(1, big) == L.LSA_OK
    assert 0 < sz.value < 32 * (1 << 20) * 4 // 3      # (score, position) lists of 1024 per 8192 columns
    # fp32, or rows too few to fill the chip: the scores go through the workspace
    assert ws_size(0, _rows(L, 32, 32, 1 << 20), 4, 64) == L.LSA_OK and sz.value >= 32 * (1 << 20) * 4
    assert ws_size(1, _rows(L, 1, 1, 20000)) == L.LSA_OK and sz.value >= 20000 * 4
    assert ws_size(1, big, 32) == L.LSA_ERR_UNSUPPORTED
    assert ws_size(1, big, k=0) == L.LSA_ERR_UNSUPPORTED
    assert ws_size(1, big, k=4097) == L.LSA_ERR_UNSUPPORTED
    assert ws_size(5, big) == L.LSA_ERR_INVALID
    assert lib.lsa_index_topk_workspace_size(1, ctypes.byref(big), 64, 128, 1024, None) == L.LSA_ERR_INVALID
    call = lambda r, ws, n, bud=b, idx=fake: lib.lsa_index_topk(1, ctypes.byref(r), fake, fake, fake, 64, 128, bud,
                                                                idx, ws, n, None)
    assert ws_size(1, big) == L.LSA_OK
    assert call(big, fake, sz.value - 1) == L.LSA_ERR_WORKSPACE
    assert call(big, None, sz.value) == L.LSA_ERR_WORKSPACE
    assert call(big, ctypes.c_void_p(0x1010), sz.value) == L.LSA_ERR_INVALID      # not 256-byte aligned
    assert call(big, fake, sz.value, idx=None) == L.LSA_ERR_INVALID
    assert call(big, fake, sz.value, bud=L.Budget(-1, 1024, 1024)) == L.LSA_ERR_INVALID
    assert call(_rows(L, 1, 0, 0), None, 0) == L.LSA_OK                            # no rows: nothing to do
    # the variant with the library's own scratch array: the same checks, then its size, before any HIP call
    na = lambda r, dt=1, H=64, D=128, bud=b, idx=fake: lib.lsa_index_topk_noalloc(dt, ctypes.byref(r), fake, fake,
                                                                                  fake, H, D, bud, idx, None)
    assert sz.value <= 64 << 20                      # 32 decode rows at 1M fit the 64 MiB array
    assert na(big, H=32) == L.LSA_ERR_UNSUPPORTED
    assert na(big, bud=L.Budget(16, 1024, 4097)) == L.LSA_ERR_UNSUPPORTED
    assert na(big, dt=5) == L.LSA_ERR_INVALID
    assert na(big, idx=None) == L.LSA_ERR_INVALID
    huge = _rows(L, 32, 32, 1 << 20)                 # fp32 rows score through the workspace: 128 MiB
    assert na(huge, dt=0, H=4, D=64) == L.LSA_ERR_UNSUPPORTED
    assert b"scratch" in lib.lsa_last_error()
    assert na(_rows(L, 1, 0, 0)) == L.LSA_OK


def test_index_topk_fp8_validation_and_workspace(L):
    lib = L.lib()
    fake = ctypes.c_void_p(0x1000)
    b = L.Budget(16, 1024, 1024)
    sz = ctypes.c_size_t()
    big = _rows(L, 32, 32, 1 << 20)
    assert lib.lsa_index_topk_fp8_workspace_size(ctypes.byref(big), 64, 128, 1024, ctypes.byref(sz)) == L.LSA_OK
    assert 0 < sz.value < 32 * (1 << 20) * 4 // 3      # candidate lists, no score matrix
    small = _rows(L, 1, 1, 20000)
    assert lib.lsa_index_topk_fp8_workspace_size(ctypes.byref(small), 64, 128, 1024, ctypes.byref(sz)) == L.LSA_OK
    assert sz.value >= 20000 * 4
    assert lib.lsa_index_topk_fp8_workspace_size(ctypes.byref(big), 32, 128, 1024, ctypes.byref(sz)) == \
        L.LSA_ERR_UNSUPPORTED
    assert lib.lsa_index_topk_fp8_workspace_size(ctypes.byref(big), 64, 128, 0, ctypes.byref(sz)) == \
        L.LSA_ERR_UNSUPPORTED
    assert lib.lsa_index_topk_fp8_workspace_size(ctypes.byref(big), 64, 128, 1024, None) == L.LSA_ERR_INVALID
    assert lib.lsa_index_topk_fp8_workspace_size(ctypes.byref(big), 64, 128, 1024, ctypes.byref(sz)) == L.LSA_OK
    call = lambda ws, n, k8=fake, bud=b: lib.lsa_index_topk_fp8(ctypes.byref(big), fake, fake, fake, k8, fake, 64, 128,
                                                               bud, fake, ws, n, None)
    assert call(fake, sz.value - 1) == L.LSA_ERR_WORKSPACE
    assert call(fake, sz.value, k8=None) == L.LSA_ERR_INVALID
    assert call(ctypes.c_void_p(0x1010), sz.value) == L.LSA_ERR_INVALID          # not 256-byte aligned
    assert call(fake, sz.value, bud=L.Budget(16, -1, 1024)) == L.LSA_ERR_INVALID
    assert lib.lsa_index_topk_fp8(ctypes.byref(_rows(L, 1, 0, 0)), None, None, None, None, None, 64, 128, b, None,
                                  None, 0, None) == L.LSA_OK


def test_attn_and_layer_validation(L):
    lib = L.lib()
    fake = ctypes.c_void_p(0x1000)
    r = _rows(L)
    b = L.Budget(16, 1024, 1024)
    call = lambda dt, H, dqk, dv: lib.lsa_hybrid_attn(dt, ctypes.byref(r), fake, fake, H, dqk, dv, 0.04, b, fake,
                                                      None, fake, fake, fake, 1 << 30, None)
    assert call(1, 100, 576, 512) == L.LSA_ERR_UNSUPPORTED   # heads not a multiple of 32
    assert call(1, 128, 512, 512) == L.LSA_ERR_UNSUPPORTED
    assert call(0, 4, 2048, 512) == L.LSA_ERR_UNSUPPORTED
    assert call(1, 0, 576, 512) == L.LSA_ERR_INVALID
    assert lib.lsa_hybrid_attn(1, ctypes.byref(r), fake, fake, 128, 576, 512, 0.04, L.Budget(16, 1024, 5000), fake,
                               None, fake, fake, fake, 1 << 30, None) == L.LSA_ERR_UNSUPPORTED
    cfg = L.layer_cfg(dict(HI=64, dI=128, H=128, Dqk=576, Dv=512, scale=0.04, k_sink=16, k_swa=1024, k_sparse=1024),
                      None)
    cfg.dtype = 1
    sz = ctypes.c_size_t()
    assert lib.lsa_layer_workspace_size(ctypes.byref(cfg), ctypes.byref(r), 0, ctypes.byref(sz)) == L.LSA_OK
    assert lib.lsa_layer_fwd(ctypes.byref(cfg), ctypes.byref(r), None, fake, fake, fake, None, None, fake, fake, fake,
                             fake, fake, fake, sz.value - 1, None) == L.LSA_ERR_WORKSPACE
    cfg.n_heads_idx = 16
    assert lib.lsa_layer_workspace_size(ctypes.byref(cfg), ctypes.byref(r), 0, ctypes.byref(sz)) == \
        L.LSA_ERR_UNSUPPORTED
    cfg.n_heads_idx = 64
    cfg.is_owner = 1
    assert lib.lsa_layer_fwd(ctypes.byref(cfg), ctypes.byref(r), None, None, None, None, None, None, fake, fake, fake,
                             fake, fake, fake, 1 << 40, None) == L.LSA_ERR_INVALID     # owner without q_idx
    cfg.B = 24
    cfg.hi_min_len = 0
    assert lib.lsa_layer_fwd(ctypes.byref(cfg), ctypes.byref(r), None, fake, fake, fake, fake, fake, fake, fake, fake,
                             fake, fake, fake, 1 << 40, None) == L.LSA_ERR_INVALID     # HI with B not dividing P
