"""lsa_index_topk_noalloc (the selection with the library's own device scratch array) against
lsa_index_topk with a caller workspace: identical index sets, bit for bit, on consecutive calls that
shrink, so that what an earlier call left in the shared array cannot leak into a later one."""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_weighted_amd as lsa
import synth
from parity_util import log

pytestmark = pytest.mark.gpu
DEV = "cuda"


def make_rows(lengths, rows, seed):
    g = synth.generator(seed, DEV)
    kv_off = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64)
    n = len(rows)
    desc = lsa.RowsDesc(kv_off.to(DEV), torch.tensor([r[0] for r in rows], dtype=torch.int32, device=DEV),
                        torch.tensor([r[1] for r in rows], dtype=torch.int32, device=DEV), max(lengths))
    q_idx = synth.normal((n, 64, 128), 1 / math.sqrt(128), g, DEV, torch.bfloat16)
    w = synth.softplus_normal((n, 64), g, DEV)
    k_idx = synth.normal((int(kv_off[-1]), 128), 1 / math.sqrt(128), g, DEV, torch.bfloat16)
    return desc, q_idx, w, k_idx


LENGTHS = [1, 17, 1041, 1042, 3001, 8192, 8193, 20000, 40000, 200001]
SMALL_ROWS = [(b, L - 1) for b, L in enumerate(LENGTHS)] + [(8, 9000), (9, 8192 + 1040), (6, 8193), (5, 8192)]
# 42 rows x 13 chunks of 16384 columns take the 16384-column fused pass; 14 rows x 25 chunks the
# 8192-column one; 2 rows the separate scoring and top-K passes (the scores then sit in the scratch)
CASES = [(LENGTHS, SMALL_ROWS + [(9, 200000 - 4001 * i) for i in range(1, 29)], 71),
         (LENGTHS, SMALL_ROWS, 72),
         ([20000, 9000], [(0, 19999), (1, 8999)], 73)]


def test_index_topk_noalloc_matches_workspace_entry_point():
    for k in (1024, 4096, 7):
        for lengths, rows, seed in CASES:
            desc, q_idx, w, k_idx = make_rows(lengths, rows, seed)
            bud = (16, 1024, k)
            log(f"noalloc index_topk: {len(rows)} rows, max_len {max(lengths)}, k={k}")
            want = lsa.lsa_index_topk(desc, q_idx, w, k_idx, bud)
            idx = torch.full((len(rows), k), -7, dtype=torch.int32, device=DEV)
            torch.cuda.synchronize()
            before = torch.cuda.memory_allocated()
            got = lsa.lsa_index_topk_noalloc(desc, q_idx, w, k_idx, bud, idx=idx)
            torch.cuda.synchronize()
            assert torch.cuda.memory_allocated() == before
            assert got is idx
            assert torch.equal(got, want), f"{len(rows)} rows, k={k}"
            del got, idx, want     # (so that the next case's memory check sees no frees either)


def test_index_topk_noalloc_rejects_beyond_scratch():
    # fp32 rows scored in the workspace: 8 rows x 4M columns need 128 MiB of scores
    L = 4 << 20
    desc = lsa.RowsDesc(torch.tensor([0, L], dtype=torch.int64, device=DEV),
                        torch.zeros(8, dtype=torch.int32, device=DEV),
                        torch.full((8,), L - 1, dtype=torch.int32, device=DEV), L)
    q_idx = torch.zeros((8, 4, 64), dtype=torch.float32, device=DEV)
    w = torch.zeros((8, 4), dtype=torch.float32, device=DEV)
    k_idx = torch.zeros((1, 64), dtype=torch.float32, device=DEV)   # never read: the call is refused first
    with pytest.raises(lsa.LsaError) as e:
        lsa.lsa_index_topk_noalloc(desc, q_idx, w, k_idx, (16, 1024, 1024),
                                   idx=torch.empty((8, 1024), dtype=torch.int32, device=DEV))
    assert e.value.code == lsa.LSA_ERR_UNSUPPORTED and "scratch" in str(e.value)
