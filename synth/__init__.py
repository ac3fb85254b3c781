"""Seeded synthetic inputs for the LSA layer forward (shared by the tests, the smoke check and the
benchmark).

This module only draws and shapes inputs.  It holds none of the method's arithmetic: no indexer
score, no selection, no attention.  Draws use torch's counter-based Philox generator on the target
device (``torch.Generator(device).manual_seed(seed)``), so a workload is a pure function of
(config, seed, device).  Tensors that the CPU oracle needs are copied to the host from these
inputs; nothing here is ever produced by the HIP library.

Value recipe (the pages give no data; the stated stand-in):
  * indexer queries and keys  q_idx, k_idx ~ N(0, 1/d_idx)
  * indexer head weights      w = softplus(N(0, 1))  (fp32)
  * attention queries, latent q, kv ~ N(0, 1);  softmax scale 1/sqrt(576)
  * needles: a key position s in the middle region of a later query row r is overwritten with
    k_idx[s] = 3 * u / |u|,  u = sum_j w[r, j] * q_idx[r, j]   (a key aligned with what r asks for)
bf16 tensors are drawn in fp32 and rounded to nearest-even by torch.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

# ----------------------------------------------------------------------------- host bf16 helpers


def bf16_to_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> host np.uint16 raw bits (a copy)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def to_host(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy in the oracle's convention: bf16 as uint16 bits, everything else as is."""
    if t.dtype == torch.bfloat16:
        return bf16_to_bits(t)
    return t.detach().to("cpu").contiguous().numpy().copy()


def bits_to_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(torch.bfloat16)


# ----------------------------------------------------------------------------- draws

_CHUNK = 1 << 26  # elements per draw (fp32 scratch of 256 MB)


def normal(shape, std, gen, device, dtype):
    """N(0, std^2) drawn in fp32 chunks and stored as ``dtype`` (rounded to nearest-even)."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        x = torch.randn(hi - lo, generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[lo:hi].copy_(x)
        del x
    return out


def softplus_normal(shape, gen, device):
    return F.softplus(torch.randn(shape, generator=gen, device=device, dtype=torch.float32))


def generator(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def needle_span(t, k_sink, k_swa):
    """[lo, hi): where a needle for a query at position t is placed -- past the first k_sink tokens
    and before the last k_swa, as the workloads prescribe (the span the indexer has to search)."""
    return k_sink, max(k_sink, t - k_swa + 1)


def plant_needle(k_idx, tok, q_row, w_row):
    """k_idx[tok] = 3 u / |u| with u = sum_j w_j q_j (fp32), stored in k_idx's dtype."""
    u = (w_row.float()[:, None] * q_row.float()).sum(0)
    k_idx[tok] = (3.0 * u / u.norm()).to(k_idx.dtype)


# ----------------------------------------------------------------------------- workloads


def _budget(k_sink, k_swa, k_sparse):
    return dict(k_sink=k_sink, k_swa=k_swa, k_sparse=k_sparse)


def decode_batch(lengths, *, HI=64, dI=128, H=128, Dqk=576, Dv=512, k_sink=16, k_swa=1024, k_sparse=1024,
                 drafts=1, needles=64, needle_pages=0, P=128, B=128, M=1024, hi_min_len=None, dtype=torch.bfloat16,
                 device="cuda", seed=0, with_attn=True):
    """A decode batch: one sequence per entry of ``lengths``; each sequence has ``drafts`` query rows,
    all at t = L - 1 (MTP drafts share the sequence's KV; the first draft owns the index set)."""
    g = generator(seed, device)
    lengths = [int(x) for x in lengths]
    n_seq = len(lengths)
    kv_off = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64)
    tot = int(kv_off[-1])
    n_rows = n_seq * drafts
    row_seq = torch.arange(n_seq, dtype=torch.int32).repeat_interleave(drafts)
    row_pos = torch.tensor([lengths[b] - 1 for b in range(n_seq) for _ in range(drafts)], dtype=torch.int32)
    idx_row = torch.arange(n_rows, dtype=torch.int32) // drafts * drafts
    s_idx = 1.0 / math.sqrt(dI)
    q_idx = normal((n_rows, HI, dI), s_idx, g, device, dtype)
    w = softplus_normal((n_rows, HI), g, device)
    k_idx = normal((tot, dI), s_idx, g, device, dtype)
    q = normal((n_rows, H, Dqk), 1.0, g, device, dtype) if with_attn else None
    kv = normal((tot, Dqk), 1.0, g, device, dtype) if with_attn else None
    # Needles: positions drawn on the host from a seeded numpy generator.
    hrng = np.random.default_rng(seed + 7919)
    needle_pos = []
    for b in range(n_seq):
        L = lengths[b]
        r = b * drafts
        t = L - 1
        mlo, mhi = needle_span(t, k_sink, k_swa)
        picks = []
        if needle_pages and mhi - mlo > 2 * P:
            first_page = (mlo + P - 1) // P
            last_page = mhi // P  # pages [first_page, last_page) lie wholly inside mid
            n_avail = last_page - first_page
            if n_avail > 0:
                pg = hrng.choice(n_avail, size=min(needle_pages, n_avail), replace=False) + first_page
                picks = [int(p * P + hrng.integers(0, P)) for p in pg]
        elif needles and mhi > mlo:
            picks = [int(x) for x in hrng.choice(mhi - mlo, size=min(needles, mhi - mlo), replace=False) + mlo]
        for s in picks:
            plant_needle(k_idx, int(kv_off[b]) + s, q_idx[r], w[r])
        needle_pos.append(sorted(picks))
    cfg = dict(HI=HI, dI=dI, H=H, Dqk=Dqk, Dv=Dv, scale=1.0 / math.sqrt(Dqk), P=P, B=B, M=M,
               hi_min_len=(1 << 62) if hi_min_len is None else int(hi_min_len), is_owner=1,
               **_budget(k_sink, k_swa, k_sparse))
    return dict(cfg=cfg, kv_off=kv_off.to(device), kv_off_host=kv_off, row_seq=row_seq.to(device),
                row_pos=row_pos.to(device), row_pos_host=row_pos, row_seq_host=row_seq,
                idx_row=idx_row.to(device) if drafts > 1 else None, idx_row_host=idx_row if drafts > 1 else None,
                q_idx=q_idx, w=w, k_idx=k_idx, q=q, kv=kv, lengths=lengths, max_len=max(lengths),
                needles=needle_pos)


def prefill_chunk(prefix, chunk, *, HI=64, dI=128, H=128, Dqk=576, Dv=512, k_sink=16, k_swa=1024,
                  k_sparse=1024, needles=0, dtype=torch.bfloat16, device="cuda", seed=0, with_attn=True,
                  n_layers=1, P=128, B=128, M=1024, hi_min_len=None):
    """One sequence of prefix+chunk tokens; the chunk's rows t = prefix .. prefix+chunk-1 attend causally.
    n_layers > 1 adds independent q / kv per extra (CLI reuse) layer."""
    g = generator(seed, device)
    L = prefix + chunk
    kv_off = torch.tensor([0, L], dtype=torch.int64)
    n_rows = chunk
    row_seq = torch.zeros(n_rows, dtype=torch.int32)
    row_pos = torch.arange(prefix, L, dtype=torch.int32)
    s_idx = 1.0 / math.sqrt(dI)
    q_idx = normal((n_rows, HI, dI), s_idx, g, device, dtype)
    w = softplus_normal((n_rows, HI), g, device)
    k_idx = normal((L, dI), s_idx, g, device, dtype)
    layers = []
    if with_attn:
        for _ in range(n_layers):
            layers.append((normal((n_rows, H, Dqk), 1.0, g, device, dtype), normal((L, Dqk), 1.0, g, device, dtype)))
    hrng = np.random.default_rng(seed + 7919)
    needle_pos = []
    for _ in range(needles):
        r = int(hrng.integers(0, n_rows))
        t = prefix + r
        mlo, mhi = needle_span(t, k_sink, k_swa)
        if mhi > mlo:
            s = int(hrng.integers(mlo, mhi))
            plant_needle(k_idx, s, q_idx[r], w[r])
            needle_pos.append((r, s))
    cfg = dict(HI=HI, dI=dI, H=H, Dqk=Dqk, Dv=Dv, scale=1.0 / math.sqrt(Dqk), P=P, B=B, M=M,
               hi_min_len=(1 << 62) if hi_min_len is None else int(hi_min_len), is_owner=1,
               **_budget(k_sink, k_swa, k_sparse))
    return dict(cfg=cfg, kv_off=kv_off.to(device), kv_off_host=kv_off, row_seq=row_seq.to(device),
                row_pos=row_pos.to(device), row_pos_host=row_pos, row_seq_host=row_seq, idx_row=None,
                idx_row_host=None, q_idx=q_idx, w=w, k_idx=k_idx, q=layers[0][0] if layers else None,
                kv=layers[0][1] if layers else None, layers=layers, lengths=[L], max_len=L, needles=needle_pos)


# ----------------------------------------------------------------------------- the named workloads


def tiny_prefill(device="cuda", seed=0):
    """L = 2048 tokens, one sequence, every row t = 0..2047 causal, fp32; HI=4, dI=64; H=4 over a
    576-dim latent; K = 256 = 16 sink + 128 window + 112 sparse; 8 needles; flat indexer."""
    g = generator(seed, device)
    L, HI, dI, H, Dqk, Dv = 2048, 4, 64, 4, 576, 512
    k_sink, k_swa, k_sparse = 16, 128, 112
    dtype = torch.float32
    kv_off = torch.tensor([0, L], dtype=torch.int64)
    row_seq = torch.zeros(L, dtype=torch.int32)
    row_pos = torch.arange(L, dtype=torch.int32)
    q_idx = normal((L, HI, dI), 1.0 / math.sqrt(dI), g, device, dtype)
    w = softplus_normal((L, HI), g, device)
    k_idx = normal((L, dI), 1.0 / math.sqrt(dI), g, device, dtype)
    q = normal((L, H, Dqk), 1.0, g, device, dtype)
    kv = normal((L, Dqk), 1.0, g, device, dtype)
    hrng = np.random.default_rng(seed + 7919)
    needles = []
    for s in hrng.choice(np.arange(16, 1920), size=8, replace=False):
        r = int(hrng.integers(int(s) + k_swa, L))
        plant_needle(k_idx, int(s), q_idx[r], w[r])
        needles.append((r, int(s)))
    cfg = dict(HI=HI, dI=dI, H=H, Dqk=Dqk, Dv=Dv, scale=1.0 / math.sqrt(Dqk), P=128, B=128, M=1024,
               hi_min_len=1 << 62, is_owner=1, **_budget(k_sink, k_swa, k_sparse))
    return dict(cfg=cfg, kv_off=kv_off.to(device), kv_off_host=kv_off, row_seq=row_seq.to(device),
                row_pos=row_pos.to(device), row_pos_host=row_pos, row_seq_host=row_seq, idx_row=None,
                idx_row_host=None, q_idx=q_idx, w=w, k_idx=k_idx, q=q, kv=kv, lengths=[L], max_len=L,
                needles=needles)


def decode_sweep(L, device="cuda", seed=0, batch=32, **kw):
    """Batch of single-token decode queries at KV length L (bf16, HI=64, dI=128, H=128, K=16+1024+1024,
    64 planted needles per sequence, flat indexer)."""
    return decode_batch([L] * batch, device=device, seed=seed, **kw)


def hi_decode(device="cuda", seed=0, batch=8, L=1 << 20, **kw):
    """1M-context decode with Hierarchical Indexing: P = B = 128, M = 1024; 32 needle pages per sequence."""
    return decode_batch([L] * batch, device=device, seed=seed, needles=0, needle_pages=32, hi_min_len=0, **kw)


def ragged_mtp_lengths(seed=0, n=64, lo=4096, hi=524288):
    r = np.random.default_rng(seed + 104729)
    return [int(math.floor(math.exp(x))) for x in r.uniform(math.log(lo), math.log(hi), size=n)]


def ragged_mtp(device="cuda", seed=0, n=64, **kw):
    """64 sequences with log-uniform lengths in [4K, 512K]; 3 MTP draft rows per sequence sharing the
    first draft's index set; HI for L >= 256K (P = B = 128, M = 1024); 64 needles per sequence."""
    return decode_batch(ragged_mtp_lengths(seed, n), device=device, seed=seed, drafts=3, hi_min_len=262144, **kw)


def chunked_prefill_cli(device="cuda", seed=0, prefix=131072, chunk=8192, **kw):
    """An 8192-token causal chunk over a 131072-token prefix; owner layer (indexer + topK + attention)
    and one CLI reuse layer with independent q / kv."""
    return prefill_chunk(prefix, chunk, device=device, seed=seed, n_layers=2, **kw)


def hi_prefill(L, device="cuda", seed=0, q_len=2048, **kw):
    """Chunked prefill under Hierarchical Indexing: the last q_len rows of an L-token sequence, sub-block
    B = 8, page P = 128, M = 1024 recalled pages (the HI-vs-flat prefill measurement of the pages:
    q_len 2048, KV 32K .. 1M); independent Gaussian indexer inputs, no needles."""
    kw.setdefault("with_attn", False)
    return prefill_chunk(L - q_len, q_len, device=device, seed=seed, P=128, B=8, M=1024, hi_min_len=0, **kw)
