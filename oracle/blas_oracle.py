"""fp64 numpy oracle for packed variable-length attention forward.

TEST INFRASTRUCTURE ONLY (same status as attn_oracle.c; nothing in the HIP
library or its binding imports it).

Same definition as attn_oracle.c, written with whole-matrix numpy steps so
that thousands of sampled query rows at full sequence length finish in
seconds: per segment b and head h, with the requested query rows Q_r of the
segment, its keys K and values V (bf16 widened exactly to fp64):
    S   = scale * Q_r K^T               (matrix product: a library step)
    m   = row max of S                  (pass 1)
    E   = exp(S - m);  l = row sum of E (pass 2)
    O   = (E V) / l;   LSE = m + ln l
Segments without keys give O = 0 and LSE = -inf. Sources: the varlen forward
with its (out, lse) return on the "[FA4] cute varlen backward: int32 overflow
in _bwd_preprocess ..." page ("Real-world trigger"), segment tables of the
"[FA4][SM120] flash_attn_varlen_func ... illegal memory access" page ("Bug 2
details"), SDPA as ground truth on the "ffpa-attn PR #387" page ("Verification").
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import _bits, default_threads


def _widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _source(x):
    """(array, widen): float64 arrays are used as they are; bf16 inputs (bits or
    CPU tensors) are widened exactly, slice by slice."""
    if isinstance(x, np.ndarray) and x.dtype == np.float64:
        return x, (lambda a: a)
    return _bits(x), _widen


def attn_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, rows=None,
                    row_chunk: int = 128, threads: int | None = None, causal: bool = False):
    """Returns (out [R, H, D] float64, lse [R, H] float64) for the requested
    global query rows (all rows if None), in the order given. (segment, head)
    pairs run on `threads` Python threads, each with single-threaded BLAS.
    causal: row r of a segment sees keys j <= r + Lk - Lq (bottom-right
    aligned, the same reading as the C oracle); a row that sees no key gives
    o = 0 and lse = -inf. q, k, v are bf16 (bits or CPU tensors) or float64
    arrays (the fp8 oracle passes dequantized values)."""
    (qb, wq), (kb, wk), (vb, wv) = _source(q), _source(k), _source(v)
    if qb.ndim != 3 or kb.ndim != 3 or kb.shape != vb.shape or kb.shape[1:] != qb.shape[1:]:
        raise ValueError("q must be [Nq,H,D] and k, v [Nk,H,D] with the same H, D")
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    if len(cq) != len(ck) or len(cq) < 2 or cq[0] != 0 or ck[0] != 0:
        raise ValueError("bad cu_seqlens")
    if np.any(np.diff(cq) < 0) or np.any(np.diff(ck) < 0) or cq[-1] > qb.shape[0] or ck[-1] > kb.shape[0]:
        raise ValueError("cu_seqlens decrease or index past the q / k rows")
    rows = np.arange(cq[-1], dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    seg = np.searchsorted(cq, rows, side="right") - 1
    if rows.size and (np.any(rows < 0) or np.any(rows >= cq[-1])):
        raise ValueError("row outside the segments")
    _, H, D = qb.shape
    out = np.zeros((rows.size, H, D), dtype=np.float64)
    lse = np.zeros((rows.size, H), dtype=np.float64)
    def one(b, h):
        sel = np.nonzero(seg == b)[0]
        ks, ke = int(ck[b]), int(ck[b + 1])
        if ke == ks:
            lse[sel, h] = -np.inf
            return
        K = wk(kb[ks:ke, h, :])
        V = wv(vb[ks:ke, h, :])
        for c0 in range(0, sel.size, row_chunk):
            idx = sel[c0:c0 + row_chunk]
            Q = wq(qb[rows[idx], h, :])
            S = scale * (Q @ K.T)
            if causal:
                last = rows[idx] - cq[b] + (ke - ks) - (cq[b + 1] - cq[b])  # last visible key
                S = np.where(np.arange(ke - ks)[None, :] > last[:, None], -np.inf, S)
            m = S.max(axis=1, keepdims=True)
            seen = np.isfinite(m[:, 0])
            E = np.exp(S - np.where(seen[:, None], m, 0.0))
            l = E.sum(axis=1)
            out[idx, h, :] = np.where(seen[:, None], (E @ V) / np.where(seen, l, 1.0)[:, None], 0.0)
            with np.errstate(divide="ignore"):
                lse[idx, h] = np.where(seen, m[:, 0] + np.log(l), -np.inf)

    work = [(int(b), h) for b in np.unique(seg) for h in range(H)]
    nthreads = max(1, min(int(threads or default_threads()), len(work)))
    if nthreads == 1:
        for b, h in work:
            one(b, h)
        return out, lse
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(nthreads) as ex:
        for f in [ex.submit(one, b, h) for b, h in work]:
            f.result()
    return out, lse
