"""fp64 numpy oracle for packed variable-length attention, forward and backward.

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

attn_varlen_bwd is the backward of the same forward (attn_bwd_oracle.c's
chain rule) with the same whole-matrix steps; its docstring lists them.
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


def attn_varlen_bwd(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool = False,
                    row_chunk: int = 256, threads: int | None = None):
    """Exact fp64 gradients (dq [Nq,H,D], dk [Nk,H,D], dv [Nk,H,D]) of the
    forward above for the upstream gradient dout [Nq,H,D] (all bf16), with
    whole-matrix numpy steps so that segments of tens of thousands of rows
    finish in seconds. The same chain rule as attn_bwd_oracle.c, per segment b
    and head h, with the segment's query rows Q, keys K, values V and upstream
    gradient G (matrix products are library steps):
        S  = scale * Q K^T;  P = row softmax of S (max, then exp and sum)
        O  = P V;            D = row sums of G * O
        dP = G V^T;          dS = P * (dP - D)
        dQ = scale * dS K;   dK = scale * dS^T Q;   dV = P^T G
    Query rows are taken in chunks of `row_chunk`; dK and dV sum the chunks in
    order. causal: row r sees keys j <= r + Lk - Lq, so a chunk's products
    stop at its last row's last visible key (the keys past it carry zero
    weight); rows that see no key get dQ = 0 and contribute nothing. Rows past cu_seqlens_q[-1] and keys past
    cu_seqlens_k[-1] get 0. D uses this oracle's exact O; the _bwd_preprocess
    page names the reduction over dout and out without its formula, and this
    is its plain reading."""
    (qb, wq), (kb, wk), (vb, wv), (gb, wg) = _source(q), _source(k), _source(v), _source(dout)
    if qb.ndim != 3 or gb.shape != qb.shape or kb.shape != vb.shape or kb.shape[1:] != qb.shape[1:]:
        raise ValueError("q and dout must be [Nq,H,D], k and v [Nk,H,D]")
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    if len(cq) != len(ck) or len(cq) < 2 or cq[0] != 0 or ck[0] != 0:
        raise ValueError("bad cu_seqlens")
    if np.any(np.diff(cq) < 0) or np.any(np.diff(ck) < 0) or cq[-1] > qb.shape[0] or ck[-1] > kb.shape[0]:
        raise ValueError("cu_seqlens decrease or index past the q / k rows")
    _, H, D = qb.shape
    dq = np.zeros(qb.shape, dtype=np.float64)
    dk = np.zeros(kb.shape, dtype=np.float64)
    dv = np.zeros(kb.shape, dtype=np.float64)

    def one(b, h):
        qs, qe, ks, ke = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        if qe == qs or ke == ks:
            return
        K = wk(kb[ks:ke, h, :])
        V = wv(vb[ks:ke, h, :])
        dK = np.zeros_like(K)
        dV = np.zeros_like(V)
        for c0 in range(qs, qe, row_chunk):
            c1 = min(qe, c0 + row_chunk)
            Q = wq(qb[c0:c1, h, :])
            G = wg(gb[c0:c1, h, :])
            n = ke - ks  # keys that any row of the chunk may see (all of them unless causal)
            if causal:
                last = np.arange(c0, c1) - qs + (ke - ks) - (qe - qs)  # last visible key of each row
                n = min(n, int(last[-1]) + 1)
                if n <= 0:
                    continue  # no row of the chunk sees a key: dq stays 0
            S = scale * (Q @ K[:n].T)
            if causal:
                S = np.where(np.arange(n)[None, :] > last[:, None], -np.inf, S)
            m = S.max(axis=1, keepdims=True)
            seen = np.isfinite(m[:, 0])
            E = np.exp(S - np.where(seen[:, None], m, 0.0))
            l = E.sum(axis=1, keepdims=True)
            P = np.where(seen[:, None], E / np.where(seen[:, None], l, 1.0), 0.0)
            O = P @ V[:n]
            Dr = (G * O).sum(axis=1, keepdims=True)
            dS = P * (G @ V[:n].T - Dr)
            dq[c0:c1, h, :] = scale * (dS @ K[:n])
            dK[:n] += scale * (dS.T @ Q)
            dV[:n] += P.T @ G
        dk[ks:ke, h, :] = dK
        dv[ks:ke, h, :] = dV

    work = [(b, h) for b in range(len(cq) - 1) for h in range(H)]
    nthreads = max(1, min(int(threads or default_threads()), len(work)))
    if nthreads == 1:
        for b, h in work:
            one(b, h)
        return dq, dk, dv
    from threadpoolctl import threadpool_limits
    blas = max(1, int(threads or default_threads()) // nthreads)
    with threadpool_limits(limits=blas, user_api="blas"), ThreadPoolExecutor(nthreads) as ex:
        for f in [ex.submit(one, b, h) for b, h in work]:
            f.result()
    return dq, dk, dv
