"""CPU oracle for packed variable-length attention, forward and backward (fp64).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers. The HIP library never
imports, links or calls anything here, and nothing here imports the HIP
library or its binding.

The arithmetic lives in ``attn_oracle.c`` (forward) and ``attn_bwd_oracle.c``
(gradients), plain C in IEEE fp64 with a two-pass softmax; this module only
compiles them with gcc and marshals numpy arrays, except for the backward's
per-row preprocessing reduction, written out below in numpy. Parity pinned by
the ``-m "not gpu"`` tests in ``tests/test_oracle.py`` and
``tests/test_oracle_bwd.py`` (brute force on tiny inputs, finite differences,
a library special case, closed forms and invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRCS = (_HERE / "attn_oracle.c", _HERE / "attn_bwd_oracle.c")
_LIB = _HERE / "liboracle.so"
_lib = None


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc into oracle/liboracle.so."""
    stale = not _LIB.exists() or any(_LIB.stat().st_mtime < s.stat().st_mtime for s in _SRCS)
    if force or stale:
        tmp = _LIB.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
               "-o", str(tmp), *map(str, _SRCS), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path) -> ctypes.CDLL:
    """ctypes handle on a compiled oracle (the default build or a test variant)."""
    lib = ctypes.CDLL(str(path))
    for f in (lib.oracle_attn_varlen_fwd, lib.oracle_attn_varlen_fwd_causal):
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int32] * 3 + [ctypes.c_double,
                      ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                      ctypes.c_int32]
    if hasattr(lib, "oracle_attn_varlen_bwd"):
        f = lib.oracle_attn_varlen_bwd
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int32] * 3 + [ctypes.c_double, ctypes.c_int32] + \
            [ctypes.c_void_p] * 3 + [ctypes.c_int32]
        f = lib.oracle_attn_varlen_bwd_dq_rows
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int32] * 3 + [ctypes.c_double, ctypes.c_int32,
                      ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32]
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = load_library(_LIB)
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _bits(x) -> np.ndarray:
    """bf16 input as a contiguous uint16 bit-pattern array (numpy or torch CPU)."""
    if isinstance(x, np.ndarray):
        if x.dtype != np.uint16:
            raise TypeError("oracle expects bf16 bit patterns as uint16")
        return np.ascontiguousarray(x)
    import torch  # local: torch only used to accept CPU tensors

    if x.dtype != torch.bfloat16 or x.device.type != "cpu":
        raise TypeError("oracle expects a CPU bfloat16 tensor")
    return np.ascontiguousarray(x.contiguous().view(torch.int16).numpy().view(np.uint16))


def attn_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, rows=None,
                    threads: int | None = None, library=None, causal: bool = False):
    """fp64 attention for the given global query rows (all rows if None).

    q: [Nq, H, D], k/v: [Nk, H, D] bf16 (uint16 bits or CPU bf16 tensors).
    Returns (out [R, H, D] float64, lse [R, H] float64, natural log).
    `library` selects another compiled oracle (tests use it for planted mistakes).
    causal: row r of a segment sees keys j <= r + Lk - Lq (bottom-right
    aligned mask, the flash-attention convention; a reading, see the C file).
    """
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    if qb.ndim != 3 or kb.shape != vb.shape or kb.ndim != 3:
        raise ValueError("q must be [Nq,H,D] and k, v [Nk,H,D]")
    _, H, D = qb.shape
    if kb.shape[1:] != (H, D):
        raise ValueError("head count / head dim mismatch")
    cq = np.ascontiguousarray(np.asarray(cu_seqlens_q, dtype=np.int32))
    ck = np.ascontiguousarray(np.asarray(cu_seqlens_k, dtype=np.int32))
    B = len(cq) - 1
    if len(ck) != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
    if B < 1 or cq[-1] > qb.shape[0] or ck[-1] > kb.shape[0]:
        raise ValueError("cu_seqlens index past the q / k rows")
    if rows is None:
        r = None
        nrows = int(cq[-1])
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = len(r)
    out = np.zeros((nrows, H, D), dtype=np.float64)
    lse = np.zeros((nrows, H), dtype=np.float64)
    if nrows == 0:
        return out, lse
    lib = library if library is not None else _load()
    fn = lib.oracle_attn_varlen_fwd_causal if causal else lib.oracle_attn_varlen_fwd
    rc = fn(
        qb.ctypes.data, kb.ctypes.data, vb.ctypes.data, cq.ctypes.data, ck.ctypes.data,
        B, H, D, float(scale), None if r is None else r.ctypes.data, nrows,
        out.ctypes.data, lse.ctypes.data, int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out, lse


def _segments(cu_seqlens_q, cu_seqlens_k, nq: int, nk: int):
    cq = np.ascontiguousarray(np.asarray(cu_seqlens_q, dtype=np.int32))
    ck = np.ascontiguousarray(np.asarray(cu_seqlens_k, dtype=np.int32))
    B = len(cq) - 1
    if len(ck) != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
    if B < 1 or cq[-1] > nq or ck[-1] > nk:
        raise ValueError("cu_seqlens index past the q / k rows")
    return cq, ck, B


def attn_varlen_bwd(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool = False,
                    threads: int | None = None, library=None):
    """Exact fp64 gradients (dq [Nq,H,D], dk [Nk,H,D], dv [Nk,H,D]) of the
    attention forward for the upstream gradient dout [Nq,H,D] (all bf16).
    Rows past cu_seqlens_q[-1] and keys past cu_seqlens_k[-1] get 0."""
    qb, kb, vb, gb = _bits(q), _bits(k), _bits(v), _bits(dout)
    if qb.ndim != 3 or gb.shape != qb.shape or kb.shape != vb.shape or kb.shape[1:] != qb.shape[1:]:
        raise ValueError("q and dout must be [Nq,H,D], k and v [Nk,H,D]")
    _, H, D = qb.shape
    cq, ck, B = _segments(cu_seqlens_q, cu_seqlens_k, qb.shape[0], kb.shape[0])
    dq = np.zeros(qb.shape, dtype=np.float64)
    dk = np.zeros(kb.shape, dtype=np.float64)
    dv = np.zeros(kb.shape, dtype=np.float64)
    lib = library if library is not None else _load()
    rc = lib.oracle_attn_varlen_bwd(qb.ctypes.data, kb.ctypes.data, vb.ctypes.data, gb.ctypes.data,
                                    cq.ctypes.data, ck.ctypes.data, B, H, D, float(scale), int(bool(causal)),
                                    dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
                                    int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return dq, dk, dv


def attn_varlen_bwd_dq_rows(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, scale: float, rows,
                            causal: bool = False, threads: int | None = None, library=None):
    """fp64 dq [R,H,D] for the listed global query rows only (rows are independent)."""
    qb, kb, vb, gb = _bits(q), _bits(k), _bits(v), _bits(dout)
    if qb.ndim != 3 or gb.shape != qb.shape or kb.shape != vb.shape or kb.shape[1:] != qb.shape[1:]:
        raise ValueError("q and dout must be [Nq,H,D], k and v [Nk,H,D]")
    _, H, D = qb.shape
    cq, ck, B = _segments(cu_seqlens_q, cu_seqlens_k, qb.shape[0], kb.shape[0])
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    dq = np.zeros((len(r), H, D), dtype=np.float64)
    if len(r) == 0:
        return dq
    lib = library if library is not None else _load()
    rc = lib.oracle_attn_varlen_bwd_dq_rows(qb.ctypes.data, kb.ctypes.data, vb.ctypes.data, gb.ctypes.data,
                                            cq.ctypes.data, ck.ctypes.data, B, H, D, float(scale),
                                            int(bool(causal)), r.ctypes.data, len(r), dq.ctypes.data,
                                            int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return dq


def bwd_preprocess(out, dout, rows=None):
    """The backward's per-row reduction D[i, h] = sum_d out[i,h,d] * dout[i,h,d]
    in fp64, for bf16 out and dout [N,H,D] (the listed rows, or all).
    The _bwd_preprocess page names this kernel without its formula; this
    reduction over dout and out is its plain reading."""
    ob = _bits(out)
    gb = _bits(dout)
    if ob.shape != gb.shape or ob.ndim != 3:
        raise ValueError("out and dout must both be [N,H,D]")
    if rows is not None:
        idx = np.asarray(rows, dtype=np.int64)
        ob, gb = ob[idx], gb[idx]
    wide = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return (wide(ob) * wide(gb)).sum(axis=-1)
