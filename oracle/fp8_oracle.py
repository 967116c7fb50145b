"""Oracle of the low-precision forward: Q and K in OCP FP8 E4M3 with one
scale per head, V and the rest in full precision.

TEST INFRASTRUCTURE ONLY (same status as attn_oracle.c; nothing in the HIP
library or its binding imports it).

The low-precision path is an approximation of attention, so its oracle
follows the method's steps, each in its plain form:
  1. amax_h = max |x[i, h, d]| over the tensor's rows [0, n) and d (exact).
  2. inv_h = 448 / amax_h and scale_h = amax_h / 448, each one IEEE fp32
     division (inv_h = 0, scale_h = 1 for an all-zero head).
  3. code = E4M3(x * inv_h), the product in fp32, rounded to the nearest
     E4M3 value, ties to even. |x * inv_h| <= 448 * (1 + 2^-23), which rounds
     to at most 448, the largest finite value (larger magnitudes would
     saturate to 448 here; step 2 never produces them).
  4. attention in fp64 (blas_oracle) on q^ = E4M3value(code_q) * scale_q and
     k^ likewise; V as given.
E4M3 (OCP 8-bit floating point, "E4M3FN"): 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6;
0x7F and 0xFF are NaN (no infinities), so the largest finite value is
0x7E = 1.75 * 2^8 = 448. Written here from that definition; the pins in
tests/test_oracle_fp8.py check it against torch's float8_e4m3fn.
The page's low-precision path (NVFP4, "ffpa-attn PR #387", "Verification":
cos ~0.982 against SDPA) is the context this stands in for on CDNA4.
"""
from __future__ import annotations

import numpy as np

from . import _bits
from . import blas_oracle

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """float32 values -> uint8 codes, round to nearest, ties to even;
    magnitudes at or above 448 give 448 (finite inputs only)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)  # exact widening
    if not np.all(np.isfinite(x)):
        raise ValueError("finite inputs only")
    sign = (x < 0) | ((x == 0) & np.signbit(x))
    a = np.abs(x)
    # binade of a (normal range 2^-6 .. 2^8); below 2^-6 the spacing is fixed
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    quantum = 2.0 ** (e - 3)                        # spacing of E4M3 values in that binade
    q = np.round(a / quantum) * quantum             # numpy rounds half to even
    q = np.minimum(q, E4M3_MAX)
    # code of the (exactly representable) value q
    qe = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    sub = q < 2.0 ** -6
    efield = np.where(sub, 0, qe + 7).astype(np.int64)
    mant = np.where(sub, q / 2.0 ** -9, (q / 2.0 ** qe - 1.0) * 8).astype(np.int64)
    code = (efield << 3) | mant
    code = np.where(q == 0, 0, code)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def quantize_per_head(x, n_rows: int | None = None):
    """bf16 [N, H, D] (bits or CPU tensor) -> (codes uint8 [n, H, D],
    scale float32 [H], inv float32 [H]) over rows [0, n)."""
    b = _bits(x)
    n = b.shape[0] if n_rows is None else n_rows
    f = (b[:n].astype(np.uint32) << 16).view(np.float32)
    amax = np.abs(f).max(axis=(0, 2)) if n > 0 else np.zeros(b.shape[1], np.float32)
    amax = amax.astype(np.float32)
    pos = amax > 0
    with np.errstate(divide="ignore"):
        inv = np.where(pos, np.float32(E4M3_MAX) / amax, np.float32(0)).astype(np.float32)
        scale = np.where(pos, amax / np.float32(E4M3_MAX), np.float32(1)).astype(np.float32)
    y = (f * inv[None, :, None]).astype(np.float32)   # fp32 product, RNE
    return e4m3_encode(y), scale, inv


def dequantize(codes, scale) -> np.ndarray:
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[None, :, None]


def attn_varlen_fwd_fp8(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, rows=None, causal: bool = False,
                        threads=None):
    """(out [R, H, D], lse [R, H]) float64 of attention on the per-head E4M3
    quantized q and k (rows [0, cu_q[-1]) and [0, cu_k[-1]) set the scales)."""
    cq, ck = int(cu_seqlens_q[-1]), int(cu_seqlens_k[-1])
    qc, qs, _ = quantize_per_head(q, cq)
    kc, ks, _ = quantize_per_head(k, ck)
    qf = dequantize(qc, qs)
    kf = dequantize(kc, ks)
    vf = blas_oracle._widen(_bits(v))
    return blas_oracle.attn_varlen_fwd(qf, kf, vf, cu_seqlens_q, cu_seqlens_k, scale, rows=rows, causal=causal,
                                       threads=threads)
