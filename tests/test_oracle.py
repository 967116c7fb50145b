"""Pins of the CPU oracle (oracle/attn_oracle.c) against facts that do not come
from the oracle itself: a brute-force evaluation in extended precision, a
library routine (torch's fp64 scaled_dot_product_attention and logsumexp),
closed forms, and invariants of the definition. A last test plants mistakes in
copies of the oracle and checks that every one of them trips a pin.

All CPU; no GPU needed.
"""
import math
import re
import shutil
import subprocess
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
from oracle import blas_oracle

ROOT = Path(__file__).resolve().parents[1]


# ---------------------------------------------------------------- helpers (test side)

def to_bf16_bits(x) -> np.ndarray:
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_case(rng, cu_q, cu_k, H, D, std=1.0):
    nq, nk = cu_q[-1], cu_k[-1]
    q = to_bf16_bits(rng.standard_normal((nq, H, D)) * std)
    k = to_bf16_bits(rng.standard_normal((nk, H, D)) * std)
    v = to_bf16_bits(rng.standard_normal((nk, H, D)) * std)
    return q, k, v


def brute_force(q, k, v, cu_q, cu_k, scale, causal=False):
    """Explicit score matrix in long double, softmax WITHOUT max subtraction
    (exp(s)/sum exp(s)); valid for the small |s| used here. causal: a 0/1
    visibility matrix, 1 where key j <= row r + Lk - Lq (bottom-right
    aligned); rows with no visible key give 0 and -inf."""
    qf, kf, vf = (bits_to_f64(x).astype(np.longdouble) for x in (q, k, v))
    nq, H, D = qf.shape
    out = np.zeros((nq, H, D), dtype=np.longdouble)
    lse = np.zeros((nq, H), dtype=np.longdouble)
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        for h in range(H):
            if qe == qs:
                continue
            if ke == ks:
                out[qs:qe, h] = 0
                lse[qs:qe, h] = -np.inf
                continue
            S = np.longdouble(scale) * (qf[qs:qe, h] @ kf[ks:ke, h].T)
            E = np.exp(S)
            if causal:
                lq, lk = qe - qs, ke - ks
                vis = np.array([[1 if j <= r + lk - lq else 0 for j in range(lk)] for r in range(lq)],
                               dtype=np.longdouble)
                E = E * vis
            Z = E.sum(axis=1, keepdims=True)
            none = Z[:, 0] == 0
            out[qs:qe, h] = np.where(none[:, None], 0, (E / np.where(none, 1, Z[:, 0])[:, None]) @ vf[ks:ke, h])
            with np.errstate(divide="ignore"):
                lse[qs:qe, h] = np.log(Z[:, 0])
    return out.astype(np.float64), lse.astype(np.float64)


def sdpa_reference(q, k, v, cu_q, cu_k, scale):
    """torch's fp64 CPU scaled_dot_product_attention per segment, LSE by torch.logsumexp."""
    qf, kf, vf = (torch.from_numpy(bits_to_f64(x)) for x in (q, k, v))
    nq, H, D = qf.shape
    out = torch.zeros((nq, H, D), dtype=torch.float64)
    lse = torch.zeros((nq, H), dtype=torch.float64)
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if qe == qs or ke == ks:
            continue
        Q = qf[qs:qe].permute(1, 0, 2).unsqueeze(0)
        K = kf[ks:ke].permute(1, 0, 2).unsqueeze(0)
        V = vf[ks:ke].permute(1, 0, 2).unsqueeze(0)
        O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
        out[qs:qe] = O[0].permute(1, 0, 2)
        S = scale * torch.matmul(Q, K.transpose(-1, -2).contiguous())
        lse[qs:qe] = torch.logsumexp(S, dim=-1)[0].T
    return out.numpy(), lse.numpy()


def c_oracle(library=None):
    """The C oracle (default build, or a planted-mistake build) as a callable."""
    def F(q, k, v, cu_q, cu_k, scale, rows=None, threads=4, causal=False):
        return oracle.attn_varlen_fwd(q, k, v, cu_q, cu_k, scale, rows=rows, threads=threads,
                                      library=library, causal=causal)
    F.bitwise = True   # row results do not depend on which other rows are evaluated
    return F


def blas_oracle_fn(q, k, v, cu_q, cu_k, scale, rows=None, threads=None, causal=False):
    return blas_oracle.attn_varlen_fwd(q, k, v, cu_q, cu_k, scale, rows=rows, row_chunk=3, causal=causal)


# a BLAS product's rounding may depend on the operand shapes, so row results
# can differ in the last bits with the set of rows evaluated together
blas_oracle_fn.bitwise = False


def same(F, a, b):
    if F.bitwise:
        return np.array_equal(a, b)
    fa, fb = np.isfinite(a), np.isfinite(b)
    return np.array_equal(fa, fb) and np.array_equal(a[~fa], b[~fb]) and np.allclose(a[fa], b[fb], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- pins (each takes an oracle callable)

def pin_brute_force(F):
    rng = np.random.default_rng(1)
    for cu_q, cu_k, H, D in [([0, 3, 3, 9], [0, 5, 6, 6], 2, 8), ([0, 7], [0, 4], 1, 4),
                             ([0, 1, 4], [0, 9, 11], 2, 6)]:
        q, k, v = rand_case(rng, cu_q, cu_k, H, D)
        scale = 1.0 / math.sqrt(D)
        o, l = F(q, k, v, cu_q, cu_k, scale)
        bo, bl = brute_force(q, k, v, cu_q, cu_k, scale)
        np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-13)
        fin = np.isfinite(bl)
        np.testing.assert_array_equal(np.isfinite(l), fin)
        np.testing.assert_allclose(l[fin], bl[fin], rtol=1e-12, atol=1e-13)
        assert np.all(l[~fin] == -np.inf)


def pin_small_integers(F):
    """Small-integer inputs: scores are exact, so O and LSE follow from a few
    exponentials; compare with Python's own math on exact rationals."""
    from fractions import Fraction
    q = to_bf16_bits([[[1, 0]], [[0, 2]]])          # 2 rows, H=1, D=2
    k = to_bf16_bits([[[1, 1]], [[2, -1]], [[0, 1]]])
    v = to_bf16_bits([[[3, 0]], [[0, 5]], [[1, 1]]])
    o, l = F(q, k, v, [0, 2], [0, 3], 1.0)
    for i, qi in enumerate(([1, 0], [0, 2])):
        s = [qi[0] * kk[0] + qi[1] * kk[1] for kk in ([1, 1], [2, -1], [0, 1])]
        w = [math.exp(x) for x in s]
        z = math.fsum(w)
        exp_o = [math.fsum(wj * vj[d] for wj, vj in zip(w, ([3, 0], [0, 5], [1, 1]))) / z for d in range(2)]
        np.testing.assert_allclose(o[i, 0], exp_o, rtol=1e-14)
        assert abs(l[i, 0] - math.log(z)) < 1e-14
    assert Fraction(1)  # (exact scores: integers)


def pin_sdpa(F):
    rng = np.random.default_rng(2)
    cu_q, cu_k, H, D = [0, 300, 700, 1000], [0, 500, 510, 1300], 2, 64
    q, k, v = rand_case(rng, cu_q, cu_k, H, D, std=1.0)
    scale = 1.0 / math.sqrt(D)
    o, l = F(q, k, v, cu_q, cu_k, scale)
    so, sl = sdpa_reference(q, k, v, cu_q, cu_k, scale)
    np.testing.assert_allclose(o, so, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(l, sl, rtol=1e-12, atol=1e-12)


def pin_closed_forms(F):
    rng = np.random.default_rng(3)
    H, D = 2, 8
    # one key: O = v0, LSE = s0
    q, k, v = rand_case(rng, [0, 4], [0, 1], H, D)
    o, l = F(q, k, v, [0, 4], [0, 1], 0.5)
    vf, qf, kf = bits_to_f64(v), bits_to_f64(q), bits_to_f64(k)
    for i in range(4):
        for h in range(H):
            np.testing.assert_array_equal(o[i, h], vf[0, h])
            s0 = 0.5 * float(np.dot(qf[i, h], kf[0, h]))
            assert abs(l[i, h] - s0) <= 1e-13 * max(1.0, abs(s0))
    # Q = 0: O = mean(V), LSE = ln(Lk)
    q0 = to_bf16_bits(np.zeros((3, H, D)))
    _, k, v = rand_case(rng, [0, 3], [0, 7], H, D)
    o, l = F(q0, k, v, [0, 3], [0, 7], 0.3)
    np.testing.assert_allclose(o, np.broadcast_to(bits_to_f64(v).mean(axis=0), o.shape), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l, math.log(7), rtol=1e-15)
    # V constant per head: O = that constant
    q, k, _ = rand_case(rng, [0, 5], [0, 6], H, D)
    vc = to_bf16_bits(np.broadcast_to(np.array([0.75, -2.5])[None, :, None], (6, H, D)))
    o, _ = F(q, k, vc, [0, 5], [0, 6], 0.25)
    np.testing.assert_allclose(o[:, 0], 0.75, rtol=1e-14)
    np.testing.assert_allclose(o[:, 1], -2.5, rtol=1e-14)
    # two keys: O = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1
    q, k, v = rand_case(rng, [0, 4], [0, 2], H, D)
    o, l = F(q, k, v, [0, 4], [0, 2], 0.7)
    qf, kf, vf = bits_to_f64(q), bits_to_f64(k), bits_to_f64(v)
    for i in range(4):
        for h in range(H):
            s0 = 0.7 * float(np.dot(qf[i, h], kf[0, h]))
            s1 = 0.7 * float(np.dot(qf[i, h], kf[1, h]))
            a0 = 1.0 / (1.0 + math.exp(s1 - s0))
            np.testing.assert_allclose(o[i, h], a0 * vf[0, h] + (1 - a0) * vf[1, h], rtol=1e-12, atol=1e-14)
            exp_l = max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1)))
            assert abs(l[i, h] - exp_l) <= 1e-12 * max(1.0, abs(exp_l))
    # empty key segment: O = 0, LSE = -inf; other segment unaffected
    q, k, v = rand_case(rng, [0, 2, 5], [0, 0, 4], H, D)
    o, l = F(q, k, v, [0, 2, 5], [0, 0, 4], 0.4)
    assert np.all(o[:2] == 0) and np.all(l[:2] == -np.inf)
    assert np.all(np.isfinite(l[2:]))


def pin_needle(F):
    """q = alpha * k_t with a large alpha: softmax is one-hot at t, O = v_t.
    Also large logits (|s| ~ 1e3) must not overflow."""
    rng = np.random.default_rng(4)
    H, D, nk = 1, 16, 12
    k = to_bf16_bits(rng.choice([-1.0, 1.0], size=(nk, H, D)))
    v = to_bf16_bits(rng.standard_normal((nk, H, D)))
    for t in (0, 5, nk - 1):
        q = to_bf16_bits(64.0 * bits_to_f64(k)[t:t + 1])
        o, l = F(q, k, v, [0, 1], [0, nk], 1.0)
        np.testing.assert_allclose(o[0, 0], bits_to_f64(v)[t, 0], rtol=0, atol=1e-6)
        assert abs(l[0, 0] - 64.0 * D) < 1e-6
        assert np.all(np.isfinite(o))


def pin_invariants(F):
    rng = np.random.default_rng(5)
    cu_q, cu_k, H, D = [0, 6, 13, 20], [0, 9, 10, 25], 2, 16
    q, k, v = rand_case(rng, cu_q, cu_k, H, D)
    scale = 0.25
    o, l = F(q, k, v, cu_q, cu_k, scale)
    # key permutation within a segment (k and v rows together)
    perm = np.concatenate([rng.permutation(np.arange(a, b)) for a, b in zip(cu_k[:-1], cu_k[1:])])
    op, lp = F(q, k[perm], v[perm], cu_q, cu_k, scale)
    np.testing.assert_allclose(op, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lp, l, rtol=1e-12, atol=1e-14)
    # segment independence: other segments' data changed, segment 1 bitwise equal
    q2, k2, v2 = rand_case(rng, cu_q, cu_k, H, D)
    q2[6:13], k2[9:10], v2[9:10] = q[6:13], k[9:10], v[9:10]
    o2, l2 = F(q2, k2, v2, cu_q, cu_k, scale)
    assert same(F, o2[6:13], o[6:13]) and same(F, l2[6:13], l[6:13])
    # packed == per-segment runs
    for b in range(3):
        ob, lb = F(q[cu_q[b]:cu_q[b + 1]], k[cu_k[b]:cu_k[b + 1]], v[cu_k[b]:cu_k[b + 1]],
                     [0, cu_q[b + 1] - cu_q[b]], [0, cu_k[b + 1] - cu_k[b]], scale)
        assert same(F, ob, o[cu_q[b]:cu_q[b + 1]]) and same(F, lb, l[cu_q[b]:cu_q[b + 1]])
    # row subset and thread count do not change values
    rows = [19, 0, 7, 12]
    orow, lrow = F(q, k, v, cu_q, cu_k, scale, rows=rows, threads=1)
    assert same(F, orow, o[rows]) and same(F, lrow, l[rows])
    # softmax rows sum to one: V = identity gives O = P
    nk = 8
    qi, ki, _ = rand_case(rng, [0, 5], [0, nk], 1, nk)
    vi = to_bf16_bits(np.eye(nk)[:, None, :])
    oi, li = F(qi, ki, vi, [0, 5], [0, nk], 0.5)
    np.testing.assert_allclose(oi.sum(axis=-1), 1.0, rtol=0, atol=1e-14)
    assert np.all(oi >= 0)
    s = 0.5 * np.einsum("id,jd->ij", bits_to_f64(qi)[:, 0], bits_to_f64(ki)[:, 0])
    np.testing.assert_allclose(oi[:, 0], np.exp(s - li), rtol=1e-12)
    # scaling q by 2 (exact in bf16) equals doubling the scale
    qd = to_bf16_bits(2.0 * bits_to_f64(q))
    o3, l3 = F(qd, k, v, cu_q, cu_k, scale)
    o4, l4 = F(q, k, v, cu_q, cu_k, 2 * scale)
    np.testing.assert_allclose(o3, o4, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l3, l4, rtol=1e-13, atol=1e-15)


# ---- causal (bottom-right aligned mask; a reading, the pages only use causal=False)

CAUSAL_CASES = [([0, 6], [0, 6], 2, 8),            # square
                ([0, 3, 9], [0, 7, 10], 2, 4),       # Lq < Lk, then Lq > Lk (rows with no key)
                ([0, 5, 5, 7], [0, 2, 4, 4], 1, 6),  # Lq > Lk, empty Lq, empty Lk
                ([0, 1, 4], [0, 9, 11], 2, 6)]


def pin_causal_brute_force(F):
    rng = np.random.default_rng(21)
    for cu_q, cu_k, H, D in CAUSAL_CASES:
        q, k, v = rand_case(rng, cu_q, cu_k, H, D)
        scale = 1.0 / math.sqrt(D)
        o, l = F(q, k, v, cu_q, cu_k, scale, causal=True)
        bo, bl = brute_force(q, k, v, cu_q, cu_k, scale, causal=True)
        np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-13)
        fin = np.isfinite(bl)
        np.testing.assert_array_equal(np.isfinite(l), fin)
        np.testing.assert_allclose(l[fin], bl[fin], rtol=1e-12, atol=1e-13)
        assert np.all(l[~fin] == -np.inf) and np.all(o[~fin] == 0)


def pin_causal_sdpa_square(F):
    """torch's fp64 SDPA with is_causal=True (top-left aligned, which equals
    bottom-right when Lq == Lk) on square segments."""
    rng = np.random.default_rng(22)
    cu = [0, 17, 17, 40]
    q, k, v = rand_case(rng, cu, cu, 3, 16)
    o, l = F(q, k, v, cu, cu, 0.25, causal=True)
    qf, kf, vf = (torch.from_numpy(bits_to_f64(x)) for x in (q, k, v))
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        if e == s:
            continue
        Q, K, V = (t[s:e].permute(1, 0, 2).unsqueeze(0) for t in (qf, kf, vf))
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=0.25, is_causal=True)
        np.testing.assert_allclose(o[s:e], ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def pin_causal_prefix(F):
    """Causal row r equals the unmasked result over the keys 0..r+Lk-Lq of its
    segment (a one-segment run with cu_k cut there)."""
    rng = np.random.default_rng(23)
    cu_q, cu_k = [0, 5, 12], [0, 9, 15]
    q, k, v = rand_case(rng, cu_q, cu_k, 2, 8)
    o, l = F(q, k, v, cu_q, cu_k, 0.3, causal=True)
    for b in range(2):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for r in range(lq):
            n = min(lk, r + lk - lq + 1)
            row = cu_q[b] + r
            if n <= 0:
                assert np.all(o[row] == 0) and np.all(l[row] == -np.inf)
                continue
            qs = q[row:row + 1]
            ks = k[cu_k[b]:cu_k[b] + n]
            vs = v[cu_k[b]:cu_k[b] + n]
            po, pl = F(qs, ks, vs, [0, 1], [0, n], 0.3)
            np.testing.assert_allclose(o[row], po[0], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(l[row], pl[0], rtol=1e-13, atol=1e-15)


def pin_causal_closed_forms(F):
    rng = np.random.default_rng(24)
    # square: row 0 sees only key 0 (o = v0, lse = s00); the last row sees all keys
    cu = [0, 8]
    q, k, v = rand_case(rng, cu, cu, 2, 8)
    o, l = F(q, k, v, cu, cu, 0.5, causal=True)
    on, ln = F(q, k, v, cu, cu, 0.5)
    np.testing.assert_array_equal(o[0], bits_to_f64(v[0]))
    s00 = 0.5 * np.sum(bits_to_f64(q[0]) * bits_to_f64(k[0]), axis=-1)
    np.testing.assert_allclose(l[0], s00, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(o[7], on[7], rtol=1e-14, atol=1e-15)
    # Lq > Lk: the first Lq - Lk rows see nothing; Lq < Lk: row 0 sees Lk - Lq + 1 keys
    q, k, v = rand_case(rng, [0, 6], [0, 2], 1, 4)
    o, l = F(q, k, v, [0, 6], [0, 2], 1.0, causal=True)
    assert np.all(o[:4] == 0) and np.all(l[:4] == -np.inf) and np.all(np.isfinite(l[4:]))
    np.testing.assert_array_equal(o[4, 0], bits_to_f64(v[0, 0]))


PINS = [pin_brute_force, pin_small_integers, pin_sdpa, pin_closed_forms, pin_needle, pin_invariants,
        pin_causal_brute_force, pin_causal_sdpa_square, pin_causal_prefix, pin_causal_closed_forms]


IMPLS = {"c": None, "blas": blas_oracle_fn}


@pytest.fixture(scope="module")
def built_oracle():
    oracle.build(force=False)


@pytest.mark.parametrize("impl", sorted(IMPLS))
@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin, impl, built_oracle):
    pin(c_oracle() if impl == "c" else IMPLS[impl])


def test_c_and_blas_oracles_agree():
    rng = np.random.default_rng(9)
    cu_q, cu_k, H, D = [0, 130, 131, 400], [0, 257, 300, 300], 3, 96
    q, k, v = rand_case(rng, cu_q, cu_k, H, D, std=1.0)
    rows = [0, 5, 129, 130, 131, 399, 250]
    o1, l1 = c_oracle()(q, k, v, cu_q, cu_k, 0.1, rows=rows)
    o2, l2 = blas_oracle_fn(q, k, v, cu_q, cu_k, 0.1, rows=rows)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-13)
    fin = np.isfinite(l1)
    assert np.array_equal(fin, np.isfinite(l2)) and np.all(l2[~fin] == -np.inf)
    np.testing.assert_allclose(l1[fin], l2[fin], rtol=1e-12, atol=1e-13)


def test_c_and_blas_oracles_agree_causal():
    rng = np.random.default_rng(10)
    cu_q, cu_k, H, D = [0, 130, 131, 400, 450], [0, 257, 300, 300, 420], 2, 64
    q, k, v = rand_case(rng, cu_q, cu_k, H, D, std=1.0)
    rows = [0, 5, 129, 130, 131, 132, 399, 250, 400, 449]
    o1, l1 = c_oracle()(q, k, v, cu_q, cu_k, 0.1, rows=rows, causal=True)
    o2, l2 = blas_oracle_fn(q, k, v, cu_q, cu_k, 0.1, rows=rows, causal=True)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-13)
    fin = np.isfinite(l1)
    assert np.array_equal(fin, np.isfinite(l2)) and np.all(l2[~fin] == -np.inf)
    np.testing.assert_allclose(l1[fin], l2[fin], rtol=1e-12, atol=1e-13)


def test_oracle_rejects_bad_arguments():
    q = to_bf16_bits(np.zeros((4, 1, 8)))
    with pytest.raises(ValueError):
        oracle.attn_varlen_fwd(q, q, q, [0, 5], [0, 4], 1.0)            # row count mismatch
    with pytest.raises(ValueError):
        oracle.attn_varlen_fwd(q, q, q, [0, 4], [0, 4], 1.0, rows=[4])  # row outside segments
    with pytest.raises(ValueError):
        oracle.attn_varlen_fwd(q, q, q, [1, 4], [0, 4], 1.0)            # cu[0] != 0


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "dropped_scale": ("scores[j] = job->scale * dot;", "scores[j] = dot;"),
    "lse_sign": ("job->lse[r * H + h] = m + log(l);", "job->lse[r * H + h] = m - log(l);"),
    "shift_sign": ("scores[j] = exp(scores[j] - m);", "scores[j] = exp(scores[j] + m);"),
    "no_normalise": ("for (int32_t d = 0; d < D; ++d) o[d] /= l;", ""),
    "v_head0": ("const uint16_t *vj = job->v + ((k0 + j) * H + h) * D;",
                "const uint16_t *vj = job->v + ((k0 + j) * H + 0) * D;"),
    "k_dim_shift": ("bf16_bits_to_double(kj[d]);", "bf16_bits_to_double(kj[(d + 1) % D]);"),
    "drop_last_key": ("int64_t nk = k1 - k0;", "int64_t nk = (k1 - k0 > 1) ? k1 - k0 - 1 : k1 - k0;"),
    "causal_top_left": ("const int64_t visible = (row - job->cu_q[b]) + nk - lq + 1;",
                        "const int64_t visible = (row - job->cu_q[b]) + 1;"),
    "causal_off_by_one": ("const int64_t visible = (row - job->cu_q[b]) + nk - lq + 1;",
                          "const int64_t visible = (row - job->cu_q[b]) + nk - lq;"),
    "causal_ignored": ("nk = visible < 0 ? 0 : (visible < nk ? visible : nk);", "(void)visible;"),
    "min_not_max": ("if (scores[j] > m) m = scores[j];", "if (scores[j] < m) m = scores[j];"),
    "q_next_row": ("const uint16_t *qi = job->q + (row * H + h) * D;",
                   "const uint16_t *qi = job->q + ((row > 0 ? row - 1 : row) * H + h) * D;"),
}


def _build_mutant(tmp_path: Path, name: str) -> Path:
    old, new = MUTANTS[name]
    src = (ROOT / "oracle" / "attn_oracle.c").read_text()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mdir = tmp_path / name
    mdir.mkdir()
    (mdir / "m.c").write_text(src.replace(old, new))
    lib = mdir / "libm.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-o", str(lib),
                    str(mdir / "m.c"), "-lm"], check=True)
    return lib


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc needed to build mutants")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, name):
    F = c_oracle(oracle.load_library(_build_mutant(tmp_path, name)))
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(F)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
