"""Pins of the backward oracle (oracle/attn_bwd_oracle.c and the preprocessing
reduction in oracle/__init__.py) against facts that do not come from the
oracle itself: central finite differences of an independent fp64 forward,
torch's autograd through its fp64 scaled_dot_product_attention, closed forms,
and invariants of the gradient. A last test plants mistakes in copies of the
oracle and checks that every one of them trips a pin.

All CPU; no GPU needed.
"""
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


def visible(cu_q, cu_k, b, r, causal):
    """Keys of segment b seen by its query row r (0-based within the segment)."""
    lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
    return lk if not causal else max(0, min(lk, r + lk - lq + 1))


def forward64(qf, kf, vf, cu_q, cu_k, scale, causal=False):
    """fp64 forward written independently of the oracle: per row, softmax over
    the visible keys with max subtraction; rows without keys give 0."""
    nq, H, D = qf.shape
    out = np.zeros((nq, H, D))
    for b in range(len(cu_q) - 1):
        for r in range(cu_q[b + 1] - cu_q[b]):
            n = visible(cu_q, cu_k, b, r, causal)
            if n == 0:
                continue
            i = cu_q[b] + r
            ks = slice(cu_k[b], cu_k[b] + n)
            for h in range(H):
                s = scale * (kf[ks, h] @ qf[i, h])
                w = np.exp(s - s.max())
                out[i, h] = (w / w.sum()) @ vf[ks, h]
    return out


def rand_case(rng, cu_q, cu_k, H, D, std=1.0):
    nq, nk = cu_q[-1], cu_k[-1]
    q = to_bf16_bits(rng.standard_normal((nq, H, D)) * std)
    k = to_bf16_bits(rng.standard_normal((nk, H, D)) * std)
    v = to_bf16_bits(rng.standard_normal((nk, H, D)) * std)
    g = to_bf16_bits(rng.standard_normal((nq, H, D)) * std)
    return q, k, v, g


def blas_bwd():
    """The numpy fp64 backward (oracle/blas_oracle.py), held to the same pins."""
    def F(q, k, v, g, cu_q, cu_k, scale, causal=False):
        return blas_oracle.attn_varlen_bwd(q, k, v, g, cu_q, cu_k, scale, causal=causal, row_chunk=7, threads=2)
    F.library = None
    return F


def c_bwd(library=None):
    def F(q, k, v, g, cu_q, cu_k, scale, causal=False):
        return oracle.attn_varlen_bwd(q, k, v, g, cu_q, cu_k, scale, causal=causal, threads=2, library=library)
    F.library = library
    return F


# ---------------------------------------------------------------- pins

TINY = [
    # (cu_q, cu_k, H, D, causal)
    ([0, 3, 8], [0, 4, 6], 2, 4, False),
    ([0, 5, 7], [0, 3, 7], 2, 4, True),        # Lq > Lk: rows 0 and 1 of segment 0 see no key
    ([0, 0, 4, 6], [0, 3, 3, 8], 1, 8, False),  # an empty query segment and an empty key segment
    ([0, 4, 9], [0, 4, 9], 2, 4, True),        # square causal
]


def pin_finite_differences(F):
    """Central differences of L = sum(dout * O) through forward64, every element."""
    rng = np.random.default_rng(5)
    for cu_q, cu_k, H, D, causal in TINY:
        q, k, v, g = rand_case(rng, cu_q, cu_k, H, D)
        scale = 0.6
        dq, dk, dv = F(q, k, v, g, cu_q, cu_k, scale, causal=causal)
        qf, kf, vf, gf = (bits_to_f64(x) for x in (q, k, v, g))
        base = [qf, kf, vf]
        eps = 1e-5
        for which, got in enumerate((dq, dk, dv)):
            x = base[which]
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                keep = x[idx]
                x[idx] = keep + eps
                lp = (gf * forward64(*base, cu_q, cu_k, scale, causal)).sum()
                x[idx] = keep - eps
                lm = (gf * forward64(*base, cu_q, cu_k, scale, causal)).sum()
                x[idx] = keep
                fd[idx] = (lp - lm) / (2 * eps)
            np.testing.assert_allclose(got, fd, rtol=0, atol=2e-7, err_msg=f"{'qkv'[which]} {cu_q} {cu_k} causal={causal}")


def pin_torch_autograd(F):
    """torch's fp64 CPU scaled_dot_product_attention with autograd, per segment."""
    rng = np.random.default_rng(6)
    for cu_q, cu_k, causal in (([0, 17, 40], [0, 29, 41], False), ([0, 23, 60], [0, 23, 60], True)):
        H, D = 2, 16
        q, k, v, g = rand_case(rng, cu_q, cu_k, H, D)
        scale = 0.3
        dq, dk, dv = F(q, k, v, g, cu_q, cu_k, scale, causal=causal)
        qt, kt, vt, gt = (torch.from_numpy(bits_to_f64(x)) for x in (q, k, v, g))
        for b in range(len(cu_q) - 1):
            qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
            qq, kk, vv = (t[s].transpose(0, 1).clone().requires_grad_() for t, s in ((qt, qs), (kt, ks), (vt, ks)))
            o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale, is_causal=causal)
            o.backward(gt[qs].transpose(0, 1))
            np.testing.assert_allclose(dq[qs], qq.grad.transpose(0, 1).numpy(), atol=1e-12, rtol=0)
            np.testing.assert_allclose(dk[ks], kk.grad.transpose(0, 1).numpy(), atol=1e-12, rtol=0)
            np.testing.assert_allclose(dv[ks], vv.grad.transpose(0, 1).numpy(), atol=1e-12, rtol=0)


def pin_closed_forms(F):
    rng = np.random.default_rng(7)
    # one key per segment: O_i = v_0 whatever q and k are, so dq = dk = 0 and dv_0 = sum_i dout_i
    cu_q, cu_k = [0, 5, 9], [0, 1, 2]
    q, k, v, g = rand_case(rng, cu_q, cu_k, 2, 8)
    dq, dk, dv = F(q, k, v, g, cu_q, cu_k, 0.5)
    gf = bits_to_f64(g)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    np.testing.assert_allclose(dv[0], gf[0:5].sum(0), atol=1e-13)
    np.testing.assert_allclose(dv[1], gf[5:9].sum(0), atol=1e-13)
    # equal keys: uniform weights 1/Lk, so dv_j = sum_i dout_i / Lk and dq = 0
    cu_q, cu_k = [0, 6], [0, 4]
    q, k, v, g = rand_case(rng, cu_q, cu_k, 1, 8)
    k[:] = k[0]
    dq, dk, dv = F(q, k, v, g, cu_q, cu_k, 0.5)
    gf = bits_to_f64(g)
    assert np.abs(dq).max() < 1e-13
    for j in range(4):
        np.testing.assert_allclose(dv[j], gf.sum(0) / 4, atol=1e-13)
    # equal values: O_i = u for every weighting, so dq = dk = 0
    q, k, v, g = rand_case(rng, cu_q, cu_k, 1, 8)
    v[:] = v[0]
    dq, dk, dv = F(q, k, v, g, cu_q, cu_k, 0.5)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    # causal with Lq = Lk = 2: row 0 sees key 0 only, so its dq is 0 and key 1 gets only row 1's weight
    cu_q = cu_k = [0, 2]
    q, k, v, g = rand_case(rng, cu_q, cu_k, 1, 4)
    dq, dk, dv = F(q, k, v, g, cu_q, cu_k, 0.5, causal=True)
    qf, kf, vf, gf = (bits_to_f64(x) for x in (q, k, v, g))
    assert np.abs(dq[0]).max() < 1e-15
    s = 0.5 * (kf[:, 0] @ qf[1, 0])
    p = np.exp(s - s.max())
    p /= p.sum()
    np.testing.assert_allclose(dv[1, 0], p[1] * gf[1, 0], atol=1e-14)
    np.testing.assert_allclose(dv[0, 0], gf[0, 0] + p[0] * gf[1, 0], atol=1e-14)


def pin_invariants(F):
    rng = np.random.default_rng(8)
    cu_q, cu_k = [0, 37, 100, 100], [0, 50, 81, 90]
    H, D = 3, 16
    for causal in (False, True):
        q, k, v, g = rand_case(rng, cu_q, cu_k, H, D)
        dq, dk, dv = F(q, k, v, g, cu_q, cu_k, 0.25, causal=causal)
        gf = bits_to_f64(g)
        for b in range(3):
            ks = slice(cu_k[b], cu_k[b + 1])
            # softmax weights of a row sum to 1: sum_j ds_j = 0, hence sum_j dk_j = 0
            assert np.abs(dk[ks].sum(0)).max() < 1e-12
            # sum_j dv_j = sum over rows that see a key of dout_i
            seen = [cu_q[b] + r for r in range(cu_q[b + 1] - cu_q[b]) if visible(cu_q, cu_k, b, r, causal) > 0]
            np.testing.assert_allclose(dv[ks].sum(0), gf[seen].sum(0) if seen else 0.0, atol=1e-12)
        # gradients are linear in dout; doubling is exact in binary floating point
        dq2, dk2, dv2 = F(q, k, v, to_bf16_bits(2 * bits_to_f64(g)), cu_q, cu_k, 0.25, causal=causal)
        assert np.array_equal(dq2, 2 * dq) and np.array_equal(dk2, 2 * dk) and np.array_equal(dv2, 2 * dv)
    # shifting every key of a segment by one vector c moves each score row by a
    # constant: the weights, dk and dv stay, and dq gains scale * c * sum_j ds_j = 0
    cu_q, cu_k = [0, 9], [0, 12]
    q = to_bf16_bits(rng.integers(-16, 17, (9, 2, 8)) / 8.0)
    k = to_bf16_bits(rng.integers(-16, 17, (12, 2, 8)) / 8.0)
    v, g = (to_bf16_bits(rng.standard_normal((n, 2, 8))) for n in (12, 9))
    c = rng.integers(-8, 9, (1, 2, 8)) / 8.0
    k2 = to_bf16_bits(bits_to_f64(k) + c)
    assert np.array_equal(bits_to_f64(k2), bits_to_f64(k) + c)  # the shift is exact in bf16
    a = F(q, k, v, g, cu_q, cu_k, 0.25)
    b2 = F(q, k2, v, g, cu_q, cu_k, 0.25)
    for x, y in zip(a, b2):
        np.testing.assert_allclose(x, y, atol=1e-12)


def pin_dq_rows_match(F):
    """dq of listed rows (row mode) equals the full computation's rows."""
    rng = np.random.default_rng(9)
    cu_q, cu_k = [0, 20, 45], [0, 33, 40]
    q, k, v, g = rand_case(rng, cu_q, cu_k, 2, 8)
    for causal in (False, True):
        dq, _, _ = F(q, k, v, g, cu_q, cu_k, 0.4, causal=causal)
        rows = [44, 0, 19, 20, 31]
        r = oracle.attn_varlen_bwd_dq_rows(q, k, v, g, cu_q, cu_k, 0.4, rows, causal=causal, threads=2,
                                           library=F.library)
        assert np.array_equal(r, dq[rows])


PINS = [pin_finite_differences, pin_torch_autograd, pin_closed_forms, pin_invariants, pin_dq_rows_match]


@pytest.fixture(scope="module")
def built_oracle():
    oracle.build(force=False)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_bwd_oracle_pin(pin, built_oracle):
    pin(c_bwd())


@pytest.mark.parametrize("pin", PINS[:-1], ids=lambda p: p.__name__)
def test_blas_bwd_oracle_pin(pin, built_oracle):
    """The same pins hold the numpy backward (row chunks of 7 rows, so every
    case spans several chunks and the chunk boundaries of dK and dV); the
    row-mode pin is the C library's own."""
    pin(blas_bwd())


@pytest.mark.parametrize("causal", [False, True])
def test_blas_bwd_agrees_with_c_bwd(causal, built_oracle):
    """Two independent implementations of the same chain rule agree on ragged
    segments with empty ones (the C oracle loops per row in fp64; the numpy one
    uses matrix products in row chunks)."""
    rng = np.random.default_rng(11)
    cu_q, cu_k = [0, 61, 61, 140, 141], [0, 45, 80, 80, 203]
    q, k, v, g = rand_case(rng, cu_q, cu_k, 3, 32)
    a = c_bwd()(q, k, v, g, cu_q, cu_k, 0.17, causal=causal)
    b = blas_oracle.attn_varlen_bwd(q, k, v, g, cu_q, cu_k, 0.17, causal=causal, row_chunk=16, threads=3)
    for x, y in zip(a, b):
        np.testing.assert_allclose(y, x, rtol=0, atol=1e-12)


def test_preprocess_reduction():
    """D[i,h] = sum_d out*dout: exact integers, and an explicit loop in long double."""
    ones = to_bf16_bits(np.ones((3, 2, 96)))
    assert np.array_equal(oracle.bwd_preprocess(ones, ones), np.full((3, 2), 96.0))
    rng = np.random.default_rng(10)
    o = to_bf16_bits(rng.standard_normal((7, 3, 64)))
    g = to_bf16_bits(rng.standard_normal((7, 3, 64)))
    got = oracle.bwd_preprocess(o, g)
    of, gf = bits_to_f64(o), bits_to_f64(g)
    for i in range(7):
        for h in range(3):
            acc = np.longdouble(0)
            for d in range(64):
                acc += np.longdouble(of[i, h, d]) * np.longdouble(gf[i, h, d])
            assert abs(got[i, h] - float(acc)) < 1e-12
    assert np.array_equal(oracle.bwd_preprocess(o, g, rows=[6, 2]), got[[6, 2]])


def test_bwd_oracle_rejects_bad_arguments():
    rng = np.random.default_rng(11)
    q, k, v, g = rand_case(rng, [0, 4], [0, 4], 1, 8)
    with pytest.raises(ValueError):
        oracle.attn_varlen_bwd(q, k, v, g, [0, 5], [0, 4], 0.5)          # past the rows
    with pytest.raises(ValueError):
        oracle.attn_varlen_bwd(q, k, v, g, [0, 3, 2], [0, 2, 4], 0.5)    # decreasing cu
    with pytest.raises(ValueError):
        oracle.attn_varlen_bwd_dq_rows(q, k, v, g, [0, 4], [0, 4], 0.5, [4])  # row outside every segment
    with pytest.raises(ValueError):
        oracle.attn_varlen_bwd(q, k, v, g[:3], [0, 3], [0, 4], 0.5)       # dout shape


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "no_D_term": ("const double ds = p[j] * (dp[j] - Di);", "const double ds = p[j] * dp[j];"),
    "D_sign": ("const double ds = p[j] * (dp[j] - Di);", "const double ds = p[j] * (dp[j] + Di);"),
    "dq_no_scale": ("for (int32_t d = 0; d < D; ++d) dq_row[d] *= job->scale;", ""),
    "dk_uses_k": ("dkj[d] += job->scale * ds * widen(qi[d]);", "dkj[d] += job->scale * ds * widen(job->k[((k0 + j) * H + h) * D + d]);"),
    "dv_uses_ds": ("dvj[d] += p[j] * widen(gi[d]);", "dvj[d] += ds * widen(gi[d]);"),
    "dp_uses_q": ("g += widen(gi[d]) * widen(vj[d]);", "g += widen(qi[d]) * widen(vj[d]);"),
    "p_unnormalised": ("p[j] /= l;", "p[j] /= 1.0;"),
    "causal_off_by_one": ("const int64_t n = (row - job->cu_q[b]) + lk - lq + 1;",
                          "const int64_t n = (row - job->cu_q[b]) + lk - lq;"),
    "causal_ignored": ("if (!job->causal) return lk;", "return lk;"),
    "dk_no_scale": ("dkj[d] += job->scale * ds * widen(qi[d]);", "dkj[d] += ds * widen(qi[d]);"),
    "v_head0": ("const uint16_t *vj = job->v + ((k0 + j) * H + h) * D;",
                "const uint16_t *vj = job->v + ((k0 + j) * H + 0) * D;"),
}


def _build_mutant(tmp_path: Path, name: str) -> Path:
    old, new = MUTANTS[name]
    src = (ROOT / "oracle" / "attn_bwd_oracle.c").read_text()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mdir = tmp_path / name
    mdir.mkdir()
    (mdir / "m.c").write_text(src.replace(old, new))
    lib = mdir / "libm.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-o", str(lib),
                    str(ROOT / "oracle" / "attn_oracle.c"), str(mdir / "m.c"), "-lm"], check=True)
    return lib


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc needed to build mutants")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_pins_catch_planted_mistake(tmp_path, name):
    F = c_bwd(oracle.load_library(_build_mutant(tmp_path, name)))
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(F)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
