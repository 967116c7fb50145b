"""GPU tests of the backward (preprocessing pass, dK/dV and dQ kernels)
against the CPU oracle's exact fp64 gradients, through the C ABI. Marked
`gpu`; every case prints its name before it touches the GPU.

The forward's out and lse fed to the backward come from the library's own
forward (its parity is tested separately); the oracle's gradients depend on
q, k, v and dout only.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import blas_oracle
import varlen_flashattention_forward_amd as avf
from varlen_flashattention_forward_amd.workloads import WORKLOADS, custom, make_dout, make_inputs, sample_rows

from parity import compare_grad

pytestmark = pytest.mark.gpu


def announce(label):
    print(f"\n[gpu-case] {label}", flush=True)


def f32(x):
    return float(np.float32(x))


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    avf.lib()
    yield
    torch.cuda.synchronize()


def forward(t, w, causal):
    o, l = avf.attn_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                               softmax_scale=w.softmax_scale, out=t["out"], lse=t["lse"], causal=causal,
                               cu_seqlens_q_host=list(w.cu_q), cu_seqlens_k_host=list(w.cu_k))
    return o, l


def backward(t, w, dout, causal, hostcu=True, **kw):
    o, l = forward(t, w, causal)
    cu = dict(cu_seqlens_q_host=list(w.cu_q), cu_seqlens_k_host=list(w.cu_k)) if hostcu else {}
    r = avf.attn_varlen_bwd(t["q"], t["k"], t["v"], o, dout, l, t["cu_q"], t["cu_k"], w.max_seqlen_q,
                            w.max_seqlen_k, softmax_scale=w.softmax_scale, causal=causal, **cu, **kw)
    torch.cuda.synchronize()
    return r


def oracle_grads(t, w, dout, causal):
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    return oracle.attn_varlen_bwd(q, k, v, dout.contiguous().cpu(), w.cu_q, w.cu_k, f32(w.softmax_scale),
                                  causal=causal)


def check_all(label, got, ref, w):
    """Compare dq over the segments' query rows and dk/dv over their key rows."""
    dq, dk, dv = (x.float().cpu().numpy() for x in got[:3])
    rq, rk, rv = ref
    nq, nk = w.total_q, w.total_k
    stats = {}
    for name, g, r, n in (("dq", dq, rq, nq), ("dk", dk, rk, nk), ("dv", dv, rv, nk)):
        if n:
            stats[name] = compare_grad(g[:n], r[:n], f"{label} {name}")
    print(f"[{label}] {stats}", flush=True)
    return stats


# ------------------------------------------------------------------ small full-oracle cases

SMALL = {
    # several dK/dV and dQ tiles, ragged tails, Lq != Lk, one-row and one-key segments
    "ragged_d128": (128, 2, [0, 1, 300, 300, 813, 1100], [0, 70, 71, 104, 744, 873]),
    "ragged_d96": (96, 3, [0, 129, 190, 577], [0, 64, 321, 322]),
    "ragged_d64": (64, 2, [0, 255, 256, 700], [0, 300, 301, 450]),
    "self_d128": (128, 1, [0, 640, 1000], None),
}


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_bwd_small_full_oracle(name, causal):
    D, H, cu_q, cu_k = SMALL[name]
    announce(f"bwd {name} causal={causal}")
    w = custom(name, H, D, cu_q, cu_k, std=1.0)
    t = make_inputs(w, "cuda", seed=3)
    dout, _ = make_dout(w, "cuda", seed=4)
    got = backward(t, w, dout, causal)
    check_all(f"{name} causal={causal}", got, oracle_grads(t, w, dout, causal), w)


def test_bwd_empty_segments():
    """Lk = 0 segment: dq = 0; Lq = 0 segment: its keys get dk = dv = 0."""
    announce("bwd empty segments")
    w = custom("empty", 2, 64, [0, 40, 40, 90], [0, 0, 33, 70], std=1.0)
    t = make_inputs(w, "cuda", seed=5)
    dout, _ = make_dout(w, "cuda", seed=6)
    dq, dk, dv, _ = backward(t, w, dout, False)
    assert torch.count_nonzero(dq[0:40]).item() == 0
    assert torch.count_nonzero(dk[0:33]).item() == 0 and torch.count_nonzero(dv[0:33]).item() == 0
    check_all("empty", (dq, dk, dv), oracle_grads(t, w, dout, False), w)


def test_bwd_causal_rows_without_keys():
    """Lq > Lk causal: rows r < Lq - Lk see no key and get dq = 0."""
    announce("bwd causal rows without keys")
    w = custom("nokeys", 2, 128, [0, 300], [0, 100], std=1.0)
    t = make_inputs(w, "cuda", seed=7)
    dout, _ = make_dout(w, "cuda", seed=8)
    dq, dk, dv, _ = backward(t, w, dout, True)
    assert torch.count_nonzero(dq[0:200]).item() == 0
    check_all("nokeys", (dq, dk, dv), oracle_grads(t, w, dout, True), w)


def test_bwd_deterministic_hostcu_and_device_cu():
    announce("bwd determinism / device cu")
    w = custom("det", 2, 96, [0, 500, 777], [0, 260, 777], std=1.0)
    t = make_inputs(w, "cuda", seed=9)
    dout, _ = make_dout(w, "cuda", seed=10)
    a = backward(t, w, dout, False)
    b = backward(t, w, dout, False)
    c = backward(t, w, dout, False, hostcu=False)
    for x, y, z in zip(a[:3], b[:3], c[:3]):
        assert torch.equal(x, y) and torch.equal(x, z)


def test_bwd_strided_dout_equals_contiguous_small():
    """The page's test at small size: dout as a row-stride-9728 view vs its
    contiguous copy gives bitwise identical gradients; both match the oracle."""
    announce("bwd strided dout small")
    w = custom("strided_small", 16, 96, [0, 700, 1300], std=0.1)
    t = make_inputs(w, "cuda", seed=11)
    dout, base = make_dout(w, "cuda", seed=12, outer_stride=9728)
    assert dout.stride() == (9728, 96, 1)
    a = backward(t, w, dout, False)
    b = backward(t, w, dout.contiguous(), False)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    check_all("strided_small", a, oracle_grads(t, w, dout, False), w)


def test_bwd_preprocess_matches_oracle_strided():
    announce("bwd preprocess strided")
    w = custom("pre", 16, 96, [0, 3000], std=0.1)
    o, _ = make_dout(w, "cuda", seed=13, outer_stride=9728)
    g, _ = make_dout(w, "cuda", seed=14, outer_stride=9728)
    delta = avf.bwd_preprocess(o, g)
    torch.cuda.synchronize()
    ref = oracle.bwd_preprocess(o.contiguous().cpu(), g.contiguous().cpu())  # [N, H]
    got = delta.t().cpu().numpy().astype(np.float64)
    assert np.abs(got - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("D", [64, 96, 128])
def test_bwd_output_strides(D):
    """dq/dk/dv written into strided views of larger buffers: values equal the
    contiguous outputs and nothing outside the views changes."""
    announce(f"bwd output strides D={D}")
    w = custom(f"ostr{D}", 3, D, [0, 150, 420], [0, 200, 333], std=1.0)
    t = make_inputs(w, "cuda", seed=15)
    dout, _ = make_dout(w, "cuda", seed=16)
    a = backward(t, w, dout, False)
    H = w.num_heads
    bufs = [torch.full((n, 2 * H * D + 64), -7.0, dtype=torch.bfloat16, device="cuda") for n in (w.total_q, w.total_k, w.total_k)]
    views = [b[:, 64:64 + 2 * H * D].view(b.shape[0], H, 2 * D)[:, :, :D] for b in bufs]
    o, l = forward(t, w, False)
    avf.attn_varlen_bwd(t["q"], t["k"], t["v"], o, dout, l, t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                        softmax_scale=w.softmax_scale, dq=views[0], dk=views[1], dv=views[2],
                        cu_seqlens_q_host=list(w.cu_q), cu_seqlens_k_host=list(w.cu_k))
    torch.cuda.synchronize()
    for x, v_, b in zip(a[:3], views, bufs):
        assert torch.equal(x, v_)
        mask = torch.ones_like(b, dtype=torch.bool)
        mask[:, 64:64 + 2 * H * D].view(b.shape[0], H, 2 * D)[:, :, :D] = False
        assert bool((b[mask] == -7.0).all())


@pytest.mark.parametrize("D,causal", [(64, False), (96, True), (128, False), (128, True)])
def test_bwd_head_major_views_bitwise(D, causal):
    """q, k, v, out, dout and dq/dk/dv all as head-major views ([H, tokens, D]
    buffers seen as [tokens, H, D]: row stride D, head stride tokens * D): the
    gradients equal the token-major ones bit for bit."""
    announce(f"bwd head-major views D={D} causal={causal}")
    cu_q, cu_k = [0, 150, 151, 420], [0, 200, 200, 333]
    wt = custom(f"bt{D}", 3, D, cu_q, cu_k, std=1.0)
    wh = custom(f"bh{D}", 3, D, cu_q, cu_k, std=1.0, layout="head_major")
    tt = make_inputs(wt, "cuda", seed=21)
    th = make_inputs(wh, "cuda", seed=21)
    dout, _ = make_dout(wt, "cuda", seed=22)

    def head_major(x):
        return x.permute(1, 0, 2).contiguous().permute(1, 0, 2)

    a = backward(tt, wt, dout, causal)
    H = wt.num_heads
    outs = [torch.empty((H, n, D), dtype=torch.bfloat16, device="cuda").permute(1, 0, 2)
            for n in (wt.total_q, wt.total_k, wt.total_k)]
    b = backward(th, wh, head_major(dout), causal, dq=outs[0], dk=outs[1], dv=outs[2])
    assert outs[0].stride() == (D, wt.total_q * D, 1)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)


# ------------------------------------------------------------------ the page's full-size case

def test_bwd_full_size_strided_dout():
    """N=410923, H=16, D=96, cu=[0,225304,410923], dout row stride 9728 (the
    _bwd_preprocess page's failing case, 225304 * 9728 > 2^31): gradients
    bitwise equal to those of a contiguous dout, dq on sampled rows against the
    oracle, and the invariants sum_j dk_j = 0 and sum_j dv_j = sum_i dout_i
    per segment and head (they hold at any size)."""
    w = WORKLOADS["bwd_9728"]
    announce("bwd full size bwd_9728")
    t = make_inputs(w, "cuda", seed=0)
    dout, base = make_dout(w, "cuda", seed=1, outer_stride=9728)
    assert 225304 * dout.stride(0) > 2 ** 31
    a = backward(t, w, dout, False)
    b = backward(t, w, dout.contiguous(), False)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    del b
    dq, dk, dv, _ = a
    rows = sample_rows(w, 16, edge=4)
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    ref = oracle.attn_varlen_bwd_dq_rows(q, k, v, dout.contiguous().cpu(), w.cu_q, w.cu_k, f32(w.softmax_scale),
                                         rows)
    compare_grad(dq[rows].float().cpu().numpy(), ref, "bwd_9728 dq rows")
    g64 = dout.double()
    for s in range(w.num_segments):
        ks = slice(w.cu_k[s], w.cu_k[s + 1])
        qs = slice(w.cu_q[s], w.cu_q[s + 1])
        sdk = dk[ks].double().sum(0)          # [H, D], exactly 0 in exact arithmetic
        sdv = dv[ks].double().sum(0)
        sg = g64[qs].sum(0)
        # dv: rounding P to bf16 moves each row's weight sum by at most 2^-9
        # and rounding dv by 2^-9 of |dv|; twice that bound. dk: twice the
        # output rounding (the weight-sum terms cancel up to random rounding).
        tol_k = 2.0 ** -8 * dk[ks].double().abs().sum(0) + 1e-6
        tol_v = 2.0 ** -8 * (dv[ks].double().abs().sum(0) + g64[qs].abs().sum(0)) + 1e-6
        print(f"[bwd_9728] segment {s}: max|sum dk| {sdk.abs().max().item():.3e} "
              f"max|sum dv - sum dout| {(sdv - sg).abs().max().item():.3e}", flush=True)
        assert bool((sdk.abs() <= tol_k).all()), s
        assert bool(((sdv - sg).abs() <= tol_v).all()), s


@pytest.mark.parametrize("split", [220752, 220753])
def test_bwd_stride_threshold_pair_full_gradients(split):
    """The _bwd_preprocess page's threshold ("Verified sample": coord * 9728
    passes 2^31 from row 220753 on) as a pair of calls that differ only in
    cu_seqlens: [0, split, split + 1536] with q, k, v, out, dout and the
    outputs dq, dk, dv all [N, 16, 96] views of [N, 9728] buffers. The second
    segment's rows start at element offset split * 9728, past 2^31 only for
    split = 220753. Segments are independent, so that segment's dq, dk and dv
    are compared in full against the oracle run on it alone; the long first
    segment's gradients must be finite, and the columns of the output buffer
    outside the three views must keep their canary."""
    n2, H, D, R = 1536, 16, 96, 9728
    N = split + n2
    announce(f"bwd stride threshold split={split}")
    torch.cuda.empty_cache()
    w = custom(f"bthresh{split}", H, D, [0, split, N], std=0.1, layout="stride9728", outer_stride=R)
    t = make_inputs(w, "cuda", seed=61)
    dout, _ = make_dout(w, "cuda", seed=62, outer_stride=R)
    assert dout.stride(0) == R and t["q"].stride(0) == R
    assert (split * R >= 2 ** 31) == (split == 220753)
    gbuf = torch.full((N, R), -7.0, dtype=torch.bfloat16, device="cuda")
    hd = H * D
    dq, dk, dv = (gbuf[:, i * hd:(i + 1) * hd].view(N, H, D) for i in range(3))
    got = backward(t, w, dout, False, dq=dq, dk=dk, dv=dv)
    assert got[0].data_ptr() == dq.data_ptr() and got[2].data_ptr() == dv.data_ptr()
    assert bool((gbuf[:, 3 * hd:] == -7.0).all()), "write outside the gradient views"
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(g[:split]).all()), name
    sl = slice(split, N)
    q, k, v = (t[n][sl].contiguous().cpu() for n in ("q", "k", "v"))
    rq, rk, rv = oracle.attn_varlen_bwd(q, k, v, dout[sl].contiguous().cpu(), [0, n2], [0, n2], f32(w.softmax_scale))
    stats = {name: compare_grad(g[sl].float().cpu().numpy(), r, f"split={split} {name}")
             for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv))}
    print(f"[bwd threshold split={split}] second segment {stats}", flush=True)
    del t, dout, gbuf, got
    torch.cuda.empty_cache()


LONG = {
    # one long segment, every element of dq, dk and dv compared
    "self_32768_d128": (128, 4, [0, 32768], [0, 32768], False),
    "cross_causal_24576x40000_d96": (96, 4, [0, 24576], [0, 40000], True),
}


@pytest.mark.parametrize("name", sorted(LONG))
def test_bwd_long_segment_full_gradients(name):
    """A segment of tens of thousands of rows (hundreds of dK/dV and dQ tiles
    along each axis): dq, dk and dv compared element by element against the
    numpy fp64 backward, which takes the same chain rule as the C oracle with
    whole-matrix steps so that it finishes in tens of seconds at this size."""
    D, H, cu_q, cu_k, causal = LONG[name]
    announce(f"bwd long segment {name}")
    w = custom(f"bwd_long_{name}", H, D, cu_q, cu_k, std=0.5)
    t = make_inputs(w, "cuda", seed=71)
    dout, _ = make_dout(w, "cuda", seed=72)
    got = backward(t, w, dout, causal)
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    ref = blas_oracle.attn_varlen_bwd(q, k, v, dout.contiguous().cpu(), w.cu_q, w.cu_k, f32(w.softmax_scale),
                                      causal=causal)
    check_all(name, got, ref, w)


def test_bwd_many_segments_span_launches():
    """200 short segments (some empty): the dK/dV and dQ plans split them over
    launches of 128 segments; gradients match the oracle everywhere."""
    announce("bwd 200 segments")
    rng = np.random.default_rng(41)
    lens_q = [0 if rng.random() < 0.1 else int(rng.integers(1, 90)) for _ in range(200)]
    lens_k = [0 if rng.random() < 0.1 else int(rng.integers(1, 90)) for _ in range(200)]
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(int).tolist()
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(int).tolist()
    w = custom("bwd_many", 2, 64, cu_q, cu_k, std=1.0)
    t = make_inputs(w, "cuda", seed=42)
    dout, _ = make_dout(w, "cuda", seed=43)
    for causal in (False, True):
        got = backward(t, w, dout, causal)
        check_all(f"bwd_many causal={causal}", got, oracle_grads(t, w, dout, causal), w)


def test_bwd_large_head_dim_128():
    """Two 32768-row segments, H=16, D=128 (the dK/dV kernel with AGPR
    accumulators at scale): strided dout gives the same gradients as its
    contiguous copy, dq on sampled rows matches the oracle, and the two
    invariants hold per segment and head."""
    announce("bwd large D=128")
    w = custom("bwd_d128", 16, 128, [0, 32768, 65536], std=0.1)
    t = make_inputs(w, "cuda", seed=51)
    dout, _ = make_dout(w, "cuda", seed=52, outer_stride=3 * 16 * 128 + 64)
    a = backward(t, w, dout, False)
    b = backward(t, w, dout.contiguous(), False)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    dq, dk, dv, _ = a
    rows = sample_rows(w, 12, edge=3)
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    ref = oracle.attn_varlen_bwd_dq_rows(q, k, v, dout.contiguous().cpu(), w.cu_q, w.cu_k, f32(w.softmax_scale), rows)
    compare_grad(dq[rows].float().cpu().numpy(), ref, "bwd_d128 dq rows")
    g64 = dout.double()
    for s in range(w.num_segments):
        ks = slice(w.cu_k[s], w.cu_k[s + 1])
        qs = slice(w.cu_q[s], w.cu_q[s + 1])
        sdk = dk[ks].double().sum(0)
        sdv = dv[ks].double().sum(0)
        tol_k = 2.0 ** -8 * dk[ks].double().abs().sum(0) + 1e-6
        tol_v = 2.0 ** -8 * (dv[ks].double().abs().sum(0) + g64[qs].abs().sum(0)) + 1e-6
        assert bool((sdk.abs() <= tol_k).all()), s
        assert bool(((sdv - g64[qs].sum(0)).abs() <= tol_v).all()), s
