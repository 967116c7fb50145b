"""GPU parity and structure tests of the HIP path (through the C ABI via the
ctypes binding) against the CPU oracle. Marked `gpu`; every case prints its
name before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import blas_oracle
import varlen_flashattention_forward_amd as avf
from varlen_flashattention_forward_amd.workloads import CANARY, WORKLOADS, custom, make_inputs, sample_rows

from parity import compare

pytestmark = pytest.mark.gpu

DEV = "cuda"


def announce(label):
    print(f"\n[gpu-case] {label}", flush=True)


def f32(x):
    """The fp32 value the library receives, widened for the oracle."""
    return float(np.float32(x))


def run_gpu(t, w, hostcu=False, out=None, lse=None):
    kw = {}
    if hostcu:
        kw = dict(cu_seqlens_q_host=list(w.cu_q), cu_seqlens_k_host=list(w.cu_k))
    o, l = avf.attn_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                               softmax_scale=w.softmax_scale, out=t["out"] if out is None else out,
                               lse=t["lse"] if lse is None else lse, **kw)
    torch.cuda.synchronize()
    return o, l


def gather(o, l, rows, total_q):
    idx = torch.tensor(rows, dtype=torch.long, device=o.device)
    og = o.index_select(0, idx).float().cpu().numpy()
    lg = l[:, :total_q].index_select(1, idx).t().cpu().numpy()
    return og, lg


def oracle_rows(t, w, rows, impl="c"):
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    if impl == "c":
        return oracle.attn_varlen_fwd(q, k, v, w.cu_q, w.cu_k, f32(w.softmax_scale), rows=rows)
    return blas_oracle.attn_varlen_fwd(q, k, v, w.cu_q, w.cu_k, f32(w.softmax_scale), rows=rows)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    avf.lib()  # raises if the HIP library is missing: no fallback path exists
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ small cases, full oracle

SMALL = {
    "dense_256": WORKLOADS["dense_256"],
    "ragged_d64": custom("ragged_d64", 3, 64, [0, 1, 300, 300, 813, 1100, 1140],
                         [0, 70, 71, 104, 744, 873, 873], std=1.0),
    "ragged_d96": custom("ragged_d96", 3, 96, [0, 1, 300, 300, 813, 1100, 1140],
                         [0, 70, 71, 104, 744, 873, 873], std=1.0),
    "ragged_d128": custom("ragged_d128", 3, 128, [0, 1, 300, 300, 813, 1100, 1140],
                          [0, 70, 71, 104, 744, 873, 873], std=1.0),
    "cross_long_k": custom("cross_long_k", 2, 128, [0, 5, 705], [0, 2000, 2130], std=0.5),
    "self_tiles_d96": custom("self_tiles_d96", 4, 96, [0, 256, 257, 769], std=0.1),
}
# Key lengths from one stage of 128 keys to nine, each stage count with and
# without a ragged tail: every position of the K (2) and V (3) buffer rings,
# and the first and last stages, meet in some segment.
_RING_LK = [1, 31, 128, 129, 255, 256, 300, 384, 400, 512, 513, 640, 700, 768, 896, 1000, 1024, 1152]
for _d in (64, 96, 128):
    _ck = np.concatenate([[0], np.cumsum(_RING_LK)]).tolist()
    _cq = [37 * i for i in range(len(_RING_LK) + 1)]
    SMALL[f"ring_stages_d{_d}"] = custom(f"ring_stages_d{_d}", 2, _d, _cq, _ck, std=1.0)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_full_oracle(name):
    w = SMALL[name]
    announce(f"small full-oracle {name}")
    t = make_inputs(w, DEV, seed=11)
    o, l = run_gpu(t, w)
    rows = list(range(w.total_q))
    og, lg = gather(o, l, rows, w.total_q)
    ro, rl = oracle_rows(t, w, rows)
    compare(og, lg, ro, rl, name)


def test_many_segments_multiple_launches():
    rng = np.random.default_rng(3)
    n = 2 * avf.segments_per_launch() + 37
    lq = rng.integers(0, 40, n)
    lk = rng.integers(0, 90, n)
    cq = np.concatenate([[0], np.cumsum(lq)]).tolist()
    ck = np.concatenate([[0], np.cumsum(lk)]).tolist()
    w = custom("many_segments", 2, 64, cq, ck, std=1.0)
    launches, _ = avf.grid_plan(w.cu_q, w.num_heads, w.head_dim, w.max_seqlen_k)
    assert launches >= 3
    announce(f"many segments B={n} launches={launches}")
    t = make_inputs(w, DEV, seed=5)
    o, l = run_gpu(t, w)
    rows = list(range(w.total_q))
    og, lg = gather(o, l, rows, w.total_q)
    ro, rl = oracle_rows(t, w, rows)
    compare(og, lg, ro, rl, "many_segments")


# ------------------------------------------------------------------ structure (bitwise)

def strided_small():
    return custom("strided_small", 4, 96, [0, 1700, 1701, 3000], std=0.1, layout="stride9728",
                  outer_stride=9728)


def test_strided_equals_contiguous_bitwise_and_canaries():
    w = strided_small()
    announce("strided vs contiguous, canaries")
    t = make_inputs(w, DEV, seed=2, lse_head_pad=7)
    o, l = run_gpu(t, w)
    # every element of the [N, 9728] output buffer outside the O slice keeps the canary
    hd = w.num_heads * w.head_dim
    rest = t["out_base"][:, hd:]
    assert bool((rest == CANARY).all())
    assert bool((t["lse"][:, w.total_q:] == CANARY).all())
    tc = dict(t)
    tc.update(q=t["q"].contiguous(), k=t["k"].contiguous(), v=t["v"].contiguous(),
              out=torch.full_like(t["q"].contiguous(), CANARY), lse=torch.full_like(t["lse"], CANARY))
    oc, lc = run_gpu(tc, w)
    assert torch.equal(o, oc)
    assert torch.equal(l[:, :w.total_q], lc[:, :w.total_q])
    rows = sample_rows(w, 64, edge=16)
    og, lg = gather(o, l, rows, w.total_q)
    ro, rl = oracle_rows(t, w, rows)
    compare(og, lg, ro, rl, "strided_small")


# key lengths that select each configuration: one 128-key stage, 64-key stages, general
HEAD_MAJOR_CASES = [(64, [0, 77, 77, 300, 301], [0, 128, 129, 200, 256], False),
                    (128, [0, 500, 520, 900], [0, 400, 912, 1024], True),
                    (96, [0, 640, 641, 1400], [0, 700, 1300, 1301], False),
                    (128, [0, 1000, 1030], [0, 1500, 1700], True)]


@pytest.mark.parametrize("D,cu_q,cu_k,causal", HEAD_MAJOR_CASES)
def test_head_major_views_equal_token_major_bitwise(D, cu_q, cu_k, causal):
    """The same values stored head by head ([H, tokens, D] buffers seen as
    [tokens, H, D] views: row stride D, head stride tokens * D) give the
    token-major results bit for bit, and match the oracle."""
    H = 3
    wt = custom(f"token_d{D}", H, D, cu_q, cu_k, std=1.0, causal=causal)
    wh = custom(f"head_d{D}", H, D, cu_q, cu_k, std=1.0, layout="head_major", causal=causal)
    announce(f"head-major vs token-major D={D} causal={causal} max_k={wt.max_seqlen_k}")
    tt = make_inputs(wt, DEV, seed=9)
    th = make_inputs(wh, DEV, seed=9)
    assert th["q"].stride() == (D, wh.total_q * D, 1) and torch.equal(th["q"], tt["q"])
    kw = dict(softmax_scale=wt.softmax_scale, causal=causal)
    ot, lt = avf.attn_varlen_fwd(tt["q"], tt["k"], tt["v"], tt["cu_q"], tt["cu_k"], wt.max_seqlen_q,
                                 wt.max_seqlen_k, out=tt["out"], lse=tt["lse"], **kw)
    oh, lh = avf.attn_varlen_fwd(th["q"], th["k"], th["v"], th["cu_q"], th["cu_k"], wh.max_seqlen_q,
                                 wh.max_seqlen_k, out=th["out"], lse=th["lse"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(ot, oh) and torch.equal(lt, lh)
    rows = list(range(wt.total_q))
    og, lg = gather(ot, lt, rows, wt.total_q)
    q, k, v = (tt[n].contiguous().cpu() for n in ("q", "k", "v"))
    ro, rl = oracle.attn_varlen_fwd(q, k, v, wt.cu_q, wt.cu_k, f32(wt.softmax_scale), rows=rows, causal=causal)
    compare(og, lg, ro, rl, wh.name)


def test_deterministic_and_hostcu_bitwise():
    w = SMALL["ragged_d128"]
    announce("determinism + host cu_seqlens entry")
    t = make_inputs(w, DEV, seed=4)
    o1, l1 = run_gpu(t, w)
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = run_gpu(t, w)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = run_gpu(t, w, hostcu=True)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_segment_independence_bitwise():
    w = custom("indep", 2, 128, [0, 300, 301, 900], [0, 500, 700, 1230], std=1.0)
    announce("segment independence")
    t = make_inputs(w, DEV, seed=8)
    o, l = run_gpu(t, w)
    for b in range(w.num_segments):
        qs, qe, ks, ke = w.cu_q[b], w.cu_q[b + 1], w.cu_k[b], w.cu_k[b + 1]
        wb = custom(f"seg{b}", 2, 128, [0, qe - qs], [0, ke - ks])
        tb = {"q": t["q"][qs:qe].contiguous(), "k": t["k"][ks:ke].contiguous(), "v": t["v"][ks:ke].contiguous(),
              "cu_q": torch.tensor(wb.cu_q, dtype=torch.int32, device=DEV),
              "cu_k": torch.tensor(wb.cu_k, dtype=torch.int32, device=DEV),
              "out": torch.empty((qe - qs, 2, 128), dtype=torch.bfloat16, device=DEV),
              "lse": torch.empty((2, qe - qs), dtype=torch.float32, device=DEV)}
        ob, lb = run_gpu(tb, wb)
        assert torch.equal(ob, o[qs:qe]), f"segment {b} differs when run alone"
        assert torch.equal(lb, l[:, qs:qe])


def test_sentinel_padded_cu_is_identical():
    """Appending a duplicate last cu entry (an empty segment) changes nothing."""
    w = SMALL["ragged_d64"]
    announce("sentinel-padded cu_seqlens")
    t = make_inputs(w, DEV, seed=6)
    o, l = run_gpu(t, w)
    o, l = o.clone(), l.clone()
    wp = custom("padded", w.num_heads, w.head_dim, list(w.cu_q) + [w.cu_q[-1]], list(w.cu_k) + [w.cu_k[-1]], std=1.0)
    tp = dict(t)
    tp.update(cu_q=torch.tensor(wp.cu_q, dtype=torch.int32, device=DEV),
              cu_k=torch.tensor(wp.cu_k, dtype=torch.int32, device=DEV),
              out=torch.full_like(o, CANARY), lse=torch.full_like(l, CANARY))
    op, lp = run_gpu(tp, wp)
    assert torch.equal(o, op) and torch.equal(l, lp)


@pytest.mark.parametrize("D", [64, 96, 128])
def test_needles_at_tile_edges(D):
    """One-hot attention: query row i is a large multiple of key t_i, so O[i] = V[t_i].
    Targets sit on the first/last key of each segment, 31/32 and 63/64 (MFMA and
    K/V tile boundaries) and in the K tail tile."""
    H = 2
    lk = [130, 64, 1, 97]
    lq = [12, 6, 2, 300]
    cq = np.concatenate([[0], np.cumsum(lq)]).tolist()
    ck = np.concatenate([[0], np.cumsum(lk)]).tolist()
    w = custom(f"needle_d{D}", H, D, cq, ck)
    announce(f"needles D={D}")
    g = torch.Generator(device=DEV).manual_seed(1)
    k = (torch.randint(0, 2, (w.total_k, H, D), generator=g, device=DEV) * 2 - 1).to(torch.bfloat16)
    v = torch.randn((w.total_k, H, D), generator=g, device=DEV).to(torch.bfloat16)
    q = torch.zeros((w.total_q, H, D), dtype=torch.bfloat16, device=DEV)
    target = []
    for b in range(w.num_segments):
        cands = sorted({0, lk[b] - 1, min(31, lk[b] - 1), min(32, lk[b] - 1), min(63, lk[b] - 1),
                        min(64, lk[b] - 1), lk[b] - 2 if lk[b] > 1 else 0, min(96, lk[b] - 1)})
        for i in range(lq[b]):
            tk = cands[i % len(cands)]
            q[cq[b] + i] = k[ck[b] + tk] * 8.0
            target.append(ck[b] + tk)
    t = {"q": q, "k": k, "v": v, "cu_q": torch.tensor(cq, dtype=torch.int32, device=DEV),
         "cu_k": torch.tensor(ck, dtype=torch.int32, device=DEV),
         "out": torch.full((w.total_q, H, D), CANARY, dtype=torch.bfloat16, device=DEV),
         "lse": torch.full((H, w.total_q), CANARY, dtype=torch.float32, device=DEV)}
    o, l = run_gpu(t, w)
    expect = v[torch.tensor(target, device=DEV)].float()
    err = (o.float() - expect).abs().max().item()
    assert err <= 2e-2, err
    lse_expect = 8.0 * D * f32(w.softmax_scale)
    assert torch.allclose(l, torch.full_like(l, lse_expect), atol=1e-3, rtol=1e-6)


def test_empty_and_keyless_segments():
    w = custom("empty_mix", 2, 64, [0, 0, 5, 5, 70, 70], [0, 9, 9, 40, 40, 41], std=1.0)
    announce("empty and key-less segments")
    t = make_inputs(w, DEV, seed=9)
    o, l = run_gpu(t, w)
    assert bool((o[0:5] == 0).all())
    assert bool(torch.isneginf(l[:, 0:5]).all())
    rows = list(range(w.total_q))
    og, lg = gather(o, l, rows, w.total_q)
    ro, rl = oracle_rows(t, w, rows)
    compare(og, lg, ro, rl, "empty_mix")


def test_zero_tokens_is_a_no_op():
    w = custom("zero", 2, 64, [0, 0], [0, 5])
    announce("zero query tokens")
    t = make_inputs(w, DEV)
    run_gpu(t, w)


def test_bad_device_cu_is_rejected_without_writing():
    w = custom("bad", 2, 64, [0, 10], [0, 12])
    announce("bad device cu_seqlens")
    t = make_inputs(w, DEV)
    bad = torch.tensor([0, 11], dtype=torch.int32, device=DEV)   # past q_tokens
    with pytest.raises(avf.AttnVarlenError) as ei:
        avf.attn_varlen_fwd(t["q"], t["k"], t["v"], bad, t["cu_k"], 11, 12, out=t["out"], lse=t["lse"])
    assert ei.value.code == -5
    torch.cuda.synchronize()
    assert bool((t["out"] == CANARY).all())


# ------------------------------------------------------------------ full-size workloads (sampled rows)

FULL = ["varlen_cross", "dense_77k", "strided_9728", "dense_117k", "shard_heads_117k", "shard_rows_117k"]
# seeded query rows per segment compared in full (every head, every column) at
# the full sizes: a segment with fewer rows is compared whole
FULL_SAMPLE = 4096


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    w = WORKLOADS[name]
    announce(f"full-size {name}")
    torch.cuda.empty_cache()
    t = make_inputs(w, DEV, seed=0)
    o, l = run_gpu(t, w)
    if w.layout == "stride9728":
        hd = w.num_heads * w.head_dim
        assert bool((t["out_base"][:, hd:] == CANARY).all()), "write outside the O slice"
    rows = sample_rows(w, FULL_SAMPLE, edge=16)
    og, lg = gather(o, l, rows, w.total_q)
    ro, rl = oracle_rows(t, w, rows, impl="blas")
    stats = compare(og, lg, ro, rl, name)
    print(f"[gpu-case] {name} {stats}", flush=True)
    del t, o, l
    torch.cuda.empty_cache()


def test_stride_threshold_pair():
    """cu boundary at 220752 vs 220753 rows with row stride 9728: the second
    segment's base crosses 2^31 elements only in the second case."""
    n = 221000
    for split in (220752, 220753):
        w = custom(f"thresh{split}", 16, 96, [0, split, n], std=0.1, layout="stride9728", outer_stride=9728)
        announce(f"stride threshold split={split}")
        t = make_inputs(w, DEV, seed=3)
        o, l = run_gpu(t, w)
        rows = [0, 1, split - 1, split, split + 1, n - 1] + list(range(split + 2, n, 29))
        og, lg = gather(o, l, rows, w.total_q)
        ro, rl = oracle_rows(t, w, rows, impl="blas")
        compare(og, lg, ro, rl, w.name)
        del t, o, l
        torch.cuda.empty_cache()


# The SM120 page's synthetic grid ("What rules things out": W windows x S
# tokens at H = 8 and 56, varlen and batched-dense calls): its corners, with
# the batched form equal to the varlen one bit for bit and sampled rows
# against the oracle.
W_BY_S = [(1, 1024, 8), (16, 1024, 56), (4, 4096, 56), (8, 24576, 8), (16, 4096, 8)]


@pytest.mark.parametrize("W,S,H", W_BY_S)
def test_pages_w_by_s_grid(W, S, H):
    D = 128
    announce(f"W x S grid W={W} S={S} H={H}")
    torch.cuda.empty_cache()
    w = custom(f"grid_{W}x{S}x{H}", H, D, [b * S for b in range(W + 1)], std=1.0)
    t = make_inputs(w, DEV, seed=W + S + H)
    o, l = run_gpu(t, w)
    qb, kb, vb = (t[n].view(W, S, H, D) for n in ("q", "k", "v"))
    ob, lb = avf.attn_fwd(qb, kb, vb)
    torch.cuda.synchronize()
    assert torch.equal(ob.reshape(W * S, H, D), o)
    assert torch.equal(lb.permute(1, 0, 2).reshape(H, W * S), l[:, :W * S])
    rows = sample_rows(w, 4, edge=1)
    og, lg = gather(o, l, rows, w.total_q)
    ro, rl = oracle_rows(t, w, rows, impl="blas")
    compare(og, lg, ro, rl, w.name)
    del t, o, l, ob, lb
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ softmax reference moves

def _run_custom(q, k, v, cq, ck, label):
    H, D = q.shape[1], q.shape[2]
    w = custom(label, H, D, cq, ck)
    t = {"q": q.to(DEV), "k": k.to(DEV), "v": v.to(DEV),
         "cu_q": torch.tensor(cq, dtype=torch.int32, device=DEV),
         "cu_k": torch.tensor(ck, dtype=torch.int32, device=DEV),
         "out": torch.full((w.total_q, H, D), CANARY, dtype=torch.bfloat16, device=DEV),
         "lse": torch.full((H, w.total_q), CANARY, dtype=torch.float32, device=DEV)}
    o, l = run_gpu(t, w)
    rows = list(range(w.total_q))
    og, lg = gather(o, l, rows, w.total_q)
    ro, rl = oracle.attn_varlen_fwd(q, k, v, cq, ck, f32(w.softmax_scale), rows=rows)
    return compare(og, lg, ro, rl, label)


@pytest.mark.parametrize("D", [64, 96, 128])
def test_reference_moves_with_growing_logits(D):
    """Logits rise along the keys by ~70 base-2 units, so the softmax reference
    has to move several times inside segments (also while the next 32-key
    block's scores are already formed); a second segment falls instead."""
    announce(f"growing logits D={D}")
    g = torch.Generator().manual_seed(D)
    H, L, nq = 2, 700, 300
    scale = 1.0 / math.sqrt(D)
    c = scale * 1.4426950408889634
    a = 8.0
    k = torch.randn((2 * L, H, D), generator=g) * 0.3
    ramp = torch.linspace(0.0, 70.0 / (c * a), L)
    k[:L, :, 0] = ramp[:, None]
    k[L:, :, 0] = ramp.flip(0)[:, None]
    q = torch.randn((2 * nq, H, D), generator=g) * 0.3
    q[:, :, 0] = a
    v = torch.randn((2 * L, H, D), generator=g)
    _run_custom(q.bfloat16(), k.bfloat16(), v.bfloat16(), [0, nq, 2 * nq], [0, L, 2 * L], f"growing_d{D}")


def test_reference_from_first_block_when_all_logits_negative():
    """Every logit is about -130 (base-2 units): the reference must be taken
    from the data, or every weight would underflow to zero."""
    announce("all-negative logits")
    g = torch.Generator().manual_seed(1)
    H, D, L, nq = 2, 128, 333, 77
    u = torch.randn((H, D), generator=g)
    u = u / u.norm(dim=-1, keepdim=True) * 32.0   # q.k ~ -1024, c*s ~ -130
    k = u[None].repeat(L, 1, 1) + torch.randn((L, H, D), generator=g) * 0.05
    q = -u[None].repeat(nq, 1, 1) + torch.randn((nq, H, D), generator=g) * 0.05
    v = torch.randn((L, H, D), generator=g)
    _run_custom(q.bfloat16(), k.bfloat16(), v.bfloat16(), [0, nq], [0, L], "all_negative")
