"""GPU tests of the causal option and of the batched dense entry point,
against the CPU oracle (causal reading: query row r of a segment sees keys
j <= r + Lk - Lq). Marked `gpu`; every case prints its name before it touches
the GPU.
"""
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
    return float(np.float32(x))


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    avf.lib()
    yield
    torch.cuda.synchronize()


def run_causal(t, w, hostcu=False):
    kw = dict(cu_seqlens_q_host=list(w.cu_q), cu_seqlens_k_host=list(w.cu_k)) if hostcu else {}
    o, l = avf.attn_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                               softmax_scale=w.softmax_scale, out=t["out"], lse=t["lse"], causal=True, **kw)
    torch.cuda.synchronize()
    return o, l


def gather(o, l, rows, total_q):
    idx = torch.tensor(rows, dtype=torch.long, device=o.device)
    return (o.index_select(0, idx).float().cpu().numpy(),
            l[:, :total_q].index_select(1, idx).t().cpu().numpy())


def oracle_causal(t, w, rows, impl="c"):
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    if impl == "c":
        return oracle.attn_varlen_fwd(q, k, v, w.cu_q, w.cu_k, f32(w.softmax_scale), rows=rows, causal=True)
    return blas_oracle.attn_varlen_fwd(q, k, v, w.cu_q, w.cu_k, f32(w.softmax_scale), rows=rows, causal=True)


# ------------------------------------------------------------------ causal, full oracle

CAUSAL = {
    "square_d128": custom("square_d128", 2, 128, [0, 300, 813], std=1.0, causal=True),
    "lq_lt_lk_d64": custom("lq_lt_lk_d64", 3, 64, [0, 100, 130], [0, 700, 1000], std=1.0, causal=True),
    "lq_gt_lk_d96": custom("lq_gt_lk_d96", 2, 96, [0, 700, 710], [0, 100, 600], std=1.0, causal=True),
    "ragged_d128": custom("ragged_d128", 2, 128, [0, 1, 300, 300, 813, 1100, 1140],
                          [0, 70, 71, 104, 744, 873, 873], std=1.0, causal=True),
    "nine_stages_d64": custom("nine_stages_d64", 2, 64, [0, 1152, 1500], std=1.0, causal=True),
    "nine_stages_d128": custom("nine_stages_d128", 1, 128, [0, 1100, 1152], std=1.0, causal=True),
}


@pytest.mark.parametrize("name", sorted(CAUSAL))
def test_causal_small_full_oracle(name):
    w = CAUSAL[name]
    announce(f"causal full-oracle {name}")
    t = make_inputs(w, DEV, seed=31)
    o, l = run_causal(t, w)
    rows = list(range(w.total_q))
    og, lg = gather(o, l, rows, w.total_q)
    ro, rl = oracle_causal(t, w, rows)
    compare(og, lg, ro, rl, name)


@pytest.mark.parametrize("D", [64, 96, 128])
def test_causal_needles_past_the_diagonal(D):
    """Each row's query is planted, scaled up, as the key just past its causal
    limit (and again as its last visible key): a mask that leaks by one key
    pulls the row to the masked key's value, which the oracle does not."""
    announce(f"causal needles D={D}")
    H, lq, lk = 2, 517, 640
    w = custom(f"needle_causal_{D}", H, D, [0, lq], [0, lk], std=0.3, causal=True)
    t = make_inputs(w, DEV, seed=5)
    q, k = t["q"], t["k"]
    g = torch.Generator(device=DEV).manual_seed(6)
    rows = torch.randperm(lq, generator=g, device=DEV)[:120]
    for r in rows.tolist():
        lim = r + lk - lq  # last visible key
        if lim + 1 < lk:
            k[lim + 1] = (q[r].float() * 8.0).to(torch.bfloat16)
        if r % 3 == 0:
            k[lim] = (q[r].float() * 6.0).to(torch.bfloat16)
    o, l = run_causal(t, w)
    all_rows = list(range(lq))
    og, lg = gather(o, l, all_rows, lq)
    ro, rl = oracle_causal(t, w, all_rows)
    compare(og, lg, ro, rl, f"needle causal D={D}")


def test_causal_rows_without_keys_are_zero():
    announce("causal rows without keys")
    w = custom("nokeys", 2, 128, [0, 900], [0, 300], std=1.0, causal=True)
    t = make_inputs(w, DEV, seed=8)
    o, l = run_causal(t, w)
    dead = 900 - 300  # rows r < Lq - Lk see no key
    assert torch.all(o[:dead] == 0)
    assert torch.all(torch.isneginf(l[:, :dead]))
    assert torch.isfinite(o.float()).all() and torch.isfinite(l[:, dead:900]).all()


def test_causal_strided_equals_contiguous_and_oracle():
    announce("causal strided 9728 view")
    w = custom("causal_strided", 4, 96, [0, 1700, 1701, 3000], std=0.1, layout="stride9728",
               outer_stride=9728, causal=True)
    t = make_inputs(w, DEV, seed=12)
    o, l = run_causal(t, w)
    rows = sample_rows(w, 300, edge=40)
    og, lg = gather(o, l, rows, w.total_q)
    ro, rl = oracle_causal(t, w, rows)
    compare(og, lg, ro, rl, "causal strided")
    # the same inputs as contiguous tensors give bitwise the same result
    tc = {n: t[n] for n in ("cu_q", "cu_k")}
    tc["q"], tc["k"], tc["v"] = (t[n].contiguous() for n in ("q", "k", "v"))
    tc["out"] = torch.empty_like(tc["q"])
    tc["lse"] = torch.empty_like(t["lse"])
    oc, lc = run_causal(tc, w)
    assert torch.equal(oc, o.contiguous()) and torch.equal(lc[:, :w.total_q], l[:, :w.total_q])
    # canaries outside the O slice are untouched
    ob = t["out_base"]
    assert torch.all(ob[:, 4 * 96:] == CANARY)


def test_causal_deterministic_and_hostcu():
    announce("causal determinism / host cu entry")
    w = custom("det", 3, 128, [0, 400, 1000], [0, 500, 1000], std=1.0, causal=True)
    t = make_inputs(w, DEV, seed=4)
    o1, l1 = run_causal(t, w)
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = run_causal(t, w, hostcu=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_causal_full_size_sampled():
    w = WORKLOADS["causal_77k"]
    announce(f"causal full-size sampled {w.name}")
    t = make_inputs(w, DEV, seed=0)
    o, l = run_causal(t, w)
    rows = sample_rows(w, 4096, edge=16)  # seeded rows compared in full (every head)
    og, lg = gather(o, l, rows, w.total_q)
    ro, rl = oracle_causal(t, w, rows, impl="blas")
    compare(og, lg, ro, rl, w.name)
    del t
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ batched dense form

def rand_bf16(shape, seed, std=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV, dtype=torch.float32) * std).to(torch.bfloat16)


def oracle_batched(q, k, v, causal, scale, rows_per_batch=None):
    """Oracle on the batched tensors flattened to W uniform segments."""
    W, Sq, H, D = q.shape
    Sk = k.shape[1]
    qf = q.contiguous().reshape(W * Sq, H, D).cpu()
    kf = k.contiguous().reshape(W * Sk, H, D).cpu()
    vf = v.contiguous().reshape(W * Sk, H, D).cpu()
    cu_q = [b * Sq for b in range(W + 1)]
    cu_k = [b * Sk for b in range(W + 1)]
    rows = None
    if rows_per_batch is not None:
        rows = [b * Sq + r for b in range(W) for r in rows_per_batch]
    o, l = oracle.attn_varlen_fwd(qf, kf, vf, cu_q, cu_k, f32(scale), rows=rows, causal=causal)
    return o, l, rows


@pytest.mark.parametrize("causal", [False, True])
def test_batched_equals_varlen_bitwise(causal):
    announce(f"batched == varlen (causal={causal})")
    W, S, H, D = 3, 400, 4, 128
    q, k, v = (rand_bf16((W, S, H, D), seed=s) for s in (1, 2, 3))
    o, l = avf.attn_fwd(q, k, v, causal=causal)
    cu = torch.tensor([b * S for b in range(W + 1)], dtype=torch.int32, device=DEV)
    ov, lv = avf.attn_varlen_fwd(q.reshape(W * S, H, D), k.reshape(W * S, H, D), v.reshape(W * S, H, D), cu, cu,
                                 S, S, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.reshape(W * S, H, D), ov)
    assert torch.equal(l.permute(1, 0, 2).reshape(H, W * S), lv)
    oo, ol, _ = oracle_batched(q, k, v, causal, 1 / 128 ** 0.5)
    compare(o.reshape(W * S, H, D).float().cpu().numpy(), l.permute(1, 0, 2).reshape(H, W * S).t().cpu().numpy(),
            oo, ol, f"batched causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_batched_strided_layouts(causal):
    """q/k/v stored [S, W, H, D] and viewed as [W, S, H, D] (batch stride H*D,
    row stride W*H*D); out written into a padded buffer whose extra rows and
    heads keep their canary; lse into a padded [W, H, S+5] buffer."""
    announce(f"batched strided layouts (causal={causal})")
    W, Sq, Sk, H, D = 5, 230, 300, 3, 96
    q = rand_bf16((Sq, W, H, D), seed=11).permute(1, 0, 2, 3)
    k = rand_bf16((Sk, W, H, D), seed=12).permute(1, 0, 2, 3)
    v = rand_bf16((Sk, W, H, D), seed=13).permute(1, 0, 2, 3)
    ob = torch.full((W, Sq + 7, H + 1, D), CANARY, dtype=torch.bfloat16, device=DEV)
    out = ob[:, 3:3 + Sq, 1:, :]
    lb = torch.full((W, H, Sq + 5), CANARY, dtype=torch.float32, device=DEV)
    lse = lb[:, :, 2:2 + Sq]
    o, l = avf.attn_fwd(q, k, v, causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    mask = torch.ones_like(ob, dtype=torch.bool)
    mask[:, 3:3 + Sq, 1:, :] = False
    assert torch.all(ob[mask] == CANARY)
    lmask = torch.ones_like(lb, dtype=torch.bool)
    lmask[:, :, 2:2 + Sq] = False
    assert torch.all(lb[lmask] == CANARY)
    oo, ol, _ = oracle_batched(q, k, v, causal, 1 / 96 ** 0.5)
    compare(o.contiguous().reshape(W * Sq, H, D).float().cpu().numpy(),
            l.permute(1, 0, 2).reshape(H, W * Sq).t().cpu().numpy(), oo, ol, f"batched strided causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_batched_sdpa_layout_views(causal):
    """q, k, v and out stored [W, H, S, D] (the layout of torch's
    scaled_dot_product_attention) and passed as [W, S, H, D] views: the same
    results, bit for bit, as contiguous [W, S, H, D] copies."""
    announce(f"batched [W, H, S, D] storage (causal={causal})")
    W, Sq, Sk, H, D = 3, 300, 520, 4, 128
    q = rand_bf16((W, H, Sq, D), seed=41).transpose(1, 2)
    k = rand_bf16((W, H, Sk, D), seed=42).transpose(1, 2)
    v = rand_bf16((W, H, Sk, D), seed=43).transpose(1, 2)
    out = torch.empty((W, H, Sq, D), dtype=torch.bfloat16, device=DEV).transpose(1, 2)
    o, l = avf.attn_fwd(q, k, v, causal=causal, out=out)
    oc, lc = avf.attn_fwd(q.contiguous(), k.contiguous(), v.contiguous(), causal=causal)
    torch.cuda.synchronize()
    assert o.stride() == (H * Sq * D, D, Sq * D, 1)
    assert torch.equal(o, oc) and torch.equal(l, lc)


def test_batched_many_batches_span_launches():
    """More batches than segments per launch: later launches must address
    their batches from the right base."""
    n = avf.segments_per_launch() + 22
    announce(f"batched W={n} over several launches")
    W, S, H, D = n, 20, 2, 64
    q, k, v = (rand_bf16((W, S, H, D), seed=s, std=1.0) for s in (21, 22, 23))
    o, l = avf.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    oo, ol, _ = oracle_batched(q, k, v, True, 1 / 8.0)
    compare(o.reshape(W * S, H, D).float().cpu().numpy(), l.permute(1, 0, 2).reshape(H, W * S).t().cpu().numpy(),
            oo, ol, "batched many")
