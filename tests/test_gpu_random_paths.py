"""Seeded random sweeps of the other entry points through the C ABI:
- the backward, with full gradients against the oracle's fp64 gradients;
- the 8-bit score product, with sampled rows against the quantized oracle;
- the sync-free forward, on sampled rows against the oracle and bitwise
  against the host-planned forward.
Cases draw random segment tables with empty segments, head counts, head_dims,
the causal mask, and for the forward entries a loose or exact max_seqlen_k
(so every configuration is hit). Marked `gpu`; every case prints its
parameters before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_oracle
import varlen_flashattention_forward_amd as avf
from varlen_flashattention_forward_amd.workloads import CANARY, custom, make_inputs, sample_rows

from parity import compare, compare_grad

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    avf.lib()
    yield
    torch.cuda.synchronize()


def f32(x):
    return float(np.float32(x))


def random_segments(rng, B, max_q, max_k, empty=0.12):
    lq = [0 if rng.random() < empty else int(rng.integers(1, max_q + 1)) for _ in range(B)]
    lk = [0 if rng.random() < empty else int(rng.integers(1, max_k + 1)) for _ in range(B)]
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(int).tolist()
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(int).tolist()
    return cq, ck


@pytest.mark.parametrize("seed", range(10))
def test_random_backward(seed):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 96, 128]))
    H = int(rng.integers(1, 4))
    causal = bool(rng.random() < 0.5)
    cq, ck = random_segments(rng, int(rng.integers(1, 8)), 300, 400)
    if cq[-1] == 0 or ck[-1] == 0:
        cq[-1], ck[-1] = cq[-1] + 1, ck[-1] + 1  # at least one query row and one key
    w = custom(f"rbwd{seed}", H, D, cq, ck, std=1.0)
    print(f"\n[gpu-case] random backward seed={seed} D={D} H={H} B={len(cq) - 1} causal={causal} "
          f"total_q={w.total_q} total_k={w.total_k}", flush=True)
    t = make_inputs(w, DEV, seed=seed)
    g = torch.Generator(device=DEV).manual_seed(seed)
    dout = torch.randn((w.total_q, H, D), generator=g, device=DEV).to(torch.bfloat16)
    o, l = avf.attn_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                               out=t["out"], lse=t["lse"], causal=causal)
    dq, dk, dv, _ = avf.attn_varlen_bwd(t["q"], t["k"], t["v"], o, dout, l, t["cu_q"], t["cu_k"], w.max_seqlen_q,
                                        w.max_seqlen_k, causal=causal)
    torch.cuda.synchronize()
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    rq, rk, rv = oracle.attn_varlen_bwd(q, k, v, dout.cpu(), w.cu_q, w.cu_k, f32(w.softmax_scale), causal=causal)
    for name, got, ref, n in (("dq", dq, rq, w.total_q), ("dk", dk, rk, w.total_k), ("dv", dv, rv, w.total_k)):
        compare_grad(got.float().cpu().numpy()[:n], ref[:n], f"{w.name} {name}")


@pytest.mark.parametrize("seed", range(8))
def test_random_fp8(seed):
    rng = np.random.default_rng(2000 + seed)
    D = int(rng.choice([64, 128]))
    H = int(rng.integers(1, 5))
    causal = bool(rng.random() < 0.4)
    cq, ck = random_segments(rng, int(rng.integers(1, 20)), 600, 900)
    if cq[-1] == 0 or ck[-1] == 0:
        cq[-1], ck[-1] = cq[-1] + 1, ck[-1] + 1  # at least one query row and one key
    w = custom(f"rfp8_{seed}", H, D, cq, ck, std=1.0, causal=causal)
    print(f"\n[gpu-case] random fp8 seed={seed} D={D} H={H} B={len(cq) - 1} causal={causal}", flush=True)
    t = make_inputs(w, DEV, seed=seed)
    o, l, _ = avf.attn_varlen_fwd_fp8(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q,
                                      max(w.max_seqlen_k, 1), out=t["out"], lse=t["lse"], causal=causal)
    torch.cuda.synchronize()
    rows = sample_rows(w, 10, seed=seed, edge=2)
    idx = torch.tensor(rows, dtype=torch.long, device=DEV)
    og = o.index_select(0, idx).float().cpu().numpy()
    lg = l[:, :w.total_q].index_select(1, idx).t().cpu().numpy()
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    ro, rl = fp8_oracle.attn_varlen_fwd_fp8(q, k, v, w.cu_q, w.cu_k, f32(w.softmax_scale), rows=rows, causal=causal)
    compare(og, lg, ro, rl, w.name)


@pytest.mark.parametrize("seed", range(8))
def test_random_sync_free_bitwise(seed):
    rng = np.random.default_rng(3000 + seed)
    D = int(rng.choice([64, 96, 128]))
    H = int(rng.integers(1, 5))
    causal = bool(rng.random() < 0.4)
    kmax = (128, 512, 2000)[seed % 3]
    cq, ck = random_segments(rng, int(rng.integers(1, 200)), 400, kmax)
    if cq[-1] == 0 or ck[-1] == 0:
        cq[-1], ck[-1] = cq[-1] + 1, ck[-1] + 1  # at least one query row and one key
    max_q = max(b - a for a, b in zip(cq[:-1], cq[1:]))
    max_k = max(b - a for a, b in zip(ck[:-1], ck[1:])) + int(rng.choice([0, 0, 100]))
    w = custom(f"rasync{seed}", H, D, cq, ck, std=1.0)
    print(f"\n[gpu-case] random sync-free seed={seed} D={D} H={H} B={len(cq) - 1} max_k={max_k} causal={causal}",
          flush=True)
    t = make_inputs(w, DEV, seed=seed)
    a_o = torch.full_like(t["out"], CANARY)
    a_l = torch.full_like(t["lse"], CANARY)
    avf.attn_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], max_q, max_k, out=a_o, lse=a_l, causal=causal,
                        cu_seqlens_q_host=cq, cu_seqlens_k_host=ck)
    b_o = torch.full_like(t["out"], CANARY)
    b_l = torch.full_like(t["lse"], CANARY)
    _, _, ws = avf.attn_varlen_fwd_async(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], max_q, max_k, out=b_o,
                                         lse=b_l, causal=causal)
    torch.cuda.synchronize()
    assert avf.async_status(ws) == 0
    rows = sample_rows(w, 64, seed=seed, edge=8)
    idx = torch.tensor(rows, dtype=torch.long, device=DEV)
    og = b_o.index_select(0, idx).float().cpu().numpy()
    lg = b_l[:, :w.total_q].index_select(1, idx).t().cpu().numpy()
    q, k, v = (t[n].cpu() for n in ("q", "k", "v"))
    ro, rl = oracle.attn_varlen_fwd(q, k, v, w.cu_q, w.cu_k, f32(w.softmax_scale), rows=rows, causal=causal)
    compare(og, lg, ro, rl, w.name)
    assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l)
