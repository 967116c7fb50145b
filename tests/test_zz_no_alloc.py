"""The no-allocation sync-free forward (attn_varlen_fwd_async_noalloc, plan in
the library's static device array) through the C ABI: each call's output
equals the workspace sync-free entry's bit for bit and matches the oracle at
the parity bar, over two calls in a row where the second is smaller (the
static plan keeps the first call's words); bad cu values are reported
through the static plan's status with the outputs untouched, and a segment
count over the static plan's limit is refused before any launch. Marked
`gpu`; every case prints its name before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import varlen_flashattention_forward_amd as avf
from varlen_flashattention_forward_amd import _binding
from varlen_flashattention_forward_amd.workloads import CANARY, custom, make_inputs

from parity import compare

pytestmark = pytest.mark.gpu


def announce(label):
    print(f"\n[gpu-case] {label}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    avf.lib()
    yield
    torch.cuda.synchronize()


def both(t, w, causal):
    """(workspace entry outputs, no-allocation entry outputs, plan address)."""
    a_o, a_l = torch.full_like(t["out"], CANARY), torch.full_like(t["lse"], CANARY)
    b_o, b_l = torch.full_like(t["out"], CANARY), torch.full_like(t["lse"], CANARY)
    _, _, ws = avf.attn_varlen_fwd_async(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q,
                                         w.max_seqlen_k, softmax_scale=w.softmax_scale, out=a_o, lse=a_l,
                                         causal=causal)
    _, _, plan = avf.attn_varlen_fwd_async_noalloc(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q,
                                                   w.max_seqlen_k, softmax_scale=w.softmax_scale, out=b_o, lse=b_l,
                                                   causal=causal)
    torch.cuda.synchronize()
    assert avf.async_status(ws) == 0
    assert plan is not None and avf.async_status(plan) == 0
    return (a_o, a_l), (b_o, b_l), plan


def check(t, w, causal, o, l, label):
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    ro, rl = oracle.attn_varlen_fwd(q, k, v, w.cu_q, w.cu_k, float(np.float32(w.softmax_scale)), causal=causal)
    stats = compare(o.float().cpu().numpy(), l[:, :w.total_q].t().cpu().numpy(), ro, rl, label)
    print(f"[gpu-case] {label} {stats}", flush=True)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_no_alloc_two_calls_second_smaller(causal):
    cases = [
        # first call: 40 segments over four configurations' worth of lengths, D = 128
        ("large", 4, 128, np.random.default_rng(11)),
        # second call: fewer segments, other head_dim and head count
        ("small", 2, 96, np.random.default_rng(12)),
    ]
    plans = []
    for i, (name, H, D, rng) in enumerate(cases):
        B = 40 if i == 0 else 5
        lq = [int(x) for x in rng.integers(0, 700 if i == 0 else 200, B)]
        lk = [int(x) for x in rng.integers(1, 900 if i == 0 else 150, B)]
        cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(int).tolist()
        cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(int).tolist()
        w = custom(f"noalloc_{name}", H, D, cu_q, cu_k, std=1.0)
        announce(f"no-alloc call {i} ({name}: B={B} H={H} D={D} causal={causal})")
        t = make_inputs(w, "cuda", seed=30 + i)
        (a_o, a_l), (b_o, b_l), plan = both(t, w, causal)
        assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l), name
        check(t, w, causal, b_o, b_l, f"no-alloc {name} causal={causal}")
        plans.append(plan)
    assert plans[0] == plans[1]  # one static plan per GPU, shared by every call


def test_no_alloc_reports_bad_cu_and_writes_nothing():
    announce("no-alloc bad cu")
    w = custom("noalloc_bad", 2, 64, [0, 100, 300], [0, 120, 250], std=1.0)
    t = make_inputs(w, "cuda", seed=40)
    o, l = torch.full_like(t["out"], CANARY), torch.full_like(t["lse"], CANARY)
    bad_k = torch.tensor([0, 200, 150], dtype=torch.int32, device="cuda")
    _, _, plan = avf.attn_varlen_fwd_async_noalloc(t["q"], t["k"], t["v"], t["cu_q"], bad_k, w.max_seqlen_q,
                                                   w.max_seqlen_k, out=o, lse=l)
    torch.cuda.synchronize()
    assert avf.async_status(plan) == _binding.ECU
    assert bool((o == CANARY).all()) and bool((l == CANARY).all())
    # the next valid call overwrites the plan and succeeds
    (a_o, a_l), (b_o, b_l), _ = both(t, w, False)
    assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l)


def test_no_alloc_refuses_more_segments_than_the_static_plan_holds():
    announce("no-alloc segment limit")
    B = 65537
    cu = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    q = torch.zeros((8, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(avf.AttnVarlenError, match="EUNSUPPORTED"):
        avf.attn_varlen_fwd_async_noalloc(q, q, q, cu, cu, 0, 0)
    # at the limit the call is accepted (every segment empty: nothing to compute)
    cu = torch.zeros(65536 + 1, dtype=torch.int32, device="cuda")
    o, l, plan = avf.attn_varlen_fwd_async_noalloc(q, q, q, cu, cu, 0, 0)
    torch.cuda.synchronize()
    assert avf.async_status(plan) == 0
