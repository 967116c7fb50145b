"""GPU tests of the one-stage configuration: the forward picks it when the
call's max_seqlen_k is at most one K/V stage (128 keys). Parity with the
oracle on ragged segments (empty, single-key, full-stage and tail segments,
query segments of several tiles), causal and not; bitwise agreement with the
general configuration on the same inputs (both run the same per-row
arithmetic in 32-row wave groups); the sync-free and batched entry points;
the rejection of a longer segment; and the full-size short-segment workload.
Marked `gpu`; every case prints its name before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import varlen_flashattention_forward_amd as avf
from varlen_flashattention_forward_amd import _binding
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


# query lengths span 0, 1, a full 128-row tile and several tiles with tails;
# key lengths 0, 1, partial stages and a full 128-key stage
_CQ = [0, 1, 129, 129, 429, 942, 1070, 1075]
_CK = [0, 1, 129, 134, 134, 261, 325, 453]


def case(D, causal):
    return custom(f"one_d{D}{'_causal' if causal else ''}", 3, D, _CQ, _CK, std=1.0, causal=causal)


def run(t, w, max_k, hostcu=False):
    o = torch.full_like(t["out"], CANARY)
    l = torch.full_like(t["lse"], CANARY)
    kw = dict(cu_seqlens_q_host=list(w.cu_q), cu_seqlens_k_host=list(w.cu_k)) if hostcu else {}
    avf.attn_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, max_k,
                        softmax_scale=w.softmax_scale, out=o, lse=l, causal=w.causal, **kw)
    torch.cuda.synchronize()
    return o, l


def check_oracle(o, l, t, w, rows=None):
    rows = list(range(w.total_q)) if rows is None else rows
    idx = torch.tensor(rows, dtype=torch.long, device=DEV)
    og = o.index_select(0, idx).float().cpu().numpy()
    lg = l[:, :w.total_q].index_select(1, idx).t().cpu().numpy()
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    ro, rl = oracle.attn_varlen_fwd(q, k, v, w.cu_q, w.cu_k, f32(w.softmax_scale), rows=rows, causal=w.causal)
    return compare(og, lg, ro, rl, w.name)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 96, 128])
def test_one_stage_full_oracle(D, causal):
    w = case(D, causal)
    assert w.max_seqlen_k == 128 and avf.block_m(D, w.max_seqlen_k) == 128
    announce(f"one-stage full oracle {w.name}")
    t = make_inputs(w, DEV, seed=21)
    o, l = run(t, w, w.max_seqlen_k)
    check_oracle(o, l, t, w)
    # LSE padding past total_q keeps its canary
    assert torch.all(l[:, w.total_q:] == CANARY)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 96, 128])
def test_one_stage_equals_general_bitwise(D, causal):
    """max_seqlen_k 128 (one stage) and 129 (general) give the same bits."""
    w = case(D, causal)
    announce(f"one-stage == general {w.name}")
    t = make_inputs(w, DEV, seed=22)
    a_o, a_l = run(t, w, 128)
    b_o, b_l = run(t, w, 129, hostcu=True)
    assert avf.block_m(D, 128) != avf.block_m(D, 129)
    assert torch.equal(a_o, b_o)
    assert torch.equal(a_l, b_l)


@pytest.mark.parametrize("causal", [False, True])
def test_one_stage_sync_free_bitwise(causal):
    w = case(128, causal)
    announce(f"one-stage sync-free {w.name}")
    t = make_inputs(w, DEV, seed=23)
    ref_o, ref_l = run(t, w, 128, hostcu=True)
    for max_k in (128, 129):
        o = torch.full_like(t["out"], CANARY)
        l = torch.full_like(t["lse"], CANARY)
        _, _, ws = avf.attn_varlen_fwd_async(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, max_k,
                                             softmax_scale=w.softmax_scale, out=o, lse=l, causal=causal)
        assert avf.async_status(ws) == 0
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), max_k


def test_one_stage_rejects_a_longer_key_segment():
    """max_seqlen_k 128 with a 129-key segment: the host entry returns
    EMAXSEQ without a launch; the sync-free entry's planner stores EMAXSEQ and
    no workgroup writes anything."""
    w = custom("one_over", 2, 128, [0, 64, 128], [0, 129, 200], std=1.0)
    announce("one-stage rejection of a 129-key segment")
    t = make_inputs(w, DEV, seed=24)
    o = torch.full_like(t["out"], CANARY)
    l = torch.full_like(t["lse"], CANARY)
    with pytest.raises(avf.AttnVarlenError, match="EMAXSEQ"):
        avf.attn_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], 64, 128, out=o, lse=l)
    _, _, ws = avf.attn_varlen_fwd_async(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], 64, 128, out=o, lse=l)
    assert avf.async_status(ws) == _binding.EMAXSEQ
    torch.cuda.synchronize()
    assert torch.all(o == CANARY) and torch.all(l == CANARY)


@pytest.mark.parametrize("causal", [False, True])
def test_one_stage_batched(causal):
    """attn_fwd on [W, S, H, D] with Sk <= 128 takes the one-stage
    configuration: equal bits to the varlen call, oracle parity."""
    announce(f"one-stage batched causal={causal}")
    W, Sq, Sk, H, D = 9, 200, 100, 3, 96
    g = torch.Generator(device=DEV).manual_seed(25)
    q, k, v = (torch.randn((W, S, H, D), generator=g, device=DEV).to(torch.bfloat16) for S in (Sq, Sk, Sk))
    o, l = avf.attn_fwd(q, k, v, causal=causal)
    cq = torch.tensor([b * Sq for b in range(W + 1)], dtype=torch.int32, device=DEV)
    ck = torch.tensor([b * Sk for b in range(W + 1)], dtype=torch.int32, device=DEV)
    ov, lv = avf.attn_varlen_fwd(q.reshape(W * Sq, H, D), k.reshape(W * Sk, H, D), v.reshape(W * Sk, H, D), cq, ck,
                                 Sq, Sk, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.reshape(W * Sq, H, D), ov)
    assert torch.equal(l.permute(1, 0, 2).reshape(H, W * Sq), lv)
    w = custom("one_batched", H, D, cq.tolist(), ck.tolist(), causal=causal)
    ro, rl = oracle.attn_varlen_fwd(q.reshape(W * Sq, H, D).cpu(), k.reshape(W * Sk, H, D).cpu(),
                                    v.reshape(W * Sk, H, D).cpu(), w.cu_q, w.cu_k, f32(w.softmax_scale),
                                    causal=causal)
    compare(ov.float().cpu().numpy(), lv.t().cpu().numpy(), ro, rl, f"one-stage batched causal={causal}")


def test_short_128_full_size_sampled():
    """The short-segment workload at its full size in the configuration the
    benchmark times (64 segments of 128 tokens, H=56, D=128): 16 sampled rows
    per segment against the oracle."""
    w = WORKLOADS["short_128"]
    assert avf.block_m(w.head_dim, w.max_seqlen_k) == 128
    announce("short_128 full size, sampled rows")
    t = make_inputs(w, DEV, seed=0)
    o, l = run(t, w, w.max_seqlen_k)
    rows = sample_rows(w, 16, edge=4)
    check_oracle(o, l, t, w, rows)
