"""GPU tests of the short-segment configurations the forward picks from the
call's max_seqlen_k: one K/V stage of 128 keys (max_seqlen_k <= 128), and
64-key stages in smaller rings (max_seqlen_k <= 512); both run 4-wave
workgroups two per CU. Covered here:
- parity with the oracle on ragged segments: empty, single-key, full-stage and
  tail segments, every stage count up to eight 64-key stages, query segments
  of several tiles; causal and not;
- bitwise agreement of the three configurations on the same inputs (they run
  the same per-row arithmetic in 32-row wave groups);
- the sync-free and batched entry points;
- the rejection of a segment longer than max_seqlen_k;
- the full-size short-segment workloads.
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
GENERAL = 1 << 20  # a max_seqlen_k that selects the general configuration


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


# one-stage case: query lengths 0, 1, a full 128-row tile and several tiles
# with tails; key lengths 0, 1, partial stages and a full 128-key stage
_CQ1 = [0, 1, 129, 129, 429, 942, 1070, 1075]
_CK1 = [0, 1, 129, 134, 134, 261, 325, 453]
# 64-key-stage case: key lengths at and around every stage boundary up to 8
# stages (all positions of the 2 K and 3 V buffers, the last-stage barrier)
_LK8 = [1, 63, 64, 65, 127, 128, 129, 191, 192, 193, 300, 447, 448, 511, 512, 0]
_LQ8 = [37, 1, 130, 64, 0, 200, 3, 129, 255, 17, 400, 90, 128, 5, 260, 40]
_CQ8 = np.concatenate([[0], np.cumsum(_LQ8)]).tolist()
_CK8 = np.concatenate([[0], np.cumsum(_LK8)]).tolist()


def case(kind, D, causal):
    cq, ck = (_CQ1, _CK1) if kind == "one" else (_CQ8, _CK8)
    return custom(f"{kind}_d{D}{'_causal' if causal else ''}", 3, D, cq, ck, std=1.0, causal=causal)


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


def test_configuration_thresholds():
    assert avf.one_stage_keys() == 128 and avf.short_stage_keys() == 512
    for D in (64, 96, 128):
        assert avf.block_m(D, 128) == avf.block_m(D, 512) == 128
        assert avf.block_m(D, GENERAL) == avf.block_m(D) != 128


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("kind", ["one", "short"])
def test_short_configs_full_oracle(kind, D, causal):
    w = case(kind, D, causal)
    assert w.max_seqlen_k == (128 if kind == "one" else 512)
    announce(f"{kind} configuration, full oracle {w.name}")
    t = make_inputs(w, DEV, seed=21)
    o, l = run(t, w, w.max_seqlen_k)
    check_oracle(o, l, t, w)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("kind", ["one", "short"])
def test_short_configs_equal_general_bitwise(kind, D, causal):
    """Every configuration that may run these segments gives the same bits."""
    w = case(kind, D, causal)
    announce(f"{kind} configuration == general {w.name}")
    t = make_inputs(w, DEV, seed=22)
    ref_o, ref_l = run(t, w, GENERAL, hostcu=True)
    # one-stage (128) and 64-key stages (129, 512) for the first case; 64-key stages for the second
    for max_k in ((128, 129, 512) if kind == "one" else (512,)):
        o, l = run(t, w, max_k)
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), max_k


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["one", "short"])
def test_short_configs_sync_free_bitwise(kind, causal):
    w = case(kind, 128, causal)
    announce(f"{kind} configuration sync-free {w.name}")
    t = make_inputs(w, DEV, seed=23)
    ref_o, ref_l = run(t, w, GENERAL, hostcu=True)
    for max_k in (w.max_seqlen_k, 512, GENERAL):
        o = torch.full_like(t["out"], CANARY)
        l = torch.full_like(t["lse"], CANARY)
        _, _, ws = avf.attn_varlen_fwd_async(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, max_k,
                                             softmax_scale=w.softmax_scale, out=o, lse=l, causal=causal)
        assert avf.async_status(ws) == 0
        check_oracle(o, l, t, w)
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), max_k


@pytest.mark.parametrize("max_k", [128, 512])
def test_short_configs_reject_a_longer_key_segment(max_k):
    """max_seqlen_k with a segment one key longer: the host entry returns
    EMAXSEQ without a launch; the sync-free entry's planner stores EMAXSEQ and
    no workgroup writes anything."""
    w = custom("over", 2, 128, [0, 64, 128], [0, max_k + 1, max_k + 60], std=1.0)
    announce(f"rejection of a {max_k + 1}-key segment at max_seqlen_k {max_k}")
    t = make_inputs(w, DEV, seed=24)
    o = torch.full_like(t["out"], CANARY)
    l = torch.full_like(t["lse"], CANARY)
    with pytest.raises(avf.AttnVarlenError, match="EMAXSEQ"):
        avf.attn_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], 64, max_k, out=o, lse=l)
    _, _, ws = avf.attn_varlen_fwd_async(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], 64, max_k, out=o, lse=l)
    assert avf.async_status(ws) == _binding.EMAXSEQ
    torch.cuda.synchronize()
    assert torch.all(o == CANARY) and torch.all(l == CANARY)


@pytest.mark.parametrize("Sk", [100, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_short_configs_batched(causal, Sk):
    """attn_fwd on [W, S, H, D] with Sk <= 512 takes a short configuration:
    equal bits to the varlen call, oracle parity."""
    announce(f"batched Sk={Sk} causal={causal}")
    W, Sq, H, D = 9, 200, 3, 96
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
    w = custom("batched", H, D, cq.tolist(), ck.tolist(), causal=causal)
    ro, rl = oracle.attn_varlen_fwd(q.reshape(W * Sq, H, D).cpu(), k.reshape(W * Sk, H, D).cpu(),
                                    v.reshape(W * Sk, H, D).cpu(), w.cu_q, w.cu_k, f32(w.softmax_scale),
                                    causal=causal)
    compare(ov.float().cpu().numpy(), lv.t().cpu().numpy(), ro, rl, f"batched Sk={Sk} causal={causal}")


@pytest.mark.parametrize("name", ["short_128", "short_256", "short_512"])
def test_short_workloads_full_size_sampled(name):
    """The short-segment workloads at full size in the configuration the
    benchmark times (64 segments, H=56, D=128): every row against the oracle
    (the segments are shorter than the 4096 seeded rows per segment that the
    other full-size checks compare)."""
    w = WORKLOADS[name]
    assert avf.block_m(w.head_dim, w.max_seqlen_k) == 128
    announce(f"{name} full size, sampled rows")
    t = make_inputs(w, DEV, seed=0)
    o, l = run(t, w, w.max_seqlen_k)
    rows = sample_rows(w, 4096, edge=4)
    assert len(rows) == w.total_q
    check_oracle(o, l, t, w, rows)
