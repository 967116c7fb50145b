"""GPU tests of the sync-free forward (device planner + bounded, looping
grid): its outputs against the CPU oracle at the parity bar (small cases in
full, larger ones on seeded rows, the SM120 page's varlen_cross call at full
size on 4096 rows per segment), bitwise agreement with the host-planned path,
one launch for any number of segments, invalid cu_seqlens values reported
through the workspace status with the outputs untouched, and capture in a HIP
graph. Marked `gpu`; every case prints its name before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import blas_oracle
import varlen_flashattention_forward_amd as avf
from varlen_flashattention_forward_amd import _binding
from varlen_flashattention_forward_amd.workloads import CANARY, WORKLOADS, custom, make_inputs, sample_rows

from parity import compare

pytestmark = pytest.mark.gpu


def f32(x):
    """The fp32 value the library receives, widened for the oracle."""
    return float(np.float32(x))


def check_oracle(o, l, t, w, causal=False, rows=None, impl="c", label=""):
    """The sync-free outputs o [total_q, H, D], l [H, >= total_q] on the given
    global query rows (all if None) against the oracle at the parity bar."""
    rows = list(range(w.total_q)) if rows is None else rows
    idx = torch.tensor(rows, dtype=torch.long, device=o.device)
    og = o.index_select(0, idx).float().cpu().numpy()
    lg = l[:, :w.total_q].index_select(1, idx).t().cpu().numpy()
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    fn = oracle.attn_varlen_fwd if impl == "c" else blas_oracle.attn_varlen_fwd
    ro, rl = fn(q, k, v, w.cu_q, w.cu_k, f32(w.softmax_scale), rows=rows, causal=causal)
    stats = compare(og, lg, ro, rl, label or w.name)
    print(f"[gpu-case] {label or w.name} oracle {stats}", flush=True)
    return stats


def announce(label):
    print(f"\n[gpu-case] {label}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    avf.lib()
    yield
    torch.cuda.synchronize()


def host_planned(t, w, causal=False):
    o = torch.full_like(t["out"], CANARY)
    l = torch.full_like(t["lse"], CANARY)
    avf.attn_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                        softmax_scale=w.softmax_scale, out=o, lse=l, causal=causal,
                        cu_seqlens_q_host=list(w.cu_q), cu_seqlens_k_host=list(w.cu_k))
    return o, l


def sync_free(t, w, causal=False, ws=None, max_q=None, max_k=None):
    o = torch.full_like(t["out"], CANARY)
    l = torch.full_like(t["lse"], CANARY)
    _, _, ws = avf.attn_varlen_fwd_async(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"],
                                         w.max_seqlen_q if max_q is None else max_q,
                                         w.max_seqlen_k if max_k is None else max_k, workspace=ws,
                                         softmax_scale=w.softmax_scale, out=o, lse=l, causal=causal)
    return o, l, ws


def random_cu(rng, B, max_len, empty_frac=0.15):
    lens = [0 if rng.random() < empty_frac else int(rng.integers(1, max_len + 1)) for _ in range(B)]
    return np.concatenate([[0], np.cumsum(lens)]).astype(int).tolist()


CASES = {
    # (H, D, cu_q, cu_k)
    "cross_d128": (4, 128, [0, 4032, 9072, 9100, 10000], [0, 1758, 3516, 5274, 7032]),
    "ragged_d96": (3, 96, [0, 1, 300, 300, 813, 1100], [0, 70, 71, 104, 744, 873]),
    "self_d64": (2, 64, [0, 255, 256, 700], None),
}


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_sync_free_equals_host_planned(name, causal):
    H, D, cu_q, cu_k = CASES[name]
    announce(f"sync-free {name} causal={causal}")
    w = custom(name, H, D, cu_q, cu_k, std=1.0)
    t = make_inputs(w, "cuda", seed=1)
    a_o, a_l = host_planned(t, w, causal)
    b_o, b_l, ws = sync_free(t, w, causal)
    torch.cuda.synchronize()
    assert avf.async_status(ws) == 0
    check_oracle(b_o, b_l, t, w, causal)
    assert torch.equal(a_o, b_o)
    assert torch.equal(a_l[:, :w.total_q], b_l[:, :w.total_q])


def test_sync_free_many_segments_one_launch():
    """300 segments (the host-planned path splits them over launches of 128)."""
    announce("sync-free 300 segments")
    rng = np.random.default_rng(2)
    cu_q = random_cu(rng, 300, 200)
    cu_k = random_cu(rng, 300, 150)
    w = custom("many", 2, 64, cu_q, cu_k, std=1.0)
    t = make_inputs(w, "cuda", seed=2)
    a_o, a_l = host_planned(t, w)
    b_o, b_l, ws = sync_free(t, w)
    torch.cuda.synchronize()
    assert avf.async_status(ws) == 0
    check_oracle(b_o, b_l, t, w)
    assert torch.equal(a_o, b_o) and torch.equal(a_l[:, :w.total_q], b_l[:, :w.total_q])


@pytest.mark.parametrize("B", [1, 63, 64, 65, 4097, 5000])
def test_sync_free_segment_search_boundaries(B):
    """Segment counts at the steps of the device decode's 64-way search (one
    step up to 64 segments, two up to 4096, three beyond), with empty segments
    in long runs so that equal prefix entries straddle probe positions."""
    announce(f"sync-free segment search B={B}")
    rng = np.random.default_rng(100 + B)
    lens_q = rng.integers(1, 40, B)
    lens_k = rng.integers(1, 40, B)
    for a in rng.integers(0, B, max(1, B // 50)):  # runs of empty query segments
        lens_q[a:a + int(rng.integers(1, 200))] = 0
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(int).tolist()
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(int).tolist()
    if cu_q[-1] == 0:
        cu_q[-1] = 1  # at least one row: make the last segment one row long
    w = custom(f"search{B}", 2, 64, cu_q, cu_k, std=1.0)
    t = make_inputs(w, "cuda", seed=7)
    a_o, a_l = host_planned(t, w)
    b_o, b_l, ws = sync_free(t, w)
    torch.cuda.synchronize()
    assert avf.async_status(ws) == 0
    check_oracle(b_o, b_l, t, w)
    assert torch.equal(a_o, b_o) and torch.equal(a_l[:, :w.total_q], b_l[:, :w.total_q])


def test_sync_free_grid_smaller_than_tile_count_loops():
    """More tiles than the 8192-workgroup cap: workgroups take several tiles."""
    announce("sync-free looping grid")
    w = custom("loop", 64, 64, [0, 33000], std=1.0)
    bm = avf.block_m(64)
    assert avf.count_tiles(w.cu_q, 64, bm) > avf.async_grid(w.total_q, 1, 64, 64, w.max_seqlen_q,
                                                            w.max_seqlen_k) == 8192
    t = make_inputs(w, "cuda", seed=3)
    a_o, a_l = host_planned(t, w)
    b_o, b_l, ws = sync_free(t, w)
    torch.cuda.synchronize()
    assert avf.async_status(ws) == 0
    check_oracle(b_o, b_l, t, w, rows=sample_rows(w, 2048, edge=16), impl="blas")
    assert torch.equal(a_o, b_o) and torch.equal(a_l[:, :w.total_q], b_l[:, :w.total_q])


@pytest.mark.parametrize("bad", ["decreasing", "past_tokens", "over_max_q", "nonzero_start"])
def test_sync_free_reports_bad_cu_and_writes_nothing(bad):
    announce(f"sync-free bad cu {bad}")
    w = custom("bad", 2, 64, [0, 100, 300], [0, 120, 250], std=1.0)
    t = make_inputs(w, "cuda", seed=4)
    cq, ck = list(w.cu_q), list(w.cu_k)
    max_q = None
    if bad == "decreasing":
        ck = [0, 200, 150]
        expect = _binding.ECU
    elif bad == "past_tokens":
        cq = [0, 100, 301]
        expect = _binding.ECU
    elif bad == "over_max_q":
        max_q = 150
        expect = _binding.EMAXSEQ
    else:
        cq = [5, 100, 300]
        expect = _binding.ECU
    t["cu_q"] = torch.tensor(cq, dtype=torch.int32, device="cuda")
    t["cu_k"] = torch.tensor(ck, dtype=torch.int32, device="cuda")
    o, l, ws = sync_free(t, w, max_q=max_q)
    torch.cuda.synchronize()
    assert avf.async_status(ws) == expect
    assert bool((o == CANARY).all()) and bool((l == CANARY).all())


def test_sync_free_in_a_hip_graph():
    """Capture one sync-free call, replay it on new inputs several times with
    eager work between replays; every replay equals the host-planned result."""
    announce("sync-free graph capture")
    w = custom("graph", 4, 128, [0, 700, 1500, 1501], [0, 400, 1200, 1900], std=1.0)
    t = make_inputs(w, "cuda", seed=5)
    ws = avf.async_workspace(w.num_segments, "cuda")
    o = torch.empty_like(t["out"])
    l = torch.empty_like(t["lse"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        # warm-up call outside capture
        avf.attn_varlen_fwd_async(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                                  workspace=ws, out=o, lse=l)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        avf.attn_varlen_fwd_async(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                                  workspace=ws, out=o, lse=l)
    for rep in range(3):
        gen = torch.Generator(device="cuda").manual_seed(100 + rep)
        t["q"].copy_(torch.randn(t["q"].shape, dtype=torch.bfloat16, device="cuda", generator=gen))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_o, ref_l = host_planned(t, w)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o), rep
        assert torch.equal(l[:, :w.total_q], ref_l[:, :w.total_q]), rep
        check_oracle(o, l, t, w, label=f"graph replay {rep}")


def test_sync_free_strided_views():
    """The page's [N, 9728] layout through the sync-free entry: equal to the
    host-planned path on the same views."""
    announce("sync-free strided 9728")
    w = custom("async_strided", 16, 96, [0, 700, 1300, 2100], std=0.1, layout="stride9728", outer_stride=9728)
    t = make_inputs(w, "cuda", seed=6)
    a_o, a_l = host_planned(t, w)
    b_o, b_l, ws = sync_free(t, w)
    torch.cuda.synchronize()
    assert avf.async_status(ws) == 0
    check_oracle(b_o, b_l, t, w)
    assert torch.equal(a_o, b_o) and torch.equal(a_l[:, :w.total_q], b_l[:, :w.total_q])


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_sync_free_head_major_views(causal):
    """Head-major views (row stride D, head stride tokens * D) of q, k, v and
    out through the sync-free entry: equal to the host-planned token-major
    results bit for bit."""
    announce(f"sync-free head-major causal={causal}")
    cu_q, cu_k = [0, 300, 301, 1000], [0, 128, 700, 1500]
    wt = custom("async_tm", 3, 128, cu_q, cu_k, std=1.0)
    wh = custom("async_hm", 3, 128, cu_q, cu_k, std=1.0, layout="head_major")
    tt, th = make_inputs(wt, "cuda", seed=8), make_inputs(wh, "cuda", seed=8)
    a_o, a_l = host_planned(tt, wt, causal)
    b_o, b_l, ws = sync_free(th, wh, causal)
    torch.cuda.synchronize()
    assert avf.async_status(ws) == 0
    assert b_o.stride() == (128, wh.total_q * 128, 1)
    check_oracle(b_o, b_l, th, wh, causal)
    assert torch.equal(a_o, b_o) and torch.equal(a_l[:, :wt.total_q], b_l[:, :wt.total_q])


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_sync_free_full_size_varlen_cross(causal):
    """The SM120 page's captured call ("Bug 2 details": eight query windows
    summing to 35280 rows against eight 17580-row key segments, H = 56,
    D = 128) through the sync-free entry, the form that page's scheduler
    fault concerns: 4096 seeded rows per segment (a shorter segment whole,
    first and last 16 rows always) against the oracle, every head and column."""
    w = WORKLOADS["varlen_cross"]
    announce(f"sync-free full-size varlen_cross causal={causal}")
    torch.cuda.empty_cache()
    t = make_inputs(w, "cuda", seed=0)
    o, l, ws = sync_free(t, w, causal)
    torch.cuda.synchronize()
    assert avf.async_status(ws) == 0
    check_oracle(o, l, t, w, causal, rows=sample_rows(w, 4096, edge=16), impl="blas",
                 label=f"sync-free varlen_cross causal={causal}")
    del t, o, l
    torch.cuda.empty_cache()
