"""GPU tests of the low-precision forward (per-head E4M3 q and k, 8-bit
score product) against oracle/fp8_oracle.py, through the C ABI. Marked
`gpu`; every case prints its name before it touches the GPU.

The quantization codes are integers that floating point decides: the
library and the oracle take that decision with the same fp32 operations
(amax, 448 / amax, x * inv, round to nearest even), so codes and amax words
are compared bit for bit. The attention that follows is compared with the
oracle's fp64 attention on the dequantized q and k at the bf16 path's bar.
"""
import numpy as np
import pytest
import torch

from oracle import blas_oracle
from oracle import fp8_oracle
import varlen_flashattention_forward_amd as avf
from varlen_flashattention_forward_amd import _binding
from varlen_flashattention_forward_amd.workloads import WORKLOADS, custom, make_inputs, sample_rows

from parity import compare

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


def run_fp8(t, w, causal=False, hostcu=True):
    kw = dict(cu_seqlens_q_host=list(w.cu_q), cu_seqlens_k_host=list(w.cu_k)) if hostcu else {}
    o, l, ws = avf.attn_varlen_fwd_fp8(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                                       softmax_scale=w.softmax_scale, out=t["out"], lse=t["lse"], causal=causal, **kw)
    torch.cuda.synchronize()
    return o, l, ws


def cpu_bits(x):
    return x.contiguous().cpu()


CASES = {
    "ragged_d128": (2, 128, [0, 1, 300, 300, 813, 1100], [0, 70, 71, 104, 744, 873]),
    "ragged_d64": (3, 64, [0, 129, 190, 577], [0, 64, 321, 322]),
    "self_d128": (2, 128, [0, 640, 1000], None),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_fp8_codes_are_the_oracles(name):
    H, D, cu_q, cu_k = CASES[name]
    announce(f"fp8 codes {name}")
    w = custom(name, H, D, cu_q, cu_k, std=1.0)
    t = make_inputs(w, "cuda", seed=21)
    t["k"][:, 1] *= 0.01  # heads of very different ranges
    _, _, ws = run_fp8(t, w)
    q8o, k8o = avf.fp8_workspace_offsets(w.total_q, w.total_k, H, D)
    wsc = ws.cpu().numpy()
    amax = wsc[:8 * H].view(np.uint32)
    q8 = wsc[q8o:q8o + w.total_q * H * D].reshape(w.total_q, H, D)
    k8 = wsc[k8o:k8o + w.total_k * H * D].reshape(w.total_k, H, D)
    rq, sq, _ = fp8_oracle.quantize_per_head(cpu_bits(t["q"]), w.total_q)
    rk, sk, _ = fp8_oracle.quantize_per_head(cpu_bits(t["k"]), w.total_k)
    assert np.array_equal(amax[:H].view(np.float32) / np.float32(448), sq)
    assert np.array_equal(amax[H:].view(np.float32) / np.float32(448), sk)
    assert np.array_equal(q8, rq) and np.array_equal(k8, rk)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_fp8_matches_quantized_oracle(name, causal):
    H, D, cu_q, cu_k = CASES[name]
    announce(f"fp8 parity {name} causal={causal}")
    w = custom(name, H, D, cu_q, cu_k, std=1.0)
    t = make_inputs(w, "cuda", seed=22)
    o, l, _ = run_fp8(t, w, causal)
    ro, rl = fp8_oracle.attn_varlen_fwd_fp8(cpu_bits(t["q"]), cpu_bits(t["k"]), cpu_bits(t["v"]), w.cu_q, w.cu_k,
                                            f32(w.softmax_scale), causal=causal)
    st = compare(o.float().cpu().numpy(), l[:, :w.total_q].t().cpu().numpy(), ro, rl, f"fp8 {name}")
    # distance to exact attention on the unquantized inputs (context, not parity)
    eo, _ = blas_oracle.attn_varlen_fwd(cpu_bits(t["q"]), cpu_bits(t["k"]), cpu_bits(t["v"]), w.cu_q, w.cu_k,
                                        f32(w.softmax_scale), causal=causal)
    g = o.float().cpu().numpy().astype(np.float64)
    cos = (g * eo).sum() / np.sqrt((g * g).sum() * (eo * eo).sum())
    print(f"[fp8 {name} causal={causal}] vs quantized oracle {st}; cosine to exact attention {cos:.6f}", flush=True)
    assert cos > 0.99


def test_fp8_device_cu_equals_host_cu():
    announce("fp8 device cu")
    H, D, cu_q, cu_k = CASES["ragged_d128"]
    w = custom("dev", H, D, cu_q, cu_k, std=1.0)
    t = make_inputs(w, "cuda", seed=23)
    a, al, _ = run_fp8(t, w)
    a, al = a.clone(), al.clone()
    b, bl, _ = run_fp8(t, w, hostcu=False)
    assert torch.equal(a, b) and torch.equal(al[:, :w.total_q], bl[:, :w.total_q])


def test_fp8_rejects_head_dim_96():
    announce("fp8 head_dim 96")
    w = custom("d96", 2, 96, [0, 100], std=1.0)
    t = make_inputs(w, "cuda", seed=24)
    with pytest.raises(avf.AttnVarlenError) as e:
        run_fp8(t, w)
    assert e.value.code == _binding.EUNSUPPORTED


def test_fp8_full_size_sampled():
    """dense_77k: 4096 seeded rows compared in full (every head) against the
    oracle, which quantizes q and k per head as the library does."""
    w = WORKLOADS["dense_77k"]
    announce("fp8 full size dense_77k")
    t = make_inputs(w, "cuda", seed=0)
    o, l, _ = run_fp8(t, w)
    rows = sample_rows(w, 4096, edge=16)
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    ro, rl = fp8_oracle.attn_varlen_fwd_fp8(q, k, v, w.cu_q, w.cu_k, f32(w.softmax_scale), rows=rows)
    idx = torch.tensor(rows, device="cuda")
    go = o.index_select(0, idx).float().cpu().numpy()
    gl = l[:, :w.total_q][:, rows].t().cpu().numpy()
    st = compare(go, gl, ro, rl, "fp8 dense_77k")
    print(f"[fp8 dense_77k] {st}", flush=True)


def test_fp8_strided_views_equal_contiguous():
    """q, k, v as views of wider buffers (row stride 3*H*D + 64), and as
    head-major views (row stride D, head stride tokens * D, out too): the same
    outputs as their contiguous copies."""
    announce("fp8 strided views")
    w = custom("fp8_strided", 4, 128, [0, 333, 900], [0, 500, 1200], std=1.0)
    H, D = 4, 128
    g = torch.Generator(device="cuda").manual_seed(31)
    def view(n):
        buf = torch.randn((n, 3 * H * D + 64), dtype=torch.bfloat16, device="cuda", generator=g)
        return buf[:, 64:64 + H * D].view(n, H, D)
    t = make_inputs(w, "cuda", seed=31)
    t["q"], t["k"], t["v"] = view(w.total_q), view(w.total_k), view(w.total_k)
    a, al, _ = run_fp8(t, w)
    a, al = a.clone(), al.clone()
    for n in ("q", "k", "v"):
        t[n] = t[n].contiguous()
    b, bl, _ = run_fp8(t, w)
    assert torch.equal(a, b) and torch.equal(al[:, :w.total_q], bl[:, :w.total_q])
    b, bl = b.clone(), bl.clone()
    for n in ("q", "k", "v"):
        t[n] = t[n].permute(1, 0, 2).contiguous().permute(1, 0, 2)
    t["out"] = torch.empty((H, w.total_q, D), dtype=torch.bfloat16, device="cuda").permute(1, 0, 2)
    c, cl, _ = run_fp8(t, w)
    assert c.stride() == (D, w.total_q * D, 1)
    assert torch.equal(c, b) and torch.equal(cl[:, :w.total_q], bl[:, :w.total_q])


def test_fp8_many_segments_span_launches():
    """300 segments: the plan splits them over launches of 128; codes index
    absolute token rows across launches."""
    announce("fp8 300 segments")
    rng = np.random.default_rng(32)
    lens_q = [0 if rng.random() < 0.1 else int(rng.integers(1, 150)) for _ in range(300)]
    lens_k = [0 if rng.random() < 0.1 else int(rng.integers(1, 150)) for _ in range(300)]
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(int).tolist()
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(int).tolist()
    w = custom("fp8_many", 2, 64, cu_q, cu_k, std=1.0)
    t = make_inputs(w, "cuda", seed=32)
    o, l, _ = run_fp8(t, w)
    rows = sample_rows(w, 4, edge=1)
    ro, rl = fp8_oracle.attn_varlen_fwd_fp8(cpu_bits(t["q"]), cpu_bits(t["k"]), cpu_bits(t["v"]), w.cu_q, w.cu_k,
                                            f32(w.softmax_scale), rows=rows)
    idx = torch.tensor(rows, device="cuda")
    compare(o.index_select(0, idx).float().cpu().numpy(), l[:, :w.total_q].index_select(1, idx).t().cpu().numpy(),
            ro, rl, "fp8 many segments")
