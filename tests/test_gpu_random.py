"""Seeded random sweep of the forward through the C ABI: random segment tables
(empty segments, query or key lengths up to 1500, so every configuration the
host can pick - one-stage, 64-key stages, general - is hit), random head
counts and head_dims, the causal mask, padded row and head strides on every
tensor, and max_seqlen_k either exact or loose. Each case compares sampled
rows with the oracle and checks that the output buffer's padding keeps its
canary. Marked `gpu`; every case prints its parameters before it touches the
GPU.
"""
import numpy as np
import pytest
import torch

from oracle import blas_oracle
import varlen_flashattention_forward_amd as avf
from varlen_flashattention_forward_amd.workloads import CANARY, custom, sample_rows

from parity import compare

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    avf.lib()
    yield
    torch.cuda.synchronize()


def padded_view(buf_rows, H, D, head_pad, row_pad, g, fill=None):
    """A [rows, H, D] bf16 view with head stride D + head_pad and row stride
    H * (D + head_pad) + row_pad, inside a buffer of random values (or `fill`)."""
    hs = D + head_pad
    rs = H * hs + row_pad
    if fill is None:
        base = torch.randn((buf_rows, rs), generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    else:
        base = torch.full((buf_rows, rs), fill, device=DEV, dtype=torch.bfloat16)
    view = base.as_strided((buf_rows, H, D), (rs, hs, 1))
    return base, view


def draw_case(seed):
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 96, 128]))
    H = int(rng.integers(1, 7))
    B = int(rng.integers(1, 30))
    regime = seed % 3  # key lengths of one stage, a few 64-key stages, or longer
    kmax = (128, 512, 1500)[regime]
    lq = [0 if rng.random() < 0.1 else int(rng.integers(1, 700)) for _ in range(B)]
    lk = [0 if rng.random() < 0.1 else int(rng.integers(1, kmax + 1)) for _ in range(B)]
    causal = bool(rng.random() < 0.4)
    loose = bool(rng.random() < 0.3)
    head_pad = int(rng.choice([0, 8, 32]))
    row_pad = int(rng.choice([0, 8, 24, 64]))
    return D, H, lq, lk, causal, loose, head_pad, row_pad


@pytest.mark.parametrize("seed", range(24))
def test_random_case(seed):
    D, H, lq, lk, causal, loose, head_pad, row_pad = draw_case(seed)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(int).tolist()
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(int).tolist()
    max_q, max_k = max(lq), max(lk)
    if loose:
        max_q, max_k = max_q + 37, max_k + 200
    print(f"\n[gpu-case] random seed={seed} D={D} H={H} B={len(lq)} max_k={max_k} causal={causal} "
          f"head_pad={head_pad} row_pad={row_pad} block_m={avf.block_m(D, max_k)}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(seed)
    nq, nk = max(cu_q[-1], 1), max(cu_k[-1], 1)
    _, q = padded_view(nq, H, D, head_pad, row_pad, g)
    _, k = padded_view(nk, H, D, head_pad, row_pad, g)
    _, v = padded_view(nk, H, D, head_pad, row_pad, g)
    obuf, out = padded_view(nq, H, D, head_pad, row_pad, g, fill=CANARY)
    lse = torch.full((H, nq + 3), CANARY, device=DEV, dtype=torch.float32)
    cq = torch.tensor(cu_q, dtype=torch.int32, device=DEV)
    ck = torch.tensor(cu_k, dtype=torch.int32, device=DEV)
    avf.attn_varlen_fwd(q, k, v, cq, ck, max_q, max_k, out=out, lse=lse, causal=causal)
    torch.cuda.synchronize()
    # padding of the output buffer (extra head columns and row tail) untouched
    hs = D + head_pad
    mask = torch.ones_like(obuf, dtype=torch.bool)
    for h in range(H):
        mask[:cu_q[-1], h * hs:h * hs + D] = False
    assert bool((obuf[mask] == CANARY).all()), "write outside out"
    assert bool((lse[:, cu_q[-1]:] == CANARY).all()), "write outside lse"
    if cu_q[-1] == 0:
        return
    w = custom(f"random{seed}", H, D, cu_q, cu_k, causal=causal)
    rows = sample_rows(w, 12, seed=seed, edge=3)
    idx = torch.tensor(rows, dtype=torch.long, device=DEV)
    og = out.index_select(0, idx).float().cpu().numpy()
    lg = lse[:, :cu_q[-1]].index_select(1, idx).t().cpu().numpy()
    ro, rl = blas_oracle.attn_varlen_fwd(q[:cu_q[-1]].contiguous().cpu(), k[:cu_k[-1]].contiguous().cpu(),
                                         v[:cu_k[-1]].contiguous().cpu(), cu_q, cu_k,
                                         float(np.float32(w.softmax_scale)), rows=rows, causal=causal)
    compare(og, lg, ro, rl, w.name)
