"""Seeded synthetic inputs for packed variable-length attention.

This module draws random inputs and builds segment tables only; it holds none
of the attention arithmetic. Both the HIP path (tests, benchmark) and the CPU
oracle (tests) consume the bf16 tensors it returns, so how they are drawn never
affects parity.

Workloads (shapes taken from the pages; values are synthetic stand-ins because
the pages' workloads are a private video model and a private training job):

* ``dense_256``: one dense segment, S=256, H=2, D=64, N(0,1)*0.1.
* ``varlen_cross``: the captured window call of the FA4 SM120 issue page
  ("Bug 2 details"): 8 query segments summing to 35280 rows, H=56, D=128,
  8 key/value segments of 17580 rows each, N(0,1)*0.1.
* ``dense_77k``: S=77000, H=56, D=128, N(0,1): the length at which the NVFP4
  path of the ffpa-attn PR #387 page aborts ("Minimal reproduction").
* ``strided_9728``: N=410923 tokens in two segments [0,225304,410923], H=16,
  D=96, N(0,1)*0.1, every tensor an [N,H,D] view of an [N,9728] buffer (the
  cat([attn, mlp]) layout of the "_bwd_preprocess" overflow page).
* ``dense_117k``: S=117000, H=56, D=128, N(0,1) (the ~117k-token generation
  of the ffpa-attn page's "Verification").
* ``causal_77k``: ``dense_77k`` with the causal mask (query row r of a segment
  sees keys j <= r + Lk - Lq); the pages only run causal=False, so this is an
  extension, with FLOPs counted over the visible (query, key) pairs.
* ``short_128``, ``short_256``, ``short_512``: 64 segments of S = 128, 256,
  512 tokens, H=56, D=128, N(0,1)*0.1: the short-segment regime, where the
  arithmetic intensity falls below the MFMA/HBM ridge and the forward is
  measured in HBM GB/s; shorter than the W x S sweep (S = 1024 .. 24576) of
  the FA4 SM120 issue page ("What rules things out").
* ``bwd_9728``: the backward case of the _bwd_preprocess page ("Verified
  sample", repro script): N=410923 in segments [0,225304,410923], H=16, D=96;
  q, k, v one contiguous randn(3, N, H, D)*0.1 draw, dout (``make_dout``) an
  [N, H, D] view with row stride 9728, N(0,1)*0.1 from its own seed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    num_heads: int
    head_dim: int
    cu_q: tuple
    cu_k: tuple
    std: float
    self_attention: bool        # cu_q == cu_k, q/k/v drawn together
    layout: str = "contiguous"  # or "stride9728", or "head_major"
    outer_stride: int = 0       # elements per token row of the shared buffer
    causal: bool = False        # row r of a segment sees keys j <= r + Lk - Lq
    notes: str = field(default="", compare=False)

    @property
    def num_segments(self) -> int:
        return len(self.cu_q) - 1

    @property
    def total_q(self) -> int:
        return self.cu_q[-1]

    @property
    def total_k(self) -> int:
        return self.cu_k[-1]

    @property
    def max_seqlen_q(self) -> int:
        return max((b - a for a, b in zip(self.cu_q[:-1], self.cu_q[1:])), default=0)

    @property
    def max_seqlen_k(self) -> int:
        return max((b - a for a, b in zip(self.cu_k[:-1], self.cu_k[1:])), default=0)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def visible_keys(self, row: int) -> int:
        """Keys global query row `row` attends to (all of its segment's unless causal)."""
        b = max(i for i in range(self.num_segments) if self.cu_q[i] <= row)
        lq = self.cu_q[b + 1] - self.cu_q[b]
        lk = self.cu_k[b + 1] - self.cu_k[b]
        if not self.causal:
            return lk
        return max(0, min(lk, row - self.cu_q[b] + lk - lq + 1))

    def flops(self) -> int:
        """4 * D * H * (attended (query, key) pairs) summed over segments, an
        exact integer: 4 * Lq * Lk * D * H per segment without the causal mask."""
        tot = 0
        for b in range(self.num_segments):
            lq = self.cu_q[b + 1] - self.cu_q[b]
            lk = self.cu_k[b + 1] - self.cu_k[b]
            if self.causal:
                # row r sees clamp(r + lk - lq + 1, 0, lk) keys
                pairs = sum(max(0, min(lk, r + lk - lq + 1)) for r in range(lq))
            else:
                pairs = lq * lk
            tot += 4 * pairs * self.head_dim * self.num_heads
        return tot

    def algorithmic_bytes(self) -> int:
        """Q, K, V and O in bf16 plus the fp32 LSE, each moved once."""
        hd = self.num_heads * self.head_dim
        return 2 * hd * (2 * self.total_q + 2 * self.total_k) + 4 * self.num_heads * self.total_q


def _cu_uniform(n_seg: int, length: int) -> tuple:
    return tuple(i * length for i in range(n_seg + 1))


WORKLOADS = {
    "dense_256": Workload("dense_256", 2, 64, (0, 256), (0, 256), 0.1, True),
    "varlen_cross": Workload(
        "varlen_cross", 56, 128,
        (0, 4032, 9072, 14112, 19152, 24292, 29232, 34272, 35280),
        _cu_uniform(8, 17580), 0.1, False),
    "dense_77k": Workload("dense_77k", 56, 128, (0, 77000), (0, 77000), 1.0, True),
    "strided_9728": Workload("strided_9728", 16, 96, (0, 225304, 410923), (0, 225304, 410923),
                             0.1, True, layout="stride9728", outer_stride=9728),
    "dense_117k": Workload("dense_117k", 56, 128, (0, 117000), (0, 117000), 1.0, True),
    "causal_77k": Workload("causal_77k", 56, 128, (0, 77000), (0, 77000), 1.0, True, causal=True),
    "short_128": Workload("short_128", 56, 128, _cu_uniform(64, 128), _cu_uniform(64, 128), 0.1, True),
    "short_256": Workload("short_256", 56, 128, _cu_uniform(64, 256), _cu_uniform(64, 256), 0.1, True),
    "short_512": Workload("short_512", 56, 128, _cu_uniform(64, 512), _cu_uniform(64, 512), 0.1, True),
    # one GPU's share of dense_117k split eight ways: by heads (7 of 56), or by
    # query rows (context parallel: 14625 rows against all 117000 keys)
    "shard_heads_117k": Workload("shard_heads_117k", 7, 128, (0, 117000), (0, 117000), 1.0, True),
    "shard_rows_117k": Workload("shard_rows_117k", 56, 128, (0, 14625), (0, 117000), 1.0, False),
    # backward: contiguous q, k, v; dout an [N, H, D] view of an [N, 9728] buffer (make_dout)
    "bwd_9728": Workload("bwd_9728", 16, 96, (0, 225304, 410923), (0, 225304, 410923), 0.1, True,
                         outer_stride=9728),
}

#: Canary written into the parts of an output buffer the kernel must not touch.
CANARY = -1234.0  # exactly representable in bf16


def custom(name: str, num_heads: int, head_dim: int, cu_q, cu_k=None, std: float = 0.1,
           layout: str = "contiguous", outer_stride: int = 0, causal: bool = False) -> Workload:
    cu_q = tuple(int(x) for x in cu_q)
    self_attn = cu_k is None
    cu_k = cu_q if cu_k is None else tuple(int(x) for x in cu_k)
    return Workload(name, num_heads, head_dim, cu_q, cu_k, std, self_attn, layout, outer_stride, causal)


def _generator(device, seed: int) -> torch.Generator:
    return torch.Generator(device=device).manual_seed(seed)


def make_inputs(w: Workload, device="cuda", seed: int = 0, lse_head_pad: int = 0):
    """Draw q, k, v for workload `w` and allocate out/lse.

    Returns a dict with q, k, v, out (bf16 [tokens, H, D] views), lse (fp32
    [H, total_q + lse_head_pad] with a canary tail), cu_q/cu_k (int32 tensors on
    `device`) and `out_base` (the full buffer `out` lives in, canary-filled).
    """
    H, D = w.num_heads, w.head_dim
    g = _generator(device, seed)
    bf = torch.bfloat16
    if w.layout == "stride9728":
        if not w.self_attention:
            raise ValueError("the strided layout is a self-attention layout")
        S = w.outer_stride
        if 3 * H * D > S:
            raise ValueError("outer stride too small for q, k, v slices")
        n = w.total_q
        x = torch.empty((n, S), dtype=bf, device=device)
        x.normal_(generator=g)
        x.mul_(w.std)
        hd = H * D
        q = x[:, 0:hd].view(n, H, D)
        k = x[:, hd:2 * hd].view(n, H, D)
        v = x[:, 2 * hd:3 * hd].view(n, H, D)
        y = torch.full((n, S), CANARY, dtype=bf, device=device)
        out = y[:, 0:hd].view(n, H, D)
        out_base = y
    else:
        if w.self_attention:
            qkv = torch.randn((3, w.total_q, H, D), dtype=bf, device=device, generator=g)
            if w.std != 1.0:
                qkv.mul_(w.std)
            q, k, v = qkv[0], qkv[1], qkv[2]
        else:
            q = torch.randn((w.total_q, H, D), dtype=bf, device=device, generator=g)
            k = torch.randn((w.total_k, H, D), dtype=bf, device=device, generator=g)
            v = torch.randn((w.total_k, H, D), dtype=bf, device=device, generator=g)
            if w.std != 1.0:
                q.mul_(w.std)
                k.mul_(w.std)
                v.mul_(w.std)
        if w.layout == "head_major":
            # the same values stored head by head: [H, tokens, D] buffers seen
            # as [tokens, H, D] views (row stride D, head stride tokens * D)
            q, k, v = (x.permute(1, 0, 2).contiguous().permute(1, 0, 2) for x in (q, k, v))
            out_base = torch.full((H, w.total_q, D), CANARY, dtype=bf, device=device)
            out = out_base.permute(1, 0, 2)
        elif w.layout == "contiguous":
            out_base = torch.full((w.total_q, H, D), CANARY, dtype=bf, device=device)
            out = out_base
        else:
            raise ValueError(f"unknown layout {w.layout!r}")
    lse = torch.full((H, w.total_q + lse_head_pad), CANARY, dtype=torch.float32, device=device)
    cu_q = torch.tensor(w.cu_q, dtype=torch.int32, device=device)
    cu_k = torch.tensor(w.cu_k, dtype=torch.int32, device=device)
    return {"q": q, "k": k, "v": v, "out": out, "out_base": out_base, "lse": lse,
            "cu_q": cu_q, "cu_k": cu_k}


def sample_rows(w: Workload, per_segment: int, seed: int = 0, edge: int = 64) -> list:
    """Global query rows to compare: all rows of a segment when it has at most
    `per_segment`; otherwise its first and last `edge` rows plus
    `per_segment - 2*edge` distinct rows drawn from the rest (CPU generator,
    one generator for all segments, segments in order)."""
    g = torch.Generator().manual_seed(seed)
    rows = []
    for b in range(w.num_segments):
        a, e = w.cu_q[b], w.cu_q[b + 1]
        n = e - a
        if n <= per_segment:
            rows.extend(range(a, e))
            continue
        ed = min(edge, per_segment // 2)
        mid = n - 2 * ed
        pick = torch.randperm(mid, generator=g)[: per_segment - 2 * ed] + (a + ed)
        rows.extend(range(a, a + ed))
        rows.extend(sorted(int(x) for x in pick))
        rows.extend(range(e - ed, e))
    return rows


def make_dout(w: Workload, device="cuda", seed: int = 1, outer_stride: int = 0):
    """Upstream gradient dout for the backward: bf16 N(0,1)*std drawn from its
    own generator (seed `seed`). With outer_stride > 0 it is the [total_q, H, D]
    view of columns [0, H*D) of an [total_q, outer_stride] buffer, the layout
    a cat([attn_out, other], dim=1) hands to the attention backward (row
    stride H*D + other width, 9728 on the _bwd_preprocess page); otherwise
    contiguous. Returns (dout, base buffer)."""
    H, D = w.num_heads, w.head_dim
    n = w.total_q
    g = _generator(device, seed)
    if outer_stride:
        if outer_stride < H * D:
            raise ValueError("outer stride smaller than H*D")
        base = torch.empty((n, outer_stride), dtype=torch.bfloat16, device=device)
        base.normal_(generator=g)
        base.mul_(w.std)
        return base[:, : H * D].view(n, H, D), base
    d = torch.randn((n, H, D), dtype=torch.bfloat16, device=device, generator=g)
    if w.std != 1.0:
        d.mul_(w.std)
    return d, d
