"""Host-side tests of libattn_varlen.so: exported symbols, argument checks,
64-bit offset arithmetic and the exact tile plan. No GPU needed: nothing here
launches a kernel or touches device memory.
"""
import ctypes
import json
import math
import random
import re
from pathlib import Path

import pytest

import varlen_flashattention_forward_amd as avf
from varlen_flashattention_forward_amd import _binding
from varlen_flashattention_forward_amd.workloads import WORKLOADS

ROOT = Path(__file__).resolve().parents[1]
GOLDEN = json.loads((ROOT / "tests" / "golden" / "pages_integers.json").read_text())


@pytest.fixture(scope="module", autouse=True)
def built():
    if not _binding.LIB_PATH.exists():
        from varlen_flashattention_forward_amd import build
        build.build()
    avf.lib()


def header_functions():
    text = (ROOT / "include" / "attn_varlen.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_(?:varlen|fwd)_?\w*)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(str(_binding.LIB_PATH))
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/attn_varlen.h but not exported"
    assert sorted(_binding.EXPORTED_SYMBOLS) == names


# ------------------------------------------------------------ 64-bit offsets (pages' numbers)

def test_offset_matches_pages_verified_sample():
    g = GOLDEN["offset_wrap"]
    off = avf.element_offset(g["coord"], g["row_stride"], 0, 0)
    assert off == g["true_offset"] == 2_191_757_312
    # what an int32 accumulator would have produced, per the page, is not what we form
    wrapped = (off + 2**31) % 2**32 - 2**31
    assert wrapped == g["offset_as_signed_i32"]
    assert wrapped % 2**64 == g["offset_sign_extended_u64"]
    assert off != wrapped
    parts = g["row_stride_parts"]
    assert parts["heads"] * parts["head_dim"] + parts["mlp_dim"] == g["row_stride"]


def test_offset_threshold_and_largest_strided_offset():
    g = GOLDEN["offset_wrap"]
    t = g["wrap_threshold_approx"]
    assert avf.element_offset(t, g["row_stride"], 0, 0) >= 2**31
    assert avf.element_offset(t - 1, g["row_stride"], 0, 0) < 2**31
    # last element of the strided layout: row N-1, head 15, plus the 3rd slice (v) offset
    n = g["total_tokens"]
    last = avf.element_offset(n - 1, 9728, 15, 96) + 2 * 1536 + 95
    assert last == (n - 1) * 9728 + 15 * 96 + 3072 + 95
    assert last * 2 > 2**32          # byte offsets past 2^32 as well
    # head offsets combine in 64 bits too
    assert avf.element_offset(3, 1 << 22, (1 << 31) - 1, 1 << 22) == 3 * (1 << 22) + ((1 << 31) - 1) * (1 << 22)


# ------------------------------------------------------------ exact tile accounting

def test_tile_count_matches_pages_valid_tiles():
    g = GOLDEN["varlen_grid"]
    assert avf.count_tiles(g["cu_seqlens_q"], g["num_heads"], g["tile_m"]) == g["valid_tiles"]
    # the variant with every middle window 5040 rows has the same count
    cu2 = list(g["cu_seqlens_q"])
    cu2[5] = 24192
    assert avf.count_tiles(cu2, g["num_heads"], g["tile_m"]) == g["valid_tiles"]


def test_our_grid_is_exact_for_every_workload():
    for w in WORKLOADS.values():
        bm = avf.block_m(w.head_dim, w.max_seqlen_k)
        # segments of at most one K/V stage take the one-stage configuration (128-row tiles)
        assert bm == (128 if w.max_seqlen_k <= avf.short_stage_keys() else avf.block_m(w.head_dim))
        exact = w.num_heads * sum(math.ceil((b - a) / bm) for a, b in zip(w.cu_q[:-1], w.cu_q[1:]))
        launches, wgs = avf.grid_plan(w.cu_q, w.num_heads, w.head_dim, w.max_seqlen_k)
        assert wgs == exact == avf.count_tiles(w.cu_q, w.num_heads, bm)
        assert launches == 1


def test_num_tiles_is_the_exact_grid_of_a_call():
    for w in WORKLOADS.values():
        _, wgs = avf.grid_plan(w.cu_q, w.num_heads, w.head_dim, w.max_seqlen_k)
        assert avf.num_tiles(w.cu_q, w.num_heads, w.head_dim, w.max_seqlen_k) == wgs
    # the SM120 page's cu_seqlens_q at 56 heads: 15680 valid tiles at tile_m = 128,
    # which a call with at most 512 keys per segment (128-row tiles) launches exactly
    g = GOLDEN["varlen_grid"]
    assert avf.block_m(128, 512) == g["tile_m"]
    assert avf.num_tiles(g["cu_seqlens_q"], g["num_heads"], 128, 512) == g["valid_tiles"]
    assert avf.num_tiles(g["cu_seqlens_q"], g["num_heads"], 128, 17580) == \
        avf.count_tiles(g["cu_seqlens_q"], g["num_heads"], avf.block_m(128))
    assert avf.num_tiles([0], 56, 128, 1000) == 0
    for bad, code in (([1, 5], _binding.ECU), ([0, 5, 4], _binding.ECU)):
        with pytest.raises(avf.AttnVarlenError) as e:
            avf.num_tiles(bad, 2, 128, 100)
        assert e.value.code == code
    with pytest.raises(avf.AttnVarlenError):
        avf.num_tiles([0, 5], 2, 80, 100)


def test_oversized_segment_is_rejected_before_any_launch():
    # The second segment alone needs 2^23 tiles (over the per-launch limit);
    # the first is small. Every entry point must refuse the call before any
    # HIP call, so no launch for the first segment (or fp8 quantization, or
    # backward preprocessing) is left queued. Without a GPU here, a HIP call
    # would have returned EHIP instead.
    H, D, n = 8, 128, 1 << 28
    cq = [0, 1, 1 + n]
    lay = layout(H=H, D=D, nq=1 + n, nk=1 + n)
    assert v(cu_q=cq, cu_k=cq, H=H, D=D, max_q=n, max_k=n, lay=lay) == _binding.EUNSUPPORTED
    L = avf.lib()
    c = (ctypes.c_int32 * 3)(*cq)
    rc = L.attn_varlen_fwd_hostcu(P, P, P, c, c, 2, H, D, n, n, ctypes.byref(lay), 0.125, P, P, None)
    assert rc == _binding.EUNSUPPORTED, avf.last_error()
    big = 1 << 40
    rc = L.attn_varlen_fwd_fp8_hostcu(P, P, P, c, c, 2, H, D, n, n, ctypes.byref(lay), 0.125, 0, P, big, P, P, None)
    assert rc == _binding.EUNSUPPORTED, avf.last_error()
    bl = bwd_layout(H=H, D=D, nq=1 + n, nk=1 + n)
    rc = L.attn_varlen_bwd_hostcu(P, P, P, P, P, P, c, c, 2, H, D, n, n, ctypes.byref(bl), 0.125, 0, P, P, P, P,
                                  None)
    assert rc == _binding.EUNSUPPORTED, avf.last_error()


def test_grid_plan_splits_long_segment_lists():
    spl = avf.segments_per_launch()
    rng = random.Random(0)
    lens = [rng.choice([0, 1, 7, 64, 255, 256, 257, 1000]) for _ in range(3 * spl + 5)]
    cu = [0]
    for x in lens:
        cu.append(cu[-1] + x)
    for max_k in (max(lens), 512, 128):
        launches, wgs = avf.grid_plan(cu, 3, 128, max_k)
        bm = avf.block_m(128, max_k)
        assert bm == (avf.block_m(128) if max_k > 512 else 128)
        assert wgs == 3 * sum(math.ceil(x / bm) for x in lens)
        assert launches == math.ceil(len(lens) / spl)


def test_grid_plan_keeps_each_launch_below_2_to_32_work_items():
    # eight-wave workgroups (512 threads): a launch holds at most 2^23 - 1
    # tiles. Two segments of 2^27 rows at H = 8 and 256-row tiles make 2^23
    # tiles, so they take two launches; a segment that alone needs more tiles
    # than one launch holds is rejected.
    bm = avf.block_m(128)
    assert bm == 256
    n = 1 << 27
    launches, wgs = avf.grid_plan([0, n, 2 * n], 8, 128, n)
    assert wgs == 2 * 8 * (n // bm) == 1 << 23
    assert launches == 2
    launches, wgs = avf.grid_plan([0, n - bm, 2 * n - bm], 8, 128, n)
    assert wgs == (1 << 23) - 8 and launches == 1
    with pytest.raises(avf.AttnVarlenError) as e:
        avf.grid_plan([0, 2 * n], 16, 128, 2 * n)
    assert e.value.code == _binding.EUNSUPPORTED


@pytest.mark.parametrize("seed", range(6))
def test_decode_is_a_bijection_onto_valid_tiles(seed):
    rng = random.Random(seed)
    B = rng.randint(1, avf.segments_per_launch())
    H = rng.choice([1, 2, 3, 8, 56])
    bm = rng.choice([64, 128, 256])
    cu = [0]
    for _ in range(B):
        cu.append(cu[-1] + rng.choice([0, 0, 1, bm - 1, bm, bm + 1, rng.randint(1, 5 * bm)]))
    T = avf.count_tiles(cu, H, bm)
    seen = set()
    for wg in range(T):
        s, m, h = avf.decode_tile(cu, H, bm, wg)
        lq = cu[s + 1] - cu[s]
        assert lq > 0 and 0 <= m < math.ceil(lq / bm) and 0 <= h < H
        seen.add((s, m, h))
    assert len(seen) == T
    if T:
        with pytest.raises(avf.AttnVarlenError):
            avf.decode_tile(cu, H, bm, T)   # no workgroup beyond the exact grid


def test_first_block_past_the_pages_grid_is_outside_ours():
    g = GOLDEN["varlen_grid"]
    with pytest.raises(avf.AttnVarlenError):
        avf.decode_tile(g["cu_seqlens_q"], g["num_heads"], g["tile_m"], g["first_faulting_block"])
    avf.decode_tile(g["cu_seqlens_q"], g["num_heads"], g["tile_m"], g["first_faulting_block"] - 1)


# ------------------------------------------------------------ argument checks (no HIP calls)

P = 1 << 20  # a 16-byte-aligned fake address; validate never dereferences it


def layout(H=2, D=64, nq=10, nk=12, **kw):
    base = dict(q_row=H * D, q_head=D, k_row=H * D, k_head=D, v_row=H * D, v_head=D,
                o_row=H * D, o_head=D, lse_head=0, q_tokens=nq, k_tokens=nk)
    base.update(kw)
    return _binding.Layout(**base)


def v(cu_q=(0, 4, 10), cu_k=(0, 5, 12), H=2, D=64, max_q=6, max_k=7, lay=None, scale=0.125,
      q=P, k=P, vv=P, out=P, lse=P):
    lay = lay or layout(H, D)
    return avf.validate(q, k, vv, list(cu_q), list(cu_k), H, D, max_q, max_k, lay, scale, out, lse)


def test_validate_accepts_good_arguments():
    assert v() == 0
    assert v(lse=None) == 0
    assert v(D=96, lay=layout(D=96)) == 0 and v(D=128, lay=layout(D=128)) == 0
    # strided view of a wider buffer (row stride 9728, head stride 96)
    lay = layout(H=16, D=96, q_row=9728, q_head=96, k_row=9728, k_head=96, v_row=9728, v_head=96,
                 o_row=9728, o_head=96)
    assert v(H=16, D=96, lay=lay) == 0
    # [H, S, D] layout: head stride larger than row stride
    lay = layout(q_row=64, q_head=640, k_row=64, k_head=768, v_row=64, v_head=768, o_row=64, o_head=640)
    assert v(lay=lay) == 0
    # empty segments are fine, B = 0 is a no-op
    assert v(cu_q=(0, 0, 10), cu_k=(0, 5, 5), max_q=10) == 0
    assert avf.validate(None, None, None, [0], [0], 2, 64, 0, 0, layout(), 0.125, None, None) == 0


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), _binding.ENULL),
    (dict(out=None), _binding.ENULL),
    (dict(H=0), _binding.EINVAL),
    (dict(D=80, lay=layout(D=80)), _binding.EUNSUPPORTED),
    (dict(D=256, lay=layout(D=256)), _binding.EUNSUPPORTED),
    (dict(scale=0.0), _binding.EINVAL),
    (dict(scale=-1.0), _binding.EINVAL),
    (dict(scale=float("nan")), _binding.EINVAL),
    (dict(scale=float("inf")), _binding.EINVAL),
    (dict(q=P + 8), _binding.EALIGN),
    (dict(out=P + 2), _binding.EALIGN),
    (dict(lse=P + 2), _binding.EALIGN),
    (dict(lay=layout(k_row=132)), _binding.EALIGN),
    (dict(lay=layout(v_head=60)), _binding.EALIGN),
    (dict(lay=layout(q_row=0)), _binding.EINVAL),
    (dict(lay=layout(o_head=-64)), _binding.EINVAL),
    (dict(lay=layout(k_row=(1 << 22) + 8)), _binding.EUNSUPPORTED),
    (dict(cu_q=(1, 4, 10)), _binding.ECU),
    (dict(cu_k=(0, 6, 5)), _binding.ECU),
    (dict(cu_q=(0, 4, 11), max_q=7), _binding.ECU),   # past q_tokens = 10
    (dict(cu_k=(0, 5, 13), max_k=8), _binding.ECU),   # past k_tokens = 12
    (dict(max_q=5), _binding.EMAXSEQ),
    (dict(max_k=6), _binding.EMAXSEQ),
    (dict(max_q=-1), _binding.EINVAL),
    (dict(lay=layout(o_row=64, o_head=64)), _binding.EINVAL),      # out rows and heads alias
    (dict(lay=layout(o_row=120, o_head=64)), _binding.EINVAL),     # rows overlap within a head
    (dict(lay=layout(lse_head=8)), _binding.EINVAL),               # lse heads overlap
    (dict(lay=layout(o_head=0)), _binding.EINVAL),                 # every head writes the same out elements
])
def test_validate_rejects(kwargs, code):
    rc = v(**kwargs)
    assert rc == code, (rc, avf.last_error())
    assert avf.last_error()


def test_validate_never_needs_lse_head_with_one_head():
    assert v(H=1, lay=layout(H=1, lse_head=1)) == 0


def test_block_m_and_unsupported_dims():
    assert avf.one_stage_keys() == 128 and avf.short_stage_keys() == 512
    for d in (64, 96, 128):
        bm = avf.block_m(d)
        assert bm > 0 and bm % 32 == 0
        # max_seqlen_k picks the configuration: one stage up to 128 keys
        assert avf.block_m(d, 0) == avf.block_m(d, 1) == avf.block_m(d, 128) == 128
        assert avf.block_m(d, 129) == avf.block_m(d, 512) == 128
        assert avf.block_m(d, 513) == avf.block_m(d, 1 << 30) == bm
        with pytest.raises(avf.AttnVarlenError, match="EINVAL"):
            avf.block_m(d, -1)
    with pytest.raises(avf.AttnVarlenError):
        avf.block_m(100)
    with pytest.raises(avf.AttnVarlenError):
        avf.block_m(100, 64)


def test_forward_rejects_cpu_tensors_before_any_hip_call():
    import torch
    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        avf.attn_varlen_fwd(q, q, q, cu, cu, 4, 4)
    # the sync-free and 8-bit front ends check the same before marshalling
    with pytest.raises(ValueError, match="device tensors"):
        avf.attn_varlen_fwd_async(q, q, q, cu, cu, 4, 4, workspace=torch.zeros(64, dtype=torch.int32))
    with pytest.raises(ValueError, match="device tensors"):
        avf.attn_varlen_fwd_fp8(q, q, q, cu, cu, 4, 4, workspace=torch.zeros(1 << 12, dtype=torch.uint8))


# ------------------------------------------------------------ option flags and the batched entry

def test_validate_ex_flags():
    cq, ck = [0, 6, 10], [0, 5, 12]
    args = (P, P, P, cq, ck, 2, 64, 6, 7, layout(), 0.125, P, P)
    assert avf.validate(*args, flags=0) == 0
    assert avf.validate(*args, flags=_binding.CAUSAL) == 0
    assert avf.validate(*args, flags=2) == _binding.EINVAL
    assert avf.validate(*args, flags=_binding.CAUSAL | 4) == _binding.EINVAL


def blayout(W=3, Sq=5, Sk=7, H=2, D=64, **kw):
    """Contiguous [W, S, H, D] strides and [W, H, Sq] LSE, overridable."""
    d = dict(q_batch=Sq * H * D, q_row=H * D, q_head=D, k_batch=Sk * H * D, k_row=H * D, k_head=D,
             v_batch=Sk * H * D, v_row=H * D, v_head=D, o_batch=Sq * H * D, o_row=H * D, o_head=D,
             lse_batch=H * Sq, lse_head=Sq)
    d.update(kw)
    return avf.BatchedLayout(**d)


def vb(W=3, Sq=5, Sk=7, H=2, D=64, lay=None, flags=0, q=P, out=P, lse=P, scale=0.125):
    lay = lay if lay is not None else blayout(W, Sq, Sk, H, D)
    return avf.validate_batched(q, P, P, W, Sq, Sk, H, D, lay, scale, flags, out, lse)


def test_batched_validate_accepts():
    assert vb() == 0
    assert vb(flags=_binding.CAUSAL) == 0
    assert vb(lse=None) == 0
    assert vb(W=0) == 0 and vb(Sq=0) == 0 and vb(Sk=0) == 0
    # [S, W, H, D] storage seen as [W, S, H, D]: batch stride H*D, row stride W*H*D
    W, S, H, D = 4, 9, 2, 96
    lay = blayout(W, S, S, H, D, q_batch=H * D, q_row=W * H * D, k_batch=H * D, k_row=W * H * D,
                  v_batch=H * D, v_row=W * H * D, o_batch=H * D, o_row=W * H * D)
    assert vb(W, S, S, H, D, lay=lay) == 0


@pytest.mark.parametrize("kwargs,code", [
    (dict(W=-1), _binding.EINVAL),
    (dict(Sq=-2), _binding.EINVAL),
    (dict(flags=8), _binding.EINVAL),
    (dict(q=None), _binding.ENULL),
    (dict(q=P + 4), _binding.EALIGN),
    (dict(lay=blayout(q_batch=5 * 2 * 64 + 4)), _binding.EALIGN),   # batch stride not a multiple of 8
    (dict(lay=blayout(k_batch=-128)), _binding.EINVAL),
    (dict(lay=blayout(o_batch=4 * 2 * 64)), _binding.EINVAL),       # out batches overlap
    (dict(lay=blayout(lse_batch=5)), _binding.EINVAL),              # lse batches overlap
    (dict(lay=blayout(lse_head=3)), _binding.EINVAL),               # lse heads overlap
    (dict(lay=blayout(lse_head=0)), _binding.EINVAL),               # both heads write one lse row
    (dict(lay=blayout(o_head=0)), _binding.EINVAL),                 # both heads write one out row
    (dict(lay=blayout(lse_batch=0)), _binding.EINVAL),              # every batch writes one lse block
    (dict(W=1 << 20, Sq=1 << 12), _binding.EUNSUPPORTED),           # W * Sq >= 2^31
    (dict(D=80, lay=blayout(D=80)), _binding.EUNSUPPORTED),
])
def test_batched_validate_rejects(kwargs, code):
    assert vb(**kwargs) == code


def test_zero_strides_are_fine_where_the_extent_is_one():
    # one head: its stride never matters (the LSE and out rows cannot collide)
    assert vb(H=1, lay=blayout(H=1, lse_head=0, o_head=0)) == 0
    assert v(H=1, lay=layout(H=1, o_head=0)) == 0
    # one batch: the batch strides never matter
    assert vb(W=1, lay=blayout(W=1, lse_batch=0, o_batch=0)) == 0


# ---------------------------------------------------------------- backward (host checks only)

def bwd_layout(H=2, D=64, nq=10, nk=12, **kw):
    hd = H * D
    base = dict(q_row=hd, q_head=D, k_row=hd, k_head=D, v_row=hd, v_head=D, o_row=hd, o_head=D,
                do_row=hd, do_head=D, dq_row=hd, dq_head=D, dk_row=hd, dk_head=D, dv_row=hd, dv_head=D,
                lse_head=0, delta_head=0, q_tokens=nq, k_tokens=nk)
    base.update(kw)
    return _binding.BwdLayout(**base)


def vb_bwd(cu_q=(0, 4, 10), cu_k=(0, 5, 12), H=2, D=64, max_q=6, max_k=7, lay=None, scale=0.125, flags=0,
           ptrs=None, **repl):
    names = ("q", "k", "v", "out", "dout", "lse", "delta", "dq", "dk", "dv")
    p = dict(zip(names, [P] * 10))
    p.update(ptrs or {})
    return avf.validate_bwd(tuple(p[n] for n in names), list(cu_q), list(cu_k), H, D, max_q, max_k,
                            lay or bwd_layout(H, D, **repl), scale, flags)


def test_bwd_validate_accepts():
    assert vb_bwd() == 0
    assert vb_bwd(flags=avf.CAUSAL) == 0
    assert vb_bwd(D=96, lay=bwd_layout(D=96)) == 0
    # the page's dout view: row stride 9728
    assert vb_bwd(H=16, D=96, lay=bwd_layout(H=16, D=96, do_row=9728, do_head=96)) == 0
    assert vb_bwd(cu_q=(0,), cu_k=(0,)) == 0  # no segments


@pytest.mark.parametrize("kwargs,code", [
    (dict(ptrs={"dout": None}), _binding.ENULL),
    (dict(ptrs={"delta": None}), _binding.ENULL),
    (dict(ptrs={"dk": None}), _binding.ENULL),
    (dict(ptrs={"dq": P + 8}), _binding.EALIGN),
    (dict(ptrs={"lse": P + 2}), _binding.EALIGN),
    (dict(do_row=100), _binding.EALIGN),
    (dict(dq_row=0), _binding.EINVAL),
    (dict(dk_head=-8), _binding.EINVAL),
    (dict(dv_row=8, dv_head=8), _binding.EINVAL),            # dv rows overlap
    (dict(dq_head=0), _binding.EINVAL),                      # both heads write one dq row
    (dict(dk_head=0), _binding.EINVAL),
    (dict(dv_head=0), _binding.EINVAL),
    (dict(delta_head=8), _binding.EINVAL),                   # delta rows of head 1 overlap head 0
    (dict(lse_head=4), _binding.EINVAL),
    (dict(do_row=1 << 23), _binding.EUNSUPPORTED),
    (dict(D=80), _binding.EUNSUPPORTED),
    (dict(flags=2), _binding.EINVAL),
    (dict(nq=9), _binding.ECU),                              # cu ends past q_tokens
    (dict(cu_k=(0, 5, 4)), _binding.ECU),                   # decreasing
    (dict(max_k=4), _binding.EMAXSEQ),
    (dict(scale=0.0), _binding.EINVAL),
])
def test_bwd_validate_rejects(kwargs, code):
    D = kwargs.pop("D", 64)
    assert vb_bwd(D=D, **kwargs) == code


def test_bwd_grid_plan_counts_key_and_row_blocks():
    pre, dkdv, dq, launches = avf.bwd_grid_plan([0, 225304, 410923], [0, 225304, 410923], 16, 96)
    assert pre == 410923 * 16 // 16
    assert dkdv == 16 * (math.ceil(225304 / 128) + math.ceil(185619 / 128)) == dq
    assert launches == 2
    # cross attention: dK/dV tiles follow the key lengths, dQ tiles the query lengths
    pre, dkdv, dq, launches = avf.bwd_grid_plan([0, 5, 5, 300], [0, 0, 7, 7], 3, 128)
    assert (dkdv, dq) == (3 * 1, 3 * (1 + 3)) and pre == math.ceil(300 * 3 / 16)


def test_bwd_preprocess_rejects_before_any_hip_call():
    L = avf.lib()
    assert L.attn_varlen_bwd_preprocess(P, None, 10, 2, 64, 128, 64, 128, 64, P, 10, None) == _binding.ENULL
    assert L.attn_varlen_bwd_preprocess(P, P, 10, 2, 64, 128, 64, 128, 64, P, 5, None) == _binding.EINVAL
    assert L.attn_varlen_bwd_preprocess(P, P, 10, 2, 80, 128, 64, 128, 64, P, 10, None) == _binding.EUNSUPPORTED
    assert L.attn_varlen_bwd_preprocess(P, P, 0, 2, 64, 128, 64, 128, 64, P, 10, None) == 0  # no rows


# ---------------------------------------------------------------- sync-free forward (host side)

@pytest.mark.parametrize("seed", range(5))
def test_async_grid_bounds_the_tile_count(seed):
    """The host-only grid covers every tile for any cu consistent with
    q_tokens and max_seqlen_q (or loops over them at the cap)."""
    rng = random.Random(seed)
    for _ in range(50):
        B = rng.randint(1, 300)
        lens = [rng.choice([0, 1, rng.randint(1, 3000)]) for _ in range(B)]
        cu = [0]
        for x in lens:
            cu.append(cu[-1] + x)
        H, D = rng.choice([1, 3, 56]), rng.choice([64, 96, 128])
        q_tokens = cu[-1] + rng.randint(0, 500)
        max_q = max(lens) + rng.randint(0, 100)
        max_k = rng.choice([0, 64, 128, 129, 5000])
        bm = avf.block_m(D, max_k)
        tiles = avf.count_tiles(cu, H, bm)
        g = avf.async_grid(q_tokens, B, H, D, max_q, max_k)
        assert g % 8 == 0 and g <= 8192
        assert g >= min(tiles, 8192)
        bound = H * min(math.ceil((q_tokens + B * (bm - 1)) / bm), B * math.ceil(max_q / bm))
        assert tiles <= bound and g == min(8192, -(-bound // 8) * 8)


def test_async_workspace_bytes():
    assert avf.async_workspace_bytes(0) == 256
    assert avf.async_workspace_bytes(2) == 256
    assert avf.async_workspace_bytes(1000) == -(-(4 * (4 + 1001)) // 256) * 256
    with pytest.raises(avf.AttnVarlenError):
        avf.async_workspace_bytes(-1)


def test_async_rejects_host_errors_before_any_hip_call():
    L = avf.lib()
    lay = layout()
    cq = P
    args = lambda ws, nbytes, flags=0: (P, P, P, cq, cq, 2, 2, 64, 6, 7, ctypes.byref(lay), 0.125, flags, ws, nbytes,
                                        P, P, None)
    assert L.attn_varlen_fwd_async(*args(None, 256)) == _binding.ENULL
    assert L.attn_varlen_fwd_async(*args(P + 4, 256)) == _binding.EALIGN
    assert L.attn_varlen_fwd_async(*args(P, 16)) == _binding.EINVAL
    assert L.attn_varlen_fwd_async(*args(P, 256, flags=4)) == _binding.EINVAL
    lay_bad = layout(o_row=8, o_head=8)
    bad = (P, P, P, cq, cq, 2, 2, 64, 6, 7, ctypes.byref(lay_bad), 0.125, 0, P, 256, P, P, None)
    assert L.attn_varlen_fwd_async(*bad) == _binding.EINVAL


# ---------------------------------------------------------------- low-precision forward (host side)

def test_fp8_workspace_layout():
    q8, k8 = avf.fp8_workspace_offsets(100, 120, 2, 64)
    assert (q8, k8) == (256, 256 + 100 * 2 * 64)
    assert avf.fp8_workspace_bytes(100, 120, 2, 64) == k8 + -(-(120 * 2 * 64) // 256) * 256
    # sizes past 2^31 bytes are fine (64-bit arithmetic throughout)
    big = avf.fp8_workspace_bytes(410923, 410923, 56, 128)
    assert big == 512 + 2 * (-(-(410923 * 56 * 128) // 256) * 256) and big > 2 ** 32  # 2*56 amax words -> 512
    for D in (96, 80):
        with pytest.raises(avf.AttnVarlenError):
            avf.fp8_workspace_bytes(10, 10, 2, D)


def test_fp8_rejects_host_errors_before_any_hip_call():
    L = avf.lib()
    lay = layout()
    cq = (ctypes.c_int32 * 3)(0, 4, 10)
    ck = (ctypes.c_int32 * 3)(0, 5, 12)
    W = 1 << 20  # 256-byte aligned fake workspace address
    def call(D=64, ws=W, nbytes=1 << 20, lay_=lay, flags=0):
        return L.attn_varlen_fwd_fp8_hostcu(P, P, P, cq, ck, 2, 2, D, 6, 7, ctypes.byref(lay_), 0.125, flags, ws,
                                            nbytes, P, P, None)
    assert call(D=96, lay_=layout(D=96)) == _binding.EUNSUPPORTED
    assert call(ws=None) == _binding.ENULL
    assert call(ws=W + 16) == _binding.EALIGN
    assert call(nbytes=100) == _binding.EINVAL
    assert call(flags=8) == _binding.EINVAL


def test_bench_roofline_bound_follows_the_ridge():
    """bench.py reports MFMA-bound TFLOP/s at or above the ridge (2.5 PFLOP/s
    over 8 TB/s = 312.5 flop/B) and HBM-bound GB/s of algorithmic bytes below it."""
    import bench
    d = WORKLOADS["dense_77k"]
    r = bench.roofline_of(d.flops(), d.algorithmic_bytes(), 137.5, bench.PEAK_BF16_TFLOPS)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["achieved"] - d.flops() / 0.1375 / 1e12) < 0.01
    s = WORKLOADS["short_128"]
    r = bench.roofline_of(s.flops(), s.algorithmic_bytes(), 0.116, bench.PEAK_BF16_TFLOPS)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - s.algorithmic_bytes() / 0.116e-3 / 1e9) < 0.1
    assert bench.roofline_of(312_500, 1000, 1.0, 2500.0)["bound"] == "mfma"
    assert bench.roofline_of(312_499, 1000, 1.0, 2500.0)["bound"] == "hbm"


def test_bench_kernel_hash_ignores_comments(tmp_path, monkeypatch):
    """The key of the committed HBM counters follows the kernel's code, not
    its comments."""
    import shutil
    import bench
    for p in bench.KERNEL_SOURCES:
        (tmp_path / p).parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(ROOT / p, tmp_path / p)
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    h0 = bench.kernel_hash()
    src = tmp_path / bench.KERNEL_SOURCES[0]
    src.write_text("// a new comment line\n\n" + src.read_text().replace("\n", "  // trailing note\n", 1))
    assert bench.kernel_hash() == h0
    src.write_text(src.read_text() + "\nstatic int avf_extra_code;\n")
    assert bench.kernel_hash() != h0


def test_probe_library_exports_and_rejects_bad_arguments():
    """The calibration library (bench.py --mfma-rate / --coissue) loads and
    rejects bad arguments before any HIP call."""
    import ctypes

    from varlen_flashattention_forward_amd import build as avf_build

    if not avf_build.PROBE_LIB.exists():
        pytest.skip("probe library not built")
    P = ctypes.CDLL(str(avf_build.PROBE_LIB))
    P.avf_probe_coissue.restype = ctypes.c_int32
    P.avf_probe_coissue.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p]
    P.avf_probe_mfma.restype = ctypes.c_int32
    P.avf_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    fake = ctypes.c_void_p(4096)
    assert P.avf_probe_coissue(5, 0, fake, 1, 1, None) == -2    # not an instantiated variant
    assert P.avf_probe_coissue(4, 0, None, 1, 1, None) == -2    # no output buffer
    assert P.avf_probe_coissue(4, 0, fake, 0, 1, None) == -2    # no workgroups
    assert P.avf_probe_mfma(fake, fake, 1, 3, None) == -2       # odd iteration count
    assert P.avf_probe_mfma(ctypes.c_void_p(4097), fake, 1, 2, None) == -2  # misaligned operands


def test_mfma_rate_operand_patterns():
    """bench.py --mfma-rate operand patterns have the layout the probe kernel
    reads: per wave 8 fragments of 512 bf16, A = fragments 0-3, B = 4-7."""
    import torch

    import bench

    n = 2 * 8 * 512
    g = torch.Generator().manual_seed(0)
    for mode in bench.MFMA_OPERANDS:
        x = bench.mfma_operands(mode, n, "cpu", torch.Generator().manual_seed(0))
        assert x.dtype == torch.bfloat16 and x.numel() == n, mode
    x = bench.mfma_operands("lane-constant", n, "cpu", g).view(-1, 8, 512)
    assert torch.equal(x, x[:, :, :1].expand_as(x)) and x[:, :, 0].unique().numel() > 1
    x = bench.mfma_operands("a-random-b-ones", n, "cpu", g).view(-1, 8, 512)
    assert bool((x[:, 4:] == 1).all()) and x[:, :4].unique().numel() > 100
    x = bench.mfma_operands("a-ones-b-random", n, "cpu", g).view(-1, 8, 512)
    assert bool((x[:, :4] == 1).all()) and x[:, 4:].unique().numel() > 100
    x = bench.mfma_operands("uniform", n, "cpu", g)
    assert float(x.min()) >= 0.0 and float(x.max()) <= 1.0
