"""Pins of the low-precision oracle (oracle/fp8_oracle.py): the E4M3 format
against torch's float8_e4m3fn (a library routine), closed forms of the
format, the per-head scaling, and the reduction to exact attention when the
inputs are exactly representable. Planted mistakes must trip a pin.

All CPU; no GPU needed.
"""
import numpy as np
import pytest
import torch

from oracle import blas_oracle
from oracle import fp8_oracle as F


def to_bf16_bits(x) -> np.ndarray:
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def pin_decode_table(M):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = M.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def pin_encode_library(M):
    rng = np.random.default_rng(0)
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    vals = np.unique(vals[np.isfinite(vals) & (vals >= 0)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)          # exact ties
    x = np.concatenate([rng.standard_normal(20000) * 60, rng.standard_normal(20000) * 0.004,
                        rng.uniform(-448, 448, 20000), mids, -mids, vals, -vals]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(M.e4m3_encode(x), ref)


def pin_encode_closed_forms(M):
    x = np.float32([448.0, 1.0, 2.0 ** -9, 2.0 ** -6, -1.5, 0.0, 2.0 ** -10, 3 * 2.0 ** -10, 448.0 * (1 + 2.0 ** -23)])
    assert list(M.e4m3_encode(x)) == [0x7E, 0x38, 0x01, 0x08, 0xBC, 0x00, 0x00, 0x02, 0x7E]


def pin_per_head_scaling(M):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((300, 3, 64)).astype(np.float32)
    x[:, 1] *= 0.001           # heads with very different ranges
    x[:, 2] = 0.0              # an all-zero head
    b = to_bf16_bits(x)
    codes, scale, inv = M.quantize_per_head(b)
    xf = (b.astype(np.uint32) << 16).view(np.float32)
    for h in (0, 1):
        amax = np.abs(xf[:, h]).max()
        assert scale[h] == np.float32(amax / np.float32(448)) and inv[h] == np.float32(np.float32(448) / amax)
        i = np.unravel_index(np.abs(xf[:, h]).argmax(), xf[:, h].shape)
        assert codes[:, h][i] & 0x7F == 0x7E             # the head's largest element becomes +-448
        deq = M.e4m3_decode(codes[:, h]) * scale[h]
        big = np.abs(xf[:, h]) >= amax * 2.0 ** -6 / 448 * 8   # normal range of the format
        assert np.all(np.abs(deq - xf[:, h])[big] <= 2.0 ** -4 * np.abs(xf[:, h])[big] * (1 + 1e-6))
    assert scale[2] == 1 and inv[2] == 0 and not codes[:, 2].any()


def pin_exact_when_representable(M):
    """Inputs that are E4M3 values times a power of two, with each head's
    largest magnitude at 448 * 2^j: quantization is exact, so the result is
    exact attention on the inputs (compared with the bf16 fp64 oracle)."""
    rng = np.random.default_rng(2)
    cu_q, cu_k = [0, 37, 100], [0, 50, 120]
    H, D = 2, 32
    vals = M.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8))
    def draw(n, pw):
        c = rng.choice(vals[vals <= 64], size=(n, H, D)) * rng.choice([-1, 1], size=(n, H, D))
        c[0, :, 0] = 448.0
        return (c * 2.0 ** pw).astype(np.float32)
    q, k = to_bf16_bits(draw(100, -7)), to_bf16_bits(draw(120, -9))
    v = to_bf16_bits(rng.standard_normal((120, H, D)))
    o8, l8 = M.attn_varlen_fwd_fp8(q, k, v, cu_q, cu_k, 0.3)
    o, l = blas_oracle.attn_varlen_fwd(q, k, v, cu_q, cu_k, 0.3)
    assert np.array_equal(o8, o) and np.array_equal(l8, l)


def pin_quantized_attention_error(M):
    """On Gaussian inputs the quantized result stays close to exact attention
    (the per-element E4M3 error is at most 2^-4 relative)."""
    rng = np.random.default_rng(3)
    cu = [0, 200]
    q, k, v = (to_bf16_bits(rng.standard_normal((200, 2, 64))) for _ in range(3))
    o8, l8 = M.attn_varlen_fwd_fp8(q, k, v, cu, cu, 0.125)
    o, l = blas_oracle.attn_varlen_fwd(q, k, v, cu, cu, 0.125)
    cos = (o8 * o).sum() / np.sqrt((o8 * o8).sum() * (o * o).sum())
    assert 0.99 < cos < 1.0 and np.abs(l8 - l).max() < 0.2


PINS = [pin_decode_table, pin_encode_library, pin_encode_closed_forms, pin_per_head_scaling,
        pin_exact_when_representable, pin_quantized_attention_error]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_fp8_oracle_pin(pin):
    pin(F)


class _Mutant:
    """The oracle's steps with some replaced; the unreplaced ones are the
    oracle's own (quantization re-expressed through the mutant's encoder)."""
    def __init__(self, **repl):
        self.e4m3_decode = F.e4m3_decode
        self.e4m3_encode = F.e4m3_encode
        self.quantize_per_head = lambda x, n_rows=None: _quantize_with(self, x, n_rows)
        self.dequantize = lambda codes, scale: self.e4m3_decode(codes) * np.asarray(scale, np.float64)[None, :, None]
        self.__dict__.update(repl)

    def attn_varlen_fwd_fp8(self, q, k, v, cu_q, cu_k, scale, rows=None, causal=False, threads=None):
        qc, qs, _ = self.quantize_per_head(q, int(cu_q[-1]))
        kc, ks, _ = self.quantize_per_head(k, int(cu_k[-1]))
        vf = blas_oracle._widen(F._bits(v))
        return blas_oracle.attn_varlen_fwd(self.dequantize(qc, qs), self.dequantize(kc, ks), vf, cu_q, cu_k, scale,
                                           rows=rows, causal=causal, threads=threads)


def _quantize_with(M, x, n_rows):
    b = F._bits(x)
    n = b.shape[0] if n_rows is None else n_rows
    f = (b[:n].astype(np.uint32) << 16).view(np.float32)
    amax = np.abs(f).max(axis=(0, 2)).astype(np.float32)
    pos = amax > 0
    with np.errstate(divide="ignore"):
        inv = np.where(pos, np.float32(448) / amax, np.float32(0)).astype(np.float32)
        scale = np.where(pos, amax / np.float32(448), np.float32(1)).astype(np.float32)
    return M.e4m3_encode((f * inv[None, :, None]).astype(np.float32)), scale, inv


def _trunc_encode(x):
    x = np.asarray(x, np.float32).astype(np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.clip(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6, 8)
    q = np.floor(a / 2.0 ** (e - 3)) * 2.0 ** (e - 3)     # toward zero instead of nearest
    return F.e4m3_encode(np.copysign(np.minimum(q, 448.0), x).astype(np.float32))


def _per_tensor_quantize(x, n_rows=None):
    b = F._bits(x)
    n = b.shape[0] if n_rows is None else n_rows
    f = (b[:n].astype(np.uint32) << 16).view(np.float32)
    amax = np.float32(np.abs(f).max())
    H = b.shape[1]
    inv = np.full(H, np.float32(448) / amax, np.float32)
    scale = np.full(H, amax / np.float32(448), np.float32)
    return F.e4m3_encode((f * inv[None, :, None]).astype(np.float32)), scale, inv


MUTANTS = {
    "truncating_encode": dict(e4m3_encode=_trunc_encode),
    "bias_8_decode": dict(e4m3_decode=lambda c: F.e4m3_decode(c) / 2.0),
    "scale_dropped": dict(dequantize=lambda codes, scale: F.e4m3_decode(codes)),
    "per_tensor_scale": dict(quantize_per_head=_per_tensor_quantize),
}


def test_unmodified_mutant_passes_every_pin():
    M = _Mutant()
    for pin in PINS:
        pin(M)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_pins_catch_planted_mistake(name):
    M = _Mutant(**MUTANTS[name])
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(M)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
