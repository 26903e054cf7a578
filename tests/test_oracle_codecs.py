"""Pins for the oracle's number formats (CPU only).

bf16 and E4M3 are checked against their bit definitions (closed forms), the
rounding rule on hand-picked ties, and torch's CPU conversions (an independent
library routine) on random values.
"""

import numpy as np
import pytest
import torch

from oracle import codecs
from memory_bound_transformer_decode_amd import synth


# ------------------------------------------------------------------ bf16

def test_bf16_known_patterns():
    assert codecs.bf16_decode(np.array([0x3F80], np.uint16))[0] == 1.0
    assert codecs.bf16_decode(np.array([0xC000], np.uint16))[0] == -2.0
    assert codecs.bf16_decode(np.array([0x0001], np.uint16))[0] == 2.0 ** -133  # smallest subnormal
    assert codecs.bf16_encode(np.array([1.0]))[0] == 0x3F80
    assert codecs.bf16_encode(np.array([-0.0]))[0] == 0x8000


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert codecs.bf16_encode(np.array([1 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert codecs.bf16_round(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    # just above a tie rounds up
    assert codecs.bf16_round(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7


def test_bf16_roundtrip_all_finite_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = codecs.bf16_decode(bits)
    fin = np.isfinite(vals)
    back = codecs.bf16_encode(vals[fin])
    assert np.array_equal(back, bits[fin])


def test_bf16_matches_torch_cpu_conversion():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000),
                        rng.standard_normal(5000) * 1e-38,  # subnormal range
                        rng.standard_normal(5000) * 1e30,
                        rng.uniform(-4, 4, 5000)])
    ours = codecs.bf16_encode(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------ E4M3

def test_e4m3_table_from_definition():
    t = codecs.E4M3_TABLE
    assert t[0x7E] == 448.0  # largest finite
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])  # S.1111.111 is NaN
    assert t[0x01] == 2.0 ** -9  # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9
    assert t[0x08] == 2.0 ** -6  # smallest normal
    assert t[0x38] == 1.0
    assert t[0xB8] == -1.0
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert np.sum(np.isnan(t)) == 2  # no infinities, two NaNs
    finite = t[np.isfinite(t)]
    assert finite.max() == 448.0 and finite.min() == -448.0


def test_e4m3_rounding_and_saturation():
    enc = codecs.e4m3_encode
    assert enc(np.array([1.0625]))[0] == 0x38  # tie between 1 and 1.125 -> even (1.0)
    assert enc(np.array([1.1875]))[0] == 0x3A  # tie between 1.125 and 1.25 -> 1.25
    assert enc(np.array([500.0]))[0] == 0x7E  # saturates to 448, never NaN
    assert enc(np.array([-1e9]))[0] == 0xFE
    assert enc(np.array([2.0 ** -10]))[0] == 0x00  # tie between 0 and 2^-9 -> 0
    assert enc(np.array([3 * 2.0 ** -11]))[0] == 0x01
    assert enc(np.array([15.5 * 2.0 ** -10]))[0] == 0x08  # subnormal rounds up into the normals


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    vals = codecs.e4m3_decode(codes)
    fin = np.isfinite(vals)
    assert np.array_equal(codecs.e4m3_encode(vals[fin]), codes[fin])


def test_e4m3_matches_torch_cpu_conversion():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(20000) * 50, rng.uniform(-448, 448, 20000),
                        rng.standard_normal(5000) * 0.01])
    x32 = x.astype(np.float32)
    ours = codecs.e4m3_encode(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_fp8_model_recipe_reproduced_by_oracle_encoder():
    """The stored fp8 models are exactly per-row absmax/448 + RNE E4M3 codes."""
    g = torch.Generator().manual_seed(5)
    w32 = torch.randn(64, 200, generator=g) * 0.02
    w32[3] = 0.0  # an all-zero row gets scale 1
    q, s = synth.quantize_rows_fp8(w32)
    codes, s_ref = codecs.fp8_quantize_rows(w32.numpy())
    assert np.array_equal(s.numpy(), s_ref)
    assert s_ref[3] == 1.0
    assert np.array_equal(q.view(torch.uint8).numpy(), codes)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_stored_matrix_decode_is_exact_product(fmt):
    """decode(code) * scale is formed exactly in float64 (<= 4 x 24 significant bits)."""
    g = torch.Generator().manual_seed(7)
    w32 = torch.randn(16, 64, generator=g) * 0.02
    if fmt == "bf16":
        bits = w32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(codecs.bf16_decode(bits),
                              w32.to(torch.bfloat16).to(torch.float64).numpy())
    else:
        q, s = synth.quantize_rows_fp8(w32)
        v = codecs.e4m3_decode(q.view(torch.uint8).numpy()) * s.numpy().astype(np.float64)[:, None]
        ref = (q.to(torch.float64) * s.to(torch.float64)[:, None]).numpy()
        assert np.array_equal(v, ref)


# ------------------------------------------------------------------ int8

def test_int8_decode_twos_complement():
    """Every byte from the two's-complement definition: 0x00 = 0, 0x7F = 127, 0x80 = -128,
    0xFF = -1; agrees with numpy's own int8 view of the same bytes."""
    b = np.arange(256, dtype=np.uint8)
    v = codecs.int8_decode(b)
    assert v[0] == 0 and v[0x7F] == 127 and v[0x80] == -128 and v[0xFF] == -1 and v[0x81] == -127
    assert np.array_equal(v, b.view(np.int8).astype(np.float64))
    assert codecs.decode(b, "int8").dtype == np.float64


def test_int8_model_recipe_reproduced_by_oracle_encoder():
    """The stored int8 models are exactly per-row absmax/127 + round-half-even codes in
    [-127, 127]; the row's largest magnitude maps to +-127."""
    g = torch.Generator().manual_seed(6)
    w32 = torch.randn(64, 200, generator=g) * 0.02
    w32[5] = 0.0
    q, s = synth.quantize_rows_int8(w32)
    codes, s_ref = codecs.int8_quantize_rows(w32.numpy())
    assert np.array_equal(s.numpy(), s_ref)
    assert s_ref[5] == 1.0
    assert np.array_equal(q.view(torch.uint8).numpy(), codes)
    qi = codecs.int8_decode(codes)
    assert qi.min() >= -127 and qi.max() <= 127
    amax_col = np.argmax(np.abs(w32.numpy()), axis=1)
    for r in range(64):
        if r != 5:
            assert abs(qi[r, amax_col[r]]) == 127


def test_int8_round_half_even_ties():
    """Ties go to the even code: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, -0.5 -> 0, -1.5 -> -2."""
    w = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5]], dtype=np.float32)  # scale exactly 1
    codes, s = codecs.int8_quantize_rows(w)
    assert s[0] == 1.0
    assert codecs.int8_decode(codes).tolist() == [[127, 0, 2, 2, 0, -2]]


def test_int8_stored_matrix_decode_is_exact_product():
    g = torch.Generator().manual_seed(8)
    w32 = torch.randn(16, 64, generator=g) * 0.02
    q, s = synth.quantize_rows_int8(w32)
    v = codecs.int8_decode(q.view(torch.uint8).numpy()) * s.numpy().astype(np.float64)[:, None]
    ref = (q.to(torch.float64) * s.to(torch.float64)[:, None]).numpy()
    assert np.array_equal(v, ref)
