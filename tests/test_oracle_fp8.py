"""Pins of the oracle's fp8 (e4m3) cache variant: the codec against the format definition and
torch's own float8_e4m3fn conversions, the per-row quantiser against its defining properties,
and the fp8-cache layer step against the plain attention on the values the codes stand for.

Each test fails for a plausible mistake: a wrong exponent bias or subnormal scale, a NaN code
taken as finite, rounding away from even, an overflow to NaN instead of saturation, a scale
from the wrong statistic or in the wrong precision, K and V scales swapped or indexed by the
wrong axis, a dropped scale, an unquantised tail.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import (E4M3_MAX, bf16_bits_to_f64, dequantize_rows_e4m3, e4m3_bits_to_f64, expert_attn_layer,
                    expert_attn_layer_fp8, f64_to_bf16_bits, f64_to_e4m3_bits, quantize_rows_e4m3)
from flow_matching_action_amd import synth


# ------------------------------------------------------------------------------------- codec
def test_e4m3_known_codes():
    # values fixed by the format: bias 7, 3 significand bits, S.1111.111 = NaN, no infinities
    v = e4m3_bits_to_f64(np.array([0x38, 0x40, 0x4E, 0x7E, 0x08, 0x01, 0x07, 0x00, 0x80, 0xB8, 0x77],
                                  np.uint8))
    assert v[0] == 1.0 and v[1] == 2.0 and v[2] == 7.0
    assert v[3] == 448.0                                  # largest finite
    assert v[4] == 2.0 ** -6                              # smallest normal
    assert v[5] == 2.0 ** -9                              # smallest subnormal
    assert v[6] == 7 * 2.0 ** -9                          # largest subnormal
    assert v[7] == 0.0 and np.signbit(v[8]) and v[8] == 0.0
    assert v[9] == -1.0
    assert v[10] == 1.875 * 2.0 ** 7                      # 0.1110.111 = 240
    assert np.isnan(e4m3_bits_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()
    assert E4M3_MAX == 448.0


def test_e4m3_decode_all_codes_matches_torch():
    c = np.arange(256, dtype=np.uint8)
    got = e4m3_bits_to_f64(c)
    ref = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(got)
    assert np.array_equal(got[fin], ref[fin])
    assert fin.sum() == 254
    pos = got[:0x7F]                                      # codes 0x00 .. 0x7E: strictly increasing
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(got[0x80:0xFF], -pos)           # sign symmetry


def test_e4m3_round_trip_of_every_finite_code():
    c = np.arange(256, dtype=np.uint8)
    v = e4m3_bits_to_f64(c)
    fin = ~np.isnan(v)
    assert np.array_equal(f64_to_e4m3_bits(v[fin]), c[fin])


def _nearest_code_brute_force(x: float) -> int:
    """Nearest finite e4m3 value with ties to the even code, after saturation to +-448."""
    xs = min(max(x, -448.0), 448.0)
    c = np.arange(256, dtype=np.uint8)
    v = e4m3_bits_to_f64(c)
    ok = ~np.isnan(v) & ((c & 0x80) == (0x80 if np.signbit(xs) else 0))
    cand, vals = c[ok], v[ok]
    d = np.abs(vals - xs)
    best = d.min()
    tied = cand[d == best]
    even = tied[(tied & 1) == 0]
    return int(even[0] if len(even) else tied[0])


def test_e4m3_encode_every_bf16_input_brute_force():
    # every finite bfloat16 value in the e4m3 range and a little beyond (where it saturates)
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bf16_bits_to_f64(bits)
    x = x[np.isfinite(x) & (np.abs(x) <= 600.0) & (np.abs(x) >= 2.0 ** -12)]
    got = f64_to_e4m3_bits(x)
    sample = np.random.default_rng(0).choice(len(x), 3000, replace=False)
    for i in sample:
        assert got[i] == _nearest_code_brute_force(float(x[i])), float(x[i])


def test_e4m3_encode_matches_torch_cast_after_clipping():
    # torch's float -> float8_e4m3fn cast is an independent nearest-even implementation (it does
    # not saturate, hence the clip); exact ties sit at odd multiples of half a spacing
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200_000) * 60.0,
                        (2 * rng.integers(-900, 900, 20_000) + 1) * 2.0 ** -4,     # ties among the normals
                        (2 * rng.integers(-7, 7, 2_000) + 1) * 2.0 ** -10,         # ties among the subnormals
                        rng.uniform(-600, 600, 20_000)]).astype(np.float32)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f64_to_e4m3_bits(x.astype(np.float64)), ref)


@pytest.mark.parametrize("x,code", [(460.0, 0x7E), (464.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE),
                                    (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (-2.0 ** -11, 0x80),
                                    (1.0 + 2.0 ** -4, 0x38), (1.0 + 3 * 2.0 ** -4, 0x3A)])
def test_e4m3_saturation_and_ties(x, code):
    assert int(f64_to_e4m3_bits(x)) == code
    assert int(f64_to_e4m3_bits(np.nan)) == 0x7F


# --------------------------------------------------------------------------------- quantiser
def test_quantiser_rule_per_row():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((8, 64, 128)) * rng.uniform(0.01, 30, (8, 64, 1))).astype(np.float32)
    x[3, 5] = 0.0                                           # an all-zero row
    codes, scales = quantize_rows_e4m3(x)
    assert codes.dtype == np.uint8 and scales.dtype == np.float32 and scales.shape == (8, 64)
    amax = np.abs(x).max(-1)
    nz = amax > 0
    assert np.array_equal(scales[nz], (amax[nz] / np.float32(448.0)).astype(np.float32))
    assert scales[3, 5] == 1.0 and not codes[3, 5].any()
    # the row maximum lands on +-448 (the quotient is within one float32 ulp of 448)
    v = e4m3_bits_to_f64(codes)
    assert np.array_equal(np.abs(v).max(-1)[nz], np.full(nz.sum(), 448.0))
    # reconstruction within half a spacing: relative 2^-4 for normals, 2^-10 * scale below
    err = np.abs(dequantize_rows_e4m3(codes, scales) - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scales[..., None]) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_quantiser_divides_in_float32():
    # a row whose float64 quotient and float32 quotient land on different sides of a tie:
    # x / scale in float64 is 1.0625 + 2^-30-ish, in float32 exactly the tie 1.0625 -> even 1.0
    x = np.zeros((1, 128), np.float32)
    x[0, 0] = 448.0 * 3                                   # scale = 3 exactly
    x[0, 1] = np.float32(3 * 1.0625)                      # 3.1875: quotient 1.0625 exactly (a tie)
    codes, scales = quantize_rows_e4m3(x)
    assert scales[0] == 3.0
    assert e4m3_bits_to_f64(codes[0, 1]) == 1.0           # tie to even
    assert e4m3_bits_to_f64(codes[0, 0]) == 448.0


# ------------------------------------------------------------------------------- layer (fp8)
def _small_fp8(S=128, Smax=256, seed=11):
    return synth.layer_inputs_fp8(Smax, S, seed)


def test_fp8_layer_equals_attention_on_dequantised_cache():
    d = _small_fp8()
    r = expert_attn_layer_fp8(d["q"], d["k"], d["v"], d["gq"], d["gk"], d["Kc8"], d["Ks"], d["Vc8"], d["Vs"],
                              d["S"], d["Smax"])
    # the tails: the bf16-rounded roped k and the bf16 v, each quantised by the row rule
    kq, ks = quantize_rows_e4m3(bf16_bits_to_f64(f64_to_bf16_bits(r["k_roped"])).astype(np.float32))
    vq, vs = quantize_rows_e4m3(bf16_bits_to_f64(d["v"]).astype(np.float32))
    assert np.array_equal(r["k_tail_codes"], kq) and np.array_equal(r["k_tail_scales"], ks)
    assert np.array_equal(r["v_tail_codes"], vq) and np.array_equal(r["v_tail_scales"], vs)
    Smax = d["Smax"]
    assert np.array_equal(r["Kc8_new"][:, :Smax - 64], d["Kc8"][:, :Smax - 64])
    assert np.array_equal(r["Vs_new"][:, :Smax - 64], d["Vs"][:, :Smax - 64])
    assert np.array_equal(r["Kc8_new"][:, Smax - 64:], kq) and np.array_equal(r["Vs_new"][:, Smax - 64:], vs)


def test_fp8_layer_close_to_the_unquantised_layer():
    # Build an fp8 cache from a bf16 one with the row rule and compare the fp8 layer with the
    # bf16 layer on the original values: the difference is the e4m3 rounding only (relative
    # 2^-4 per element at most), far below what a dropped, swapped or misindexed scale does.
    b = synth.layer_inputs(256, 128, 12, filler=None)
    Kf = bf16_bits_to_f64(b["Kc"]).astype(np.float32)
    Vf = bf16_bits_to_f64(b["Vc"]).astype(np.float32)
    # rows of different size (moderate for K, whose scores feed the softmax; wide for V)
    rng = np.random.default_rng(3)
    Kf *= np.exp2(rng.integers(-1, 2, (8, 256, 1))).astype(np.float32)
    Vf *= np.exp2(rng.integers(-4, 5, (8, 256, 1))).astype(np.float32)
    Kc8, Ks = quantize_rows_e4m3(Kf)
    Vc8, Vs = quantize_rows_e4m3(Vf)
    r8 = expert_attn_layer_fp8(b["q"], b["k"], b["v"], b["gq"], b["gk"], Kc8, Ks, Vc8, Vs, 128, 256)
    r16 = expert_attn_layer(b["q"], b["k"], b["v"], b["gq"], b["gk"], f64_to_bf16_bits(Kf), f64_to_bf16_bits(Vf),
                            128, 256)
    diff = np.abs(r8["out"] - r16["out"])
    scale = np.abs(r16["out"]).max()
    assert diff.max() < 0.06 * scale
    assert np.corrcoef(r8["out"].ravel(), r16["out"].ravel())[0, 1] > 0.995
    # and the plausible mistakes are far outside that: K scales ignored, K and V scales swapped
    Kbad = e4m3_bits_to_f64(Kc8)
    out_bad = oracle.attention(r8["q_roped"], np.concatenate([Kbad[:, :192], r8["k_roped"]], 1)[:, :256],
                               dequantize_rows_e4m3(Vc8, Vs), oracle.build_mask(128, 256), 128 ** -0.5)
    assert np.abs(out_bad - r16["out"]).max() > 0.2 * scale
    r_sw = expert_attn_layer_fp8(b["q"], b["k"], b["v"], b["gq"], b["gk"], Kc8, Vs, Vc8, Ks, 128, 256)
    assert np.abs(r_sw["out"] - r16["out"]).max() > 0.2 * scale


def test_fp8_hidden_rows_change_nothing():
    d = _small_fp8()
    args = (d["q"], d["k"], d["v"], d["gq"], d["gk"])
    r0 = expert_attn_layer_fp8(*args, d["Kc8"], d["Ks"], d["Vc8"], d["Vs"], d["S"], d["Smax"])
    K2, V2, Ks2, Vs2 = d["Kc8"].copy(), d["Vc8"].copy(), d["Ks"].copy(), d["Vs"].copy()
    K2[:, 128:192] = 0x5A
    V2[:, 128:192] = 0xD3
    Ks2[:, 128:192] = 1e3
    Vs2[:, 128:192] = 7.0
    r1 = expert_attn_layer_fp8(*args, K2, Ks2, V2, Vs2, d["S"], d["Smax"])
    assert np.array_equal(r0["out"], r1["out"])


def test_fp8_tail_placement_equals_concatenation():
    # attention over [0, S) and the tail under the mask == attention over the concatenation
    d = _small_fp8(S=100)
    r = expert_attn_layer_fp8(d["q"], d["k"], d["v"], d["gq"], d["gk"], d["Kc8"], d["Ks"], d["Vc8"], d["Vs"],
                              100, 256)
    K = dequantize_rows_e4m3(r["Kc8_new"], r["Ks_new"])
    V = dequantize_rows_e4m3(r["Vc8_new"], r["Vs_new"])
    Kcat = np.concatenate([K[:, :100], K[:, 192:]], 1)
    Vcat = np.concatenate([V[:, :100], V[:, 192:]], 1)
    ref = oracle.attention(r["q_roped"], Kcat, Vcat, None, 128 ** -0.5)
    assert np.abs(ref - r["out"]).max() < 1e-12


def test_two_e4m3_parts_carry_a_scaled_bf16_value():
    # The fp8 scores take q in two e4m3 parts: a query row scaled by a power of two so that its
    # largest |element| lies in [128, 256), hi = e4m3(x) and lo = e4m3(x - hi), both to nearest
    # even. Over every bf16 value below 256 in magnitude: hi + lo is x exactly for |x| >= 1/4
    # (x's last bit is then no finer than e4m3's smallest subnormal 2^-9, and x - hi is a
    # multiple of it no larger than 8 of them), and within 2^-10 of x below.
    bits = np.arange(0x0000, 0x4380, dtype=np.uint32)       # +0 .. the largest bf16 below 256
    bits = np.concatenate([bits, bits | 0x8000]).astype(np.uint16)
    x = bf16_bits_to_f64(bits)
    assert np.all(np.abs(x) < 256)
    hi = e4m3_bits_to_f64(f64_to_e4m3_bits(x))
    lo = e4m3_bits_to_f64(f64_to_e4m3_bits(x - hi))
    big = np.abs(x) >= 0.25
    assert np.array_equal(hi[big] + lo[big], x[big])
    assert np.all(np.abs(hi + lo - x) <= 2.0 ** -10)
    assert not np.array_equal(hi[big], x[big])               # one part alone does not suffice
