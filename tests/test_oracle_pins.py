"""Pins of the fp64 oracle against closed forms, invariants, library routines and brute force.

Each test would fail for a plausible mistake in the oracle: a dropped eps or
gamma, a wrong RoPE sign or half, a wrong frequency, a wrong GQA head mapping,
a transposed operand, a mask on the wrong rows, a wrong LSE combine.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (apply_rope, attention, attention_partial, bf16_bits_to_f64, build_mask,
                    expert_attn_layer, lse_combine, place_tail, rms_norm, rope_tables)
from flow_matching_action_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ constants the pages state
def test_constants_match_pages():
    with open(os.path.join(GOLDEN, "method_constants.json")) as f:
        c = json.load(f)
    assert oracle.N_Q_HEADS == c["n_q_heads"]["value"]
    assert oracle.N_KV_HEADS == c["n_kv_heads"]["value"]
    assert oracle.N_TOK == c["n_tok"]["value"]
    assert oracle.HEAD_DIM == c["head_dim"]["value"]
    assert oracle.EPS == c["rms_eps"]["value"]
    assert oracle.ROPE_THETA == c["rope_theta"]["value"]
    assert oracle.MASK_MIN == c["mask_min"]["value"]
    w = c["worked_context"]
    m = build_mask(w["S"], w["Smax"])
    assert m.shape == (c["folded_rows_per_kv_head"]["value"], w["Smax"])
    zero = np.zeros(w["Smax"], bool)
    for a, b in w["mask_zero_spans"]:
        zero[a:b] = True
    assert np.all(m[:, zero] == 0.0) and np.all(m[:, ~zero] == c["mask_min"]["value"])
    cos, sin = rope_tables(w["S"] + w["rope_delta"])
    # table row 0 and row 63 are positions 4700 and 4763: check through frequency 0 (angle = position)
    p0, p1 = w["positions_first_last"]
    assert cos[0, 0] == math.cos(p0) and sin[-1, 0] == math.sin(p1)


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_closed_form_constant_row():
    for c in (0.5, 3.0, -2.0):
        x = np.full((1, 128), c)
        y = rms_norm(x, np.ones(128), 1e-6)
        assert np.allclose(y, c / math.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)


def test_rmsnorm_rms_of_output_and_gamma():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 128))
    m = np.mean(x * x, axis=-1)
    y = rms_norm(x, np.ones(128), 1e-6)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), np.sqrt(m / (m + 1e-6)), rtol=1e-14)
    g = rng.standard_normal(128)
    assert np.allclose(rms_norm(x, g, 1e-6), y * g, rtol=1e-14)
    # scale invariance up to eps
    assert np.allclose(rms_norm(1000 * x, g, 1e-6), rms_norm(x, g, 1e-6), rtol=1e-6)


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((16, 64, 128))
    g = 1 + 0.1 * rng.standard_normal(128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(rms_norm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------------ RoPE
def test_rope_position_zero_is_identity():
    cos, sin = rope_tables(0, n_tok=1)
    x = np.random.default_rng(3).standard_normal((4, 1, 128))
    assert np.array_equal(apply_rope(x, cos, sin), x)


def test_rope_matches_complex_rotation():
    # Independent formulation: pair (j, j+64) as z = x_j + i x_{j+64}, rotated by e^{i p w_j},
    # w_j = theta^(-j/64). Catches a wrong sign, a swapped half or a wrong frequency.
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 3, 128))
    pos0 = 4700
    cos, sin = rope_tables(pos0, n_tok=3)
    y = apply_rope(x, cos, sin)
    for i in range(3):
        p = pos0 + i
        for j in range(64):
            w = 5e6 ** (-j / 64.0)
            z = complex(x[0, i, j], x[0, i, j + 64]) * cmath.exp(1j * p * w)
            assert abs(y[0, i, j] - z.real) < 1e-9 and abs(y[0, i, j + 64] - z.imag) < 1e-9


def test_rope_unit_vector_layout():
    cos, sin = rope_tables(7, n_tok=1)
    e0 = np.zeros((1, 1, 128)); e0[..., 0] = 1
    y = apply_rope(e0, cos, sin)
    assert y[0, 0, 0] == math.cos(7) and y[0, 0, 64] == math.sin(7)      # sine lands in the upper half, +
    assert np.count_nonzero(y) == 2
    e64 = np.zeros((1, 1, 128)); e64[..., 64] = 1
    y = apply_rope(e64, cos, sin)
    assert y[0, 0, 64] == math.cos(7) and y[0, 0, 0] == -math.sin(7)


def test_rope_preserves_pair_norms_and_relative_property():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    cm, sm = rope_tables(1234, 1)
    cn, sn = rope_tables(1000, 1)
    cd, sd = rope_tables(234, 1)
    rq = apply_rope(q, cm, sm)
    pair = lambda v: v[..., :64] ** 2 + v[..., 64:] ** 2
    assert np.allclose(pair(rq), pair(q), rtol=1e-12)
    lhs = float(np.sum(rq * apply_rope(k, cn, sn)))
    rhs = float(np.sum(apply_rope(q, cd, sd) * k))
    assert abs(lhs - rhs) < 1e-9
    # composition: rope(rope(x, a), b) == rope(x, a + b)
    ca, sa = rope_tables(300, 1)
    cb, sb = rope_tables(934, 1)
    assert np.allclose(apply_rope(apply_rope(q, ca, sa), cb, sb), rq, atol=1e-10)


# ------------------------------------------------------------------ attention
def _brute_attention(q, K, V, mask, scale):
    hq, t, d = q.shape
    rep = hq // K.shape[0]
    out = np.zeros((hq, t, V.shape[-1]))
    for h in range(hq):
        g = h // rep
        for i in range(t):
            s = [sum(q[h, i, c] * K[g, j, c] for c in range(d)) * scale + mask[j] for j in range(K.shape[1])]
            mx = max(s)
            e = [math.exp(v - mx) for v in s]
            tot = sum(e)
            for c in range(V.shape[-1]):
                out[h, i, c] = sum(e[j] * V[g, j, c] for j in range(K.shape[1])) / tot
    return out


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 3, 5))
    K = rng.standard_normal((2, 7, 5))
    V = rng.standard_normal((2, 7, 6))
    mask = np.array([0, 0, -1e9, -1e9, 0, 0, 0], float)
    ref = _brute_attention(q, K, V, mask, 0.37)
    got = attention(q, K, V, np.tile(mask, (6, 1)), 0.37)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((16, 64, 128))
    K = rng.standard_normal((8, 256, 128))
    V = rng.standard_normal((8, 256, 128))
    mask = build_mask(128, 256)
    got = attention(q, K, V, mask, 128 ** -0.5)
    Kr = torch.from_numpy(K).repeat_interleave(2, dim=0)
    Vr = torch.from_numpy(V).repeat_interleave(2, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), Kr, Vr, attn_mask=torch.from_numpy(mask[:64]), scale=128 ** -0.5).numpy()
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_gqa_head_mapping():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((16, 4, 128))
    K = rng.standard_normal((8, 10, 128))
    V = np.broadcast_to(np.arange(8, dtype=float)[:, None, None], (8, 10, 128)).copy()
    out = attention(q, K, V, None, 0.1)
    for h in range(16):
        assert np.allclose(out[h], h // 2, rtol=0, atol=1e-12)


def test_zero_query_gives_mean_of_unmasked_values():
    rng = np.random.default_rng(9)
    V = rng.standard_normal((8, 256, 128))
    K = rng.standard_normal((8, 256, 128))
    q = np.zeros((16, 64, 128))
    out = attention(q, K, V, build_mask(100, 256), 0.1)
    keep = np.r_[0:100, 192:256]
    for h in range(16):
        assert np.allclose(out[h], V[h // 2, keep].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_lse_combine_equals_single_pass():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((16, 64, 128))
    K = rng.standard_normal((8, 300, 128))
    V = rng.standard_normal((8, 300, 128))
    direct = attention(q, K, V, None, 128 ** -0.5)
    perm = rng.permutation(300)
    cuts = [0, 7, 8, 120, 299, 300]
    parts = [attention_partial(q, K, V, perm[a:b], 128 ** -0.5) for a, b in zip(cuts[:-1], cuts[1:])]
    assert np.allclose(lse_combine(parts), direct, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ the full layer step
def _layer(inp, **kw):
    return expert_attn_layer(inp["q"], inp["k"], inp["v"], inp["gq"], inp["gk"], inp["Kc"], inp["Vc"],
                             inp["S"], inp["Smax"], inp["rope_delta"], **kw)


def test_hidden_rows_change_nothing():
    outs = []
    for filler in (7.0, 0.0, -3.0, 1e4):
        inp = synth.layer_inputs(256, 128, seed=11, filler=filler)
        outs.append(_layer(inp)["out"])
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_tail_placement_equals_concatenation():
    inp = synth.layer_inputs(256, 100, seed=12)
    r = _layer(inp)
    S = 100
    Kcat = np.concatenate([bf16_bits_to_f64(inp["Kc"])[:, :S], bf16_bits_to_f64(r["k_tail_bits"])], axis=1)
    Vcat = np.concatenate([bf16_bits_to_f64(inp["Vc"])[:, :S], bf16_bits_to_f64(inp["v"])], axis=1)
    ref = attention(r["q_roped"], Kcat, Vcat, None, 128 ** -0.5)
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-14)


def test_tail_write_touches_only_tail_rows():
    inp = synth.layer_inputs(256, 128, seed=13)
    r = _layer(inp)
    assert np.array_equal(r["Kc_new"][:, :192], inp["Kc"][:, :192])
    assert np.array_equal(r["Vc_new"][:, :192], inp["Vc"][:, :192])
    assert np.array_equal(r["Vc_new"][:, 192:], inp["v"])
    assert np.array_equal(r["Kc_new"][:, 192:], r["k_tail_bits"])


def test_empty_cache_is_plain_self_attention():
    inp = synth.layer_inputs(64, 0, seed=14)
    r = _layer(inp)
    ref = attention(r["q_roped"], bf16_bits_to_f64(r["k_tail_bits"]), bf16_bits_to_f64(inp["v"]), None,
                    128 ** -0.5)
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-14)


def test_identical_heads_in_a_group_give_identical_outputs():
    inp = synth.layer_inputs(256, 77, seed=15)
    inp["q"][1::2] = inp["q"][0::2]
    out = _layer(inp)["out"]
    assert np.array_equal(out[0::2], out[1::2])


def test_positions_follow_S_and_rope_delta():
    # q roped at (S, delta) equals q roped at (S + delta, 0): only their sum enters.
    inp = synth.layer_inputs(256, 50, seed=16)
    a = _layer(inp)
    inp2 = dict(inp, S=50, rope_delta=0)
    b = expert_attn_layer(inp2["q"], inp2["k"], inp2["v"], inp2["gq"], inp2["gk"], inp2["Kc"], inp2["Vc"],
                          50, 256, 0)
    assert np.array_equal(a["q_roped"], b["q_roped"])
    c = expert_attn_layer(inp["q"], inp["k"], inp["v"], inp["gq"], inp["gk"], inp["Kc"], inp["Vc"], 40, 256, 10)
    assert np.allclose(c["q_roped"], a["q_roped"], rtol=0, atol=1e-12)
    assert not np.allclose(c["out"], a["out"])   # S changes which cache rows are visible


def test_rejects_cache_without_scratch_tail():
    inp = synth.layer_inputs(256, 128, seed=17)
    with pytest.raises(ValueError):
        expert_attn_layer(inp["q"], inp["k"], inp["v"], inp["gq"], inp["gk"], inp["Kc"], inp["Vc"], 193, 256)
