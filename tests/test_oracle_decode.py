"""Pins of the oracle's text-model decode step (64 query heads, 8 kv heads, one token at pos).

Each test fails for a plausible mistake: a key range off by one (excluding the token's own key or
reading past it), the new row written to the wrong place or unrounded, a wrong GQA group size or
head order, a wrong scale, RoPE at the wrong position.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import bf16_bits_to_f64, decode_attention, f64_to_bf16_bits, text_decode_attn
from flow_matching_action_amd import synth


def _run(d, pos=None, rope_delta=0):
    pos = d["pos"] if pos is None else pos
    return text_decode_attn(d["q"], d["k"], d["v"], d["gq"], d["gk"], d["Kc"], d["Vc"], pos, rope_delta)


def test_first_position_returns_the_own_value():
    # at pos = 0 the only visible key is the token's own: the output of head h is v of its group
    d = synth.decode_inputs(64, 0, seed=1)
    r = _run(d)
    v = bf16_bits_to_f64(d["v"])
    for h in range(64):
        assert np.allclose(r["out"][h], v[h // 8], rtol=0, atol=1e-12)


def test_matches_brute_force_loops():
    d = synth.decode_inputs(40, 11, seed=2)
    r = _run(d)
    q = r["q_roped"]
    K = bf16_bits_to_f64(r["Kc_new"])
    V = bf16_bits_to_f64(r["Vc_new"])
    for h in (0, 7, 8, 33, 63):
        g = h // 8
        s = [sum(q[h, i] * K[g, j, i] for i in range(128)) / np.sqrt(128) for j in range(12)]
        m = max(s)
        w = [np.exp(x - m) for x in s]
        ref = [sum(w[j] * V[g, j, i] for j in range(12)) / sum(w) for i in range(128)]
        assert np.allclose(r["out"][h], ref, rtol=1e-12, atol=1e-14)


def test_matches_torch_sdpa():
    d = synth.decode_inputs(512, 300, seed=3)
    r = _run(d)
    q = torch.from_numpy(r["q_roped"])[:, None, :]                    # [64, 1, D]
    K = torch.from_numpy(bf16_bits_to_f64(r["Kc_new"])[:, :301])      # [8, 301, D]
    V = torch.from_numpy(bf16_bits_to_f64(r["Vc_new"])[:, :301])
    K = K.repeat_interleave(8, dim=0)
    V = V.repeat_interleave(8, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, K, V)[:, 0, :].numpy()
    assert np.abs(ref - r["out"]).max() < 1e-12


def test_new_row_written_and_rows_after_pos_ignored():
    d = synth.decode_inputs(256, 100, seed=4)
    r = _run(d)
    assert np.array_equal(r["Kc_new"][:, 100], f64_to_bf16_bits(r["k_roped"]))
    assert np.array_equal(r["Vc_new"][:, 100], d["v"])
    other = np.ones(256, bool)
    other[100] = False
    assert np.array_equal(r["Kc_new"][:, other], d["Kc"][:, other])
    d2 = dict(d)
    for n in ("Kc", "Vc"):
        d2[n] = d[n].copy()
        d2[n][:, 101:] = f64_to_bf16_bits(-3.0)
        d2[n][:, 100] = 0x7FC0            # the old row pos is overwritten before use
    r2 = _run(d2)
    assert np.array_equal(r["out"], r2["out"])


def test_group_mapping_and_rope_position():
    d = synth.decode_inputs(128, 60, seed=5)
    q = d["q"].copy()
    q[8:16] = q[8]                           # the heads of group 1 share one query
    d["q"] = q
    r = _run(d)
    assert np.array_equal(r["out"][8], r["out"][15]) and not np.array_equal(r["out"][8], r["out"][16])
    # RoPE is applied at pos + rope_delta: shifting both by the same amount keeps the scores
    # (rotation invariance of q . k for equal positions), shifting only rope_delta does not
    cos0, sin0 = oracle.rope_tables(60, 1)
    qn = oracle.rms_norm(bf16_bits_to_f64(d["q"]), bf16_bits_to_f64(d["gq"]))
    assert np.allclose(r["q_roped"], oracle.apply_rope(qn, cos0, sin0), rtol=0, atol=1e-14)
    r5 = _run(d, rope_delta=5)
    cos5, sin5 = oracle.rope_tables(65, 1)
    assert np.allclose(r5["q_roped"], oracle.apply_rope(qn, cos5, sin5), rtol=0, atol=1e-14)
    assert not np.allclose(r5["out"], r["out"])


def test_decode_attention_scale_and_range():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((64, 128))
    K = rng.standard_normal((8, 20, 128))
    V = rng.standard_normal((8, 20, 128))
    out = decode_attention(q, K, V, 9, 128 ** -0.5)
    # dropping key 9 or adding key 10 changes the result; scaling q by sqrt(2) equals scale sqrt(2)/sqrt(128)
    assert not np.allclose(out, decode_attention(q, K, V, 8, 128 ** -0.5))
    assert not np.allclose(out, decode_attention(q, K, V, 10, 128 ** -0.5))
    assert np.allclose(decode_attention(q * np.sqrt(2), K, V, 9, 128 ** -0.5),
                       decode_attention(q, K, V, 9, np.sqrt(2) * 128 ** -0.5), rtol=1e-12)
    with pytest.raises(ValueError):
        text_decode_attn(np.zeros((64, 128), np.uint16), np.zeros((8, 128), np.uint16), np.zeros((8, 128), np.uint16),
                         np.zeros(128, np.uint16), np.zeros(128, np.uint16), np.zeros((8, 20, 128), np.uint16),
                         np.zeros((8, 20, 128), np.uint16), 20)
