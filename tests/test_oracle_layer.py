"""Pins of the oracle's whole expert decoder layer (residual norms, qkv projection and head split,
attention, head concat, o projection, SwiGLU MLP, residual adds).

Each test fails for a plausible mistake: a residual add dropped or applied twice, q/k/v taken from
the wrong column blocks or heads in the wrong order, heads concatenated in the wrong order, w1 and
w3 swapped, SiLU on the wrong branch or a wrong SiLU, a projection transposed.
"""
import numpy as np
import pytest

import oracle
from oracle import bf16_bits_to_f64, expert_layer, f64_to_bf16_bits, silu
from flow_matching_action_amd import synth

B = oracle.f64_to_bf16_bits


def _layer(w, x, c, S=128, Smax=256):
    return expert_layer(x, w["ln1"], w["wqkv"], w["qn"], w["kn"], w["wo"], w["ln2"], w["w1"], w["w3"], w["w2"],
                        c["Kc"], c["Vc"], S, Smax)


@pytest.fixture(scope="module")
def base():
    return synth.layer_weights(7), synth.residual_inputs(8), synth.layer_inputs(256, 128, 1)


def test_silu_closed_forms():
    x = np.linspace(-30, 30, 1001)
    assert silu(np.array(0.0)) == 0.0
    assert np.allclose(silu(x) - silu(-x), x, rtol=0, atol=1e-12)          # x sigma(x) - (-x) sigma(-x) = x
    assert np.allclose(silu(np.array([40.0])), [40.0], rtol=1e-15)
    assert abs(silu(np.array([-40.0]))[0]) < 1e-15
    h = 1e-6
    assert abs((silu(np.array(h)) - silu(np.array(-h))) / (2 * h) - 0.5) < 1e-9  # slope 1/2 at 0


def test_zero_output_projections_leave_the_residual(base):
    w, x, c = base
    w0 = dict(w)
    w0["wo"] = np.zeros_like(w["wo"])
    w0["w2"] = np.zeros_like(w["w2"])
    r = _layer(w0, x, c)
    assert np.array_equal(r["x2"], bf16_bits_to_f64(x))
    assert np.array_equal(r["x_out"], bf16_bits_to_f64(x))
    # only the MLP off: x_out is x2 = x + o
    w1 = dict(w)
    w1["w2"] = np.zeros_like(w["w2"])
    r1 = _layer(w1, x, c)
    assert np.array_equal(r1["x_out"], r1["x2"]) and not np.array_equal(r1["x2"], bf16_bits_to_f64(x))


def test_head_split_and_concat_order(base):
    # q = 0 (zero q columns): each head's attention output is the mean of its group's visible V
    # rows; v head g is column block 24 + g of qkv, so own v rows are known; the concat puts
    # head h at columns 128h .. 128h+127 of attn.
    w, x, c = base
    w2 = dict(w)
    wqkv = bf16_bits_to_f64(w["wqkv"]).copy()
    wqkv[:, :2048] = 0.0
    w2["wqkv"] = B(wqkv)
    r = _layer(w2, x, c, S=100)
    qkv = r["qkv"]
    V = bf16_bits_to_f64(c["Vc"])
    for h in (0, 5, 15):
        g = h // 2
        own_v = qkv[:, 3072 + 128 * g:3072 + 128 * (g + 1)]               # [64, 128]
        ref = np.concatenate([V[g, :100], own_v], 0).mean(0)
        got = r["attn"][:, 128 * h:128 * (h + 1)]                          # every token row
        assert np.allclose(got, ref[None, :], rtol=0, atol=2 ** -8 * np.abs(ref).max() + 1e-6)
    # k comes from block 16 + g: with q = 0 it cannot matter, so changing it changes nothing
    wqkv2 = wqkv.copy()
    wqkv2[:, 2048:3072] = 0.0
    w3 = dict(w2)
    w3["wqkv"] = B(wqkv2)
    r3 = _layer(w3, x, c, S=100)
    assert np.array_equal(r3["attn"], r["attn"])


def test_o_projection_reads_the_concatenated_heads(base):
    w, x, c = base
    wo = np.zeros((2048, 1536))
    wo[128 * 3 + np.arange(128), np.arange(128)] = 1.0                     # o[:, :128] = head 3
    w2 = dict(w)
    w2["wo"] = B(wo)
    w2["w2"] = np.zeros_like(w["w2"])
    r = _layer(w2, x, c)
    xf = bf16_bits_to_f64(x)
    o = r["x2"] - xf
    expect = bf16_bits_to_f64(B(xf[:, :128] + r["attn"][:, 384:512])) - xf[:, :128]
    assert np.array_equal(o[:, :128], expect)
    assert np.array_equal(r["x2"][:, 128:], xf[:, 128:])


def test_swiglu_branches(base):
    # w1 = I (first 1536 of 6144 columns), w3 = 2 I, w2 = I back: d = bf16(silu(n2)) * bf16(2 n2), rounded
    w, x, c = base
    w2 = dict(w)
    eye = np.zeros((1536, 6144))
    eye[np.arange(1536), np.arange(1536)] = 1.0
    back = np.zeros((6144, 1536))
    back[np.arange(1536), np.arange(1536)] = 1.0
    w2["w1"], w2["w3"], w2["w2"] = B(eye), B(2 * eye), B(back)
    r = _layer(w2, x, c)
    n2 = r["n2"]
    rb = lambda v: bf16_bits_to_f64(B(v))  # noqa: E731
    d = rb(rb(silu(n2)) * rb(2 * n2))
    assert np.array_equal(r["x_out"], rb(r["x2"] + d))
    # swapping w1 and w3 is a different layer
    w3 = dict(w2)
    w3["w1"], w3["w3"] = w2["w3"], w2["w1"]
    assert not np.array_equal(_layer(w3, x, c)["x_out"], r["x_out"])
