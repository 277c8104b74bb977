"""Inputs at the edges of the number range, and the failure path of the bounded waits.

- Value rows of magnitude ~2^-120 (about 7.5e-37, normal in bf16 and float32; the smallest
  elements become denormal) in one key range among N(0,1) ranges, and in every visible row: the
  split partials carry a power-of-two scale, so neither the partial nor its row sum may overflow
  or underflow. With every row tiny the result is compared at the inputs' own scale (both sides
  multiplied by 2^120, exactly), where the usual bars apply.
- One value column 256 times larger than the rest: every other column keeps the usual absolute
  bar, i.e. the outlier costs its neighbours no precision (each float16 element keeps 11
  significant bits within 2^14 of its group's largest value).
- The same for the fp8 cache (the value scales are what is tiny there: float32 denormals).
- The bounded in-workgroup waits: with the wait limit forced down to one poll from the host, the
  waits give up, every workgroup still finishes, and the workspace status word says so.
"""
import numpy as np
import pytest
import torch

import oracle
from flow_matching_action_amd import synth

from gpu_util import DEV, Guarded, Layer, assert_status_clear, bf16_to_f64, down, metrics, say, up

pytestmark = pytest.mark.gpu

TINY = 2.0 ** -120


@pytest.fixture(scope="module")
def ax():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from flow_matching_action_amd import ax as lib
    return lib


def scaled_bits(bits: np.ndarray, factor: float) -> np.ndarray:
    """bf16 bits of the values times factor (a power of two: exact unless the result is denormal)."""
    return oracle.f64_to_bf16_bits(bf16_to_f64(bits) * factor)


def ref_layer(inp):
    return oracle.expert_attn_layer(inp["q"], inp["k"], inp["v"], inp["gq"], inp["gk"], inp["Kc"], inp["Vc"],
                                    inp["S"], inp["Smax"], inp["rope_delta"])


def bars(got: np.ndarray, ref: np.ndarray, label: str, scale: float = 1.0) -> dict:
    """max-abs 1e-2 and PCC 0.9999 on got * scale against ref * scale (scale a power of two)."""
    m = metrics(got * scale, ref * scale)
    print(f"{label}: max_abs={m['max_abs']:.3e} pcc={m['pcc']:.7f} rel_l2={m['rel_l2']:.3e} (x{scale:g})",
          flush=True)
    assert np.all(np.isfinite(got)), label
    assert m["max_abs"] <= 1e-2, m
    assert m["pcc"] >= 0.9999, m
    return m


# ----------------------------------------------------------------- bf16 cache
def test_tiny_value_rows_in_one_key_range(ax):
    S, Smax = 2000, 4096
    inp = synth.layer_inputs(Smax, S, seed=501)
    lo, hi = 480, 640   # the fourth of the 160-key ranges this shape is split into
    inp["Vc"] = inp["Vc"].copy()
    inp["Vc"][:, lo:hi] = scaled_bits(inp["Vc"][:, lo:hi], TINY)
    say(f"bf16 tiny value rows [{lo}, {hi}) S={S} Smax={Smax}")
    L = Layer(inp, ax)
    got = bf16_to_f64(L.run(ax))
    bars(got, ref_layer(inp)["out"], "tiny rows in one range")


def test_tiny_value_rows_everywhere(ax):
    S, Smax = 2000, 4096
    inp = synth.layer_inputs(Smax, S, seed=502)
    inp["Vc"] = inp["Vc"].copy()
    inp["Vc"][:, :S] = scaled_bits(inp["Vc"][:, :S], TINY)
    inp["v"] = scaled_bits(inp["v"], TINY)
    say(f"bf16 every visible value row tiny S={S} Smax={Smax}")
    L = Layer(inp, ax)
    got = bf16_to_f64(L.run(ax))
    ref = ref_layer(inp)["out"]
    assert np.max(np.abs(ref)) < 2.0 ** -110
    bars(got, ref, "all value rows tiny", scale=2.0 ** 120)
    # elements of ordinary size (at the inputs' scale) keep a small relative error
    big = np.abs(ref) >= 0.05 * TINY
    rel = np.abs(got[big] - ref[big]) / np.abs(ref[big])
    print(f"relative error of elements >= 0.05 x 2^-120: max {rel.max():.3e}", flush=True)
    assert rel.max() <= 2.0 ** -5


def test_outlier_value_column(ax):
    S, Smax = 3000, 4096
    col = 37                     # in the second 32-column quarter
    inp = synth.layer_inputs(Smax, S, seed=503)
    for name in ("Vc", "v"):
        inp[name] = inp[name].copy()
        inp[name][..., col] = scaled_bits(inp[name][..., col], 256.0)
    say(f"bf16 value column {col} x256 S={S} Smax={Smax}")
    L = Layer(inp, ax)
    got = bf16_to_f64(L.run(ax))
    ref = ref_layer(inp)["out"]
    err = np.abs(got - ref)
    others = np.ones(128, bool)
    others[col] = False
    print(f"outlier column: max err {err[..., col].max():.3e} (|ref| up to {np.abs(ref[..., col]).max():.2f}); "
          f"other columns: max err {err[..., others].max():.3e}", flush=True)
    # every element: the usual absolute bar at its column's scale plus its own bf16 rounding
    assert np.all(err[..., others] <= 1e-2 + 2.0 ** -8 * np.abs(ref[..., others]))
    assert np.all(err[..., col] <= 256 * 1e-2 + 2.0 ** -8 * np.abs(ref[..., col]))


# ----------------------------------------------------------------- fp8 cache
def _fp8_attention(ax, inp: dict, q_bits: np.ndarray, label: str) -> tuple[np.ndarray, np.ndarray]:
    """ax_expert_attn_fp8 on given roped q bits and a cache whose tail is already written; the
    oracle's attention over the same dequantised cache rows and the same q values."""
    S, Smax = inp["S"], inp["Smax"]
    Kc8, Ks, Vc8, Vs = inp["Kc8"], inp["Ks"], inp["Vc8"], inp["Vs"]
    K = oracle.dequantize_rows_e4m3(Kc8, Ks)
    V = oracle.dequantize_rows_e4m3(Vc8, Vs)
    mask = oracle.build_mask(S, Smax)
    ref = oracle.attention(bf16_to_f64(q_bits), K, V, mask, 128 ** -0.5)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    dKc, dKs, dVc, dVs = t(Kc8), t(Ks), t(Vc8), t(Vs)
    out_g = Guarded(16 * 64 * 128 * 2)
    out = out_g.t.view(torch.int16).view(16, 64, 128)
    ws_g = Guarded(ax.expert_attn_fp8_workspace_bytes(S, Smax))
    say(label)
    ax.expert_attn_fp8(up(q_bits), None, None, dKc, dKs, dVc, dVs, S, Smax, out, ws_g.t)
    torch.cuda.synchronize()
    out_g.check("out")
    ws_g.check("workspace")
    assert_status_clear(ax, ws_g.t)
    return bf16_to_f64(down(out)), ref


def _roped_q_bits(inp: dict) -> np.ndarray:
    q = bf16_to_f64(inp["q"])
    cos, sin = oracle.rope_tables(inp["S"] + inp["rope_delta"])
    return oracle.f64_to_bf16_bits(oracle.apply_rope(oracle.rms_norm(q, bf16_to_f64(inp["gq"])), cos, sin))


def test_fp8_tiny_value_scales_in_one_key_range(ax):
    S, Smax = 4000, 4096
    inp = synth.layer_inputs_fp8(Smax, S, seed=511)
    lo, hi = 512, 640
    inp["Vs"] = inp["Vs"].copy()
    inp["Vs"][:, lo:hi] *= np.float32(2.0 ** -124)    # 2^-128 .. 2^-130: float32 denormals, exact
    got, ref = _fp8_attention(ax, inp, _roped_q_bits(inp), f"fp8 tiny value scales [{lo}, {hi}) S={S}")
    bars(got, ref, "fp8 tiny scales in one range")


def test_fp8_tiny_value_scales_everywhere(ax):
    # Value rows quantised over the whole e4m3 range (codes up to 448, scale max|x| / 448), the
    # scales then multiplied by 2^-121: float32 denormals near 2^-128. Few keys keep the outputs
    # (averages of the value rows) inside bf16's normal range, where the output itself is exact
    # to 2^-9; both sides are compared at the rows' own scale.
    S, Smax = 256, 512
    inp = synth.layer_inputs_fp8(Smax, S, seed=512)
    rng = np.random.Generator(np.random.PCG64(5120))
    codes, scales = oracle.quantize_rows_e4m3(rng.standard_normal((8, Smax, 128), dtype=np.float32))
    inp["Vc8"] = codes
    inp["Vs"] = (scales * np.float32(2.0 ** -121)).astype(np.float32)
    assert np.all(inp["Vs"] < np.float32(2.0 ** -126))
    got, ref = _fp8_attention(ax, inp, _roped_q_bits(inp), f"fp8 every value scale a float32 denormal S={S}")
    assert np.max(np.abs(ref)) < 2.0 ** -110
    bars(got, ref, "fp8 all value scales tiny", scale=2.0 ** 121)


def test_fp8_outlier_value_column(ax):
    S, Smax = 4000, 4096
    col = 70
    inp = synth.layer_inputs_fp8(Smax, S, seed=513)
    # the column's codes carry 2^4 more (e4m3 keeps 3 mantissa bits exactly under a power-of-two
    # shift while it stays below 448): rows whose column code would saturate are left as they are
    vals = oracle.e4m3_bits_to_f64(inp["Vc8"][..., col])
    scaled = vals * 16.0
    ok = np.abs(scaled) <= 448.0
    codes = inp["Vc8"].copy()
    codes[..., col] = np.where(ok, oracle.f64_to_e4m3_bits(scaled), codes[..., col])
    inp["Vc8"] = codes
    got, ref = _fp8_attention(ax, inp, _roped_q_bits(inp), f"fp8 value column {col} x16 S={S}")
    err = np.abs(got - ref)
    others = np.ones(128, bool)
    others[col] = False
    print(f"fp8 outlier column: max err {err[..., col].max():.3e}; other columns {err[..., others].max():.3e}",
          flush=True)
    assert np.all(err[..., others] <= 1e-2 + 2.0 ** -8 * np.abs(ref[..., others]))
    assert np.all(err[..., col] <= 16 * 1e-2 + 2.0 ** -8 * np.abs(ref[..., col]))


# ----------------------------------------------------------------- bounded waits
def test_expired_waits_are_reported(ax):
    inp = synth.layer_inputs(1024, 700, seed=521)
    try:
        ax.debug_set_wait_limit(1)
        say("bf16 layer attention with the wait limit forced to one poll")
        L = Layer(inp, ax)
        ax.expert_layer_attn(L.q, L.k, L.v, L.gq, L.gk, L.cos, L.sin, 1e-6, L.Kc, L.Vc, L.S, L.Smax, L.out, L.ws)
        st = ax.workspace_status(L.ws)
        L.out_g.check("out")
        L.ws_g.check("workspace")
        print(f"status word with one-poll waits: {st:#x}", flush=True)
        assert st & ax.AX_STATUS_WAIT_EXPIRED
        fp8 = synth.layer_inputs_fp8(1024, 700, seed=522)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
        ws8 = Guarded(ax.expert_attn_fp8_workspace_bytes(700, 1024))
        out8 = torch.zeros((16, 64, 128), dtype=torch.int16, device=DEV)
        say("fp8 layer attention with the wait limit forced to one poll")
        ax.expert_layer_attn_fp8(L.q, L.k, L.v, L.gq, L.gk, L.cos, L.sin, 1e-6, t(fp8["Kc8"]), t(fp8["Ks"]),
                                 t(fp8["Vc8"]), t(fp8["Vs"]), 700, 1024, out8, ws8.t)
        st8 = ax.workspace_status(ws8.t)
        ws8.check("fp8 workspace")
        print(f"fp8 status word with one-poll waits: {st8:#x}", flush=True)
        assert st8 & ax.AX_STATUS_WAIT_EXPIRED
        d = synth.decode_inputs(1024, 700, seed=523)
        q, k, v, gq, gk = (up(d[n]) for n in ("q", "k", "v", "gq", "gk"))
        Kc, Vc = up(d["Kc"]), up(d["Vc"])
        cos, sin = (torch.from_numpy(a).to(DEV) for a in ax.rope_tables(700, 1))
        wsd = Guarded(ax.text_decode_workspace_bytes(700, 1024))
        outd = torch.zeros((64, 128), dtype=torch.int16, device=DEV)
        say("decode with the wait limit forced to one poll")
        ax.text_decode_attn(q, k, v, gq, gk, cos, sin, 1e-6, Kc, Vc, 700, 1024, outd, wsd.t)
        std = ax.workspace_status(wsd.t)
        wsd.check("decode workspace")
        print(f"decode status word with one-poll waits: {std:#x}", flush=True)
        assert std & ax.AX_STATUS_WAIT_EXPIRED
    finally:
        ax.debug_set_wait_limit(0)
    # back at the default limit the same call is clean and matches the oracle
    say("bf16 layer attention at the default wait limit")
    L2 = Layer(inp, ax)
    bars(bf16_to_f64(L2.run(ax)), ref_layer(inp)["out"], "default wait limit")
