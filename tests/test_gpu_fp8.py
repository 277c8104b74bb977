"""Parity of the fp8-cache path (e4m3 codes + float32 row scales) with the fp64 oracle, through the C ABI.

Bars: the attention output within max-abs 1e-2 and PCC >= 0.9999 of the oracle; the quantised V
tail (codes and scales) bit-exact; the quantised K tail bit-exact except where the kernel's bf16
roped k differs from the oracle's by its last bit (float32 vs float64 before one rounding), and
there within one code step; every other cache row and scale unchanged; the stand-alone tail write
bit-exact on given bf16 rows.
"""
import numpy as np
import pytest
import torch

import oracle
from flow_matching_action_amd import synth

from gpu_util import DEV, Guarded, assert_status_clear, bf16_to_f64, down, metrics, say, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ax():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from flow_matching_action_amd import ax as lib
    return lib


def up8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def down8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy()


class Layer8:
    """Device buffers of one fp8-cache layer (from synth.layer_inputs_fp8), output and workspace."""

    def __init__(self, inp: dict, ax):
        self.inp = inp
        self.S, self.Smax = inp["S"], inp["Smax"]
        self.q, self.k, self.v = up(inp["q"]), up(inp["k"]), up(inp["v"])
        self.gq, self.gk = up(inp["gq"]), up(inp["gk"])
        self.Kc, self.Vc = up8(inp["Kc8"]), up8(inp["Vc8"])
        self.Ks, self.Vs = up8(inp["Ks"]), up8(inp["Vs"])
        cos, sin = ax.rope_tables(self.S + inp["rope_delta"])
        self.cos, self.sin = torch.from_numpy(cos).to(DEV), torch.from_numpy(sin).to(DEV)
        self.out_g = Guarded(16 * 64 * 128 * 2)
        self.out = self.out_g.t.view(torch.int16).view(16, 64, 128)
        nbytes = ax.expert_attn_fp8_workspace_bytes(self.S, self.Smax)
        assert nbytes > 0
        self.ws_g = Guarded(nbytes)
        self.ws = self.ws_g.t
        assert self.Kc.shape == (8, self.Smax, 128) and self.Kc.dtype == torch.uint8
        assert self.Ks.shape == (8, self.Smax) and self.Ks.dtype == torch.float32
        assert self.Vc.shape == self.Kc.shape and self.Vs.shape == self.Ks.shape
        assert self.q.shape == (16, 64, 128) and self.k.shape == (8, 64, 128) and self.v.shape == (8, 64, 128)

    def run(self, ax, eps: float = 1e-6):
        ax.expert_layer_attn_fp8(self.q, self.k, self.v, self.gq, self.gk, self.cos, self.sin, eps, self.Kc, self.Ks,
                                 self.Vc, self.Vs, self.S, self.Smax, self.out, self.ws)
        torch.cuda.synchronize()
        self.out_g.check("out")
        self.ws_g.check("workspace")
        if self.ws is self.ws_g.t:
            assert_status_clear(ax, self.ws)
        return down(self.out)


def ref8(inp):
    return oracle.expert_attn_layer_fp8(inp["q"], inp["k"], inp["v"], inp["gq"], inp["gk"], inp["Kc8"], inp["Ks"],
                                        inp["Vc8"], inp["Vs"], inp["S"], inp["Smax"], inp["rope_delta"])


def check_out(got_bits, ref, label):
    m = metrics(bf16_to_f64(got_bits), ref["out"])
    print(f"{label}: max_abs={m['max_abs']:.3e} pcc={m['pcc']:.7f} rel_l2={m['rel_l2']:.3e}", flush=True)
    assert m["max_abs"] <= 1e-2, m
    assert m["pcc"] >= 0.9999, m


def check_cache(L: Layer8, ref, label):
    inp, t = L.inp, L.Smax - 64
    Kc, Vc, Ks, Vs = down8(L.Kc), down8(L.Vc), down8(L.Ks), down8(L.Vs)
    # untouched rows
    assert np.array_equal(Kc[:, :t], inp["Kc8"][:, :t]) and np.array_equal(Vc[:, :t], inp["Vc8"][:, :t])
    assert np.array_equal(Ks[:, :t], inp["Ks"][:, :t]) and np.array_equal(Vs[:, :t], inp["Vs"][:, :t])
    # V tail: a function of the given bf16 v only
    assert np.array_equal(Vc[:, t:], ref["v_tail_codes"]) and np.array_equal(Vs[:, t:], ref["v_tail_scales"])
    # K tail: from the kernel's own bf16 roped k
    kc, ks = Kc[:, t:], Ks[:, t:]
    same = kc == ref["k_tail_codes"]
    n_bad = int((~same).sum())
    print(f"{label}: K tail codes differing from the oracle's: {n_bad} of {same.size}; "
          f"scales differing: {int((ks != ref['k_tail_scales']).sum())} of {ks.size}", flush=True)
    assert n_bad <= same.size // 1000
    dv = np.abs(oracle.e4m3_bits_to_f64(kc) - oracle.e4m3_bits_to_f64(ref["k_tail_codes"]))
    step = np.abs(oracle.e4m3_bits_to_f64(ref["k_tail_codes"])) * 2.0 ** -3 + 2.0 ** -9
    assert np.all(dv <= step * 1.0001)
    assert np.all(np.abs(ks / ref["k_tail_scales"] - 1) <= 2.0 ** -7)


# ------------------------------------------------------------------------------ tail write
def test_fp8_tail_write_bit_exact(ax):
    inp = synth.layer_inputs(256, 128, seed=41)
    k = inp["k"].copy()
    v = inp["v"].copy()
    k[0, 0] = 0                                              # all-zero row: scale 1, codes 0
    k[0, 1] = oracle.f64_to_bf16_bits(np.full(128, 3.0e4))  # large values
    k[0, 2] = oracle.f64_to_bf16_bits(np.linspace(-1e-30, 1e-30, 128))   # tiny: subnormal bf16
    v[1, 3] = 0x8000                                         # negative zeros
    v[1, 3, 5] = oracle.f64_to_bf16_bits(2.0)
    v[2, 4] = oracle.f64_to_bf16_bits(np.r_[np.full(64, -7.5), np.full(64, 7.5 / 3)])  # ties after division
    Smax = 256
    say("cache_tail_write_fp8, 1024 rows")
    Kc = torch.full((8, Smax, 128), 0x11, dtype=torch.uint8, device=DEV)
    Vc = torch.full((8, Smax, 128), 0x22, dtype=torch.uint8, device=DEV)
    Ks = torch.full((8, Smax), 5.0, dtype=torch.float32, device=DEV)
    Vs = torch.full((8, Smax), 6.0, dtype=torch.float32, device=DEV)
    ax.cache_tail_write_fp8(up(k), up(v), Kc, Ks, Vc, Vs, Smax)
    torch.cuda.synchronize()
    kq, ksc = oracle.quantize_rows_e4m3(bf16_to_f64(k).astype(np.float32))
    vq, vsc = oracle.quantize_rows_e4m3(bf16_to_f64(v).astype(np.float32))
    Kn, Vn, Ksn, Vsn = down8(Kc), down8(Vc), down8(Ks), down8(Vs)
    assert np.array_equal(Kn[:, 192:], kq) and np.array_equal(Ksn[:, 192:], ksc)
    assert np.array_equal(Vn[:, 192:], vq) and np.array_equal(Vsn[:, 192:], vsc)
    assert (Kn[:, :192] == 0x11).all() and (Vn[:, :192] == 0x22).all()
    assert (Ksn[:, :192] == 5.0).all() and (Vsn[:, :192] == 6.0).all()


# ------------------------------------------------------------------------------ the layer step
@pytest.mark.parametrize("S,Smax", [(128, 256), (4700, 8192), (8128, 8192)])
def test_fp8_layer_matches_oracle(ax, S, Smax):
    inp = synth.layer_inputs_fp8(Smax, S, seed=5 if S == 8128 else 50 + S)
    say(f"expert_layer_attn_fp8 S={S} Smax={Smax}")
    L = Layer8(inp, ax)
    got = L.run(ax)
    ref = ref8(inp)
    check_out(got, ref, f"fp8 S={S} Smax={Smax}")
    check_cache(L, ref, f"fp8 S={S} Smax={Smax}")


@pytest.mark.parametrize("S,Smax", [(0, 64), (0, 256), (1, 128), (31, 160), (33, 200), (191, 256), (2050, 4000),
                                    (3500, 3584), (5500, 5568), (6500, 6592), (7500, 7616), (9000, 9088),
                                    (10000, 10112), (11904, 12288), (12000, 12288)])
def test_fp8_layer_edge_shapes(ax, S, Smax):
    # one cache split through twelve 32-key blocks and splits with a partial last block
    inp = synth.layer_inputs_fp8(Smax, S, seed=2000 + S)
    say(f"expert_layer_attn_fp8 edge S={S} Smax={Smax}")
    L = Layer8(inp, ax)
    check_out(L.run(ax), ref8(inp), f"fp8 S={S} Smax={Smax}")


def test_fp8_hidden_rows_are_never_read(ax):
    inp = synth.layer_inputs_fp8(1024, 300, seed=42)
    say("fp8 hidden rows: 7.0 vs NaN codes and NaN scales")
    a = Layer8(inp, ax).run(ax)
    bad = dict(inp)
    for n in ("Kc8", "Vc8"):
        bad[n] = inp[n].copy()
        bad[n][:, 300:960] = 0x7F
    for n in ("Ks", "Vs"):
        bad[n] = inp[n].copy()
        bad[n][:, 300:960] = np.nan
    b = Layer8(bad, ax).run(ax)
    assert np.array_equal(a, b)


def test_fp8_attn_entry_points_equal_layer(ax):
    # ax_expert_attn_fp8 on the library's roped q/k with the tail folded in, then with the tail
    # already in the cache, and the split + combine pair, all equal the composite call bit for bit.
    inp = synth.layer_inputs_fp8(2048, 1500, seed=43)
    say("expert_attn_fp8(k_own, v_own), expert_attn_fp8(NULL, NULL), split + combine vs expert_layer_attn_fp8")
    L = Layer8(inp, ax)
    ref_bits = L.run(ax)
    qo, ko = torch.empty_like(L.q), torch.empty_like(L.k)
    ax.qk_norm_rope(L.q, L.k, L.gq, L.gk, L.cos, L.sin, 1e-6, qo, ko)
    Kc, Vc, Ks, Vs = up8(inp["Kc8"]), up8(inp["Vc8"]), up8(inp["Ks"]), up8(inp["Vs"])
    out = torch.empty_like(L.out)
    ax.expert_attn_fp8(qo, ko, L.v, Kc, Ks, Vc, Vs, 1500, 2048, out, L.ws)
    torch.cuda.synchronize()
    assert np.array_equal(down(out), ref_bits)
    for a, b in ((Kc, L.Kc), (Vc, L.Vc), (Ks, L.Ks), (Vs, L.Vs)):
        assert np.array_equal(down8(a), down8(b))
    out.zero_()
    ax.expert_attn_fp8(qo, None, None, Kc, Ks, Vc, Vs, 1500, 2048, out, L.ws)
    torch.cuda.synchronize()
    assert np.array_equal(down(out), ref_bits)
    Kc2, Vc2, Ks2, Vs2 = up8(inp["Kc8"]), up8(inp["Vc8"]), up8(inp["Ks"]), up8(inp["Vs"])
    ws = torch.zeros_like(L.ws)
    out.zero_()
    ax.expert_layer_attn_fp8_split(L.q, L.k, L.v, L.gq, L.gk, L.cos, L.sin, 1e-6, Kc2, Ks2, Vc2, Vs2, 1500, 2048, ws)
    ax.expert_attn_fp8_combine(ws, 1500, 2048, out)
    torch.cuda.synchronize()
    assert np.array_equal(down(out), ref_bits)
    assert np.array_equal(down8(Kc2), down8(L.Kc)) and np.array_equal(down8(Ks2), down8(L.Ks))


def test_fp8_graph_replay_equals_eager(ax):
    # the fp8 step captured in a hipGraph (as the benchmark runs it): every replay, with eager
    # work between them, equals the eager call bit for bit, caches included
    inp = synth.layer_inputs_fp8(4096, 3000, seed=36)
    say("fp8 graph capture / replay x3")
    L = Layer8(inp, ax)
    eager = L.run(ax)
    caches = [down8(t) for t in (L.Kc, L.Ks, L.Vc, L.Vs)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        L.out.zero_()
        with torch.cuda.graph(g, stream=s):
            ax.expert_layer_attn_fp8(L.q, L.k, L.v, L.gq, L.gk, L.cos, L.sin, 1e-6, L.Kc, L.Ks, L.Vc, L.Vs, L.S,
                                     L.Smax, L.out, L.ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        L.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(down(L.out), eager), f"replay {rep}"
        for a, b in zip(caches, (L.Kc, L.Ks, L.Vc, L.Vs)):
            assert np.array_equal(a, down8(b)), f"replay {rep}: cache"
        assert_status_clear(ax, L.ws)
        torch.randn(1 << 20, device=DEV).sum().item()   # eager work between replays


def test_fp8_repeat_is_bitwise_deterministic(ax):
    inp = synth.layer_inputs_fp8(8192, 8128, seed=5)
    say("fp8 determinism x3, S=8128")
    L = Layer8(inp, ax)
    a = L.run(ax)
    torch.randn(1 << 22, device=DEV).sum().item()
    b = L.run(ax)
    c = L.run(ax)
    assert np.array_equal(a, b) and np.array_equal(a, c)


@pytest.mark.parametrize("step,layer", [(0, 0), (9, 63)])
def test_fp8_benchmark_inputs_match_oracle(ax, step, layer):
    # the fp8 benchmark's own inputs (device-generated cache of layer l, fresh q/k/v) at S=8128
    S, Smax = 8128, 8192
    say(f"fp8 benchmark inputs, Euler step {step}, layer {layer}")
    Kc, Ks, Vc, Vs = (t.contiguous() for t in synth.device_cache_fp8(Smax, S, layer, DEV))
    q, k, v = (t.contiguous() for t in synth.device_qkv(step, layer, DEV))
    gq, gk = (t.contiguous() for t in synth.device_gammas(layer, DEV))
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    inp = {"q": bits(q), "k": bits(k), "v": bits(v), "gq": bits(gq), "gk": bits(gk), "Kc8": down8(Kc),
           "Ks": down8(Ks), "Vc8": down8(Vc), "Vs": down8(Vs), "S": S, "Smax": Smax, "rope_delta": 0}
    ref = ref8(inp)
    cos, sin = (torch.from_numpy(t).to(DEV) for t in ax.rope_tables(S))
    out = torch.empty((16, 64, 128), dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(ax.expert_attn_fp8_workspace_bytes(S, Smax), dtype=torch.uint8, device=DEV)
    ax.expert_layer_attn_fp8(q, k, v, gq, gk, cos, sin, 1e-6, Kc, Ks, Vc, Vs, S, Smax, out, ws)
    torch.cuda.synchronize()
    check_out(bits(out), ref, f"fp8 sequence s={step} l={layer}")
    assert np.array_equal(down8(Vc)[:, Smax - 64:], ref["v_tail_codes"])


def test_fp8_scores_over_wide_range_query_rows(ax):
    # The scores take the K codes on the fp8 matrix cores against q in two e4m3 parts of the row
    # scaled by a power of two. Given bf16 q rows of very different sizes (zero, 1e-30, 2^-6 .. 64)
    # whose elements spread over 16 binades (and rows with one nonzero element), the output stays
    # within 2^-6 of each row's largest output element of the fp64 oracle on the same bf16 q: the
    # bf16 rounding of P and of the output (2^-9 each, relative) weigh more where a row's output is
    # smaller than the values it averages (5.4e-3 measured at worst). The large rows make the
    # softmax peaked, where an error of a few percent in q moves the output by far more: with q's
    # first e4m3 part alone, 410 rows of this input miss 2^-7 and the worst is 0.89.
    S, Smax = 4700, 8192
    inp = synth.layer_inputs_fp8(Smax, S, seed=77)
    rng = np.random.Generator(np.random.PCG64(78))
    mags = np.array([0.0, 1e-30, 2.0 ** -6, 1.0, 4.0, 16.0, 64.0])
    rows = 16 * 64
    mag = mags[np.arange(rows) % len(mags)].reshape(16, 64, 1)
    x = rng.standard_normal((16, 64, 128)) * np.exp2(-rng.uniform(0, 16, (16, 64, 128))) * mag
    x[3, 5] = 0.0
    x[3, 5, 17] = 9.5                                        # one nonzero element
    x[7, 9] = 0.0
    x[7, 9, 100] = -3.0e-20
    q_bits = oracle.f64_to_bf16_bits(x)
    q = bf16_to_f64(q_bits)
    say(f"expert_attn_fp8 wide-range q rows, S={S} Smax={Smax}")
    Kc, Vc, Ks, Vs = up8(inp["Kc8"]), up8(inp["Vc8"]), up8(inp["Ks"]), up8(inp["Vs"])
    out_g = Guarded(16 * 64 * 128 * 2)
    out = out_g.t.view(torch.int16).view(16, 64, 128)
    ws_g = Guarded(ax.expert_attn_fp8_workspace_bytes(S, Smax))
    ax.expert_attn_fp8(up(q_bits), None, None, Kc, Ks, Vc, Vs, S, Smax, out, ws_g.t)
    torch.cuda.synchronize()
    out_g.check("out")
    ws_g.check("workspace")
    assert_status_clear(ax, ws_g.t)
    got = bf16_to_f64(down(out))
    K = oracle.dequantize_rows_e4m3(inp["Kc8"], inp["Ks"])
    V = oracle.dequantize_rows_e4m3(inp["Vc8"], inp["Vs"])
    ref = oracle.attention(q, K, V, oracle.build_mask(S, Smax, 128, 64), 128 ** -0.5)
    err = np.abs(got - ref).max(axis=-1)
    big = np.abs(ref).max(axis=-1)
    worst = float((err / big).max())
    print(f"wide-range q: worst row error / row max = {worst:.3e} (bound 2^-6 = {2.0 ** -6:.3e})", flush=True)
    assert np.all(np.isfinite(got))
    assert np.all(err <= 2.0 ** -6 * big)
