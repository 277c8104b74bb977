"""Parity of the whole expert decoder layer and of its M = 64 projection with the fp64 oracle,
through the C ABI, on seeded inputs.

Bars. A projection output is one bf16 rounding of a float32 sum of exact bf16 products, the
oracle's one rounding of the float64 sum: within the float32 summation bound plus one rounding,
and nearly all equal. The layer: PCC >= 0.9999 on x_out, the level the pages report for their
device expert layer against their torch oracle (page code/alpamayo_tt/EXPERT_NOTES.md, section
"Accuracy": 0.99993 to 0.999998 over the layers), relative L2 <= 1e-2, and elementwise |got - ref| <= 0.05 +
2^-6 |ref| as a guard against a gross error in one element: the attention output already differs
from the oracle's by up to 1e-2 (its bf16 probabilities), and each of the bf16 roundings
after it (o, x2, n2, m, d, x_out; six in all) can fall the other way, moving an element by an ulp of up to
2^-7 |value|. Cache rows outside the tail unchanged; the tail within two bf16 ulps of the
oracle's plus the projection's float32 summation bound (its rows come through the projection's
rounding), and nearly all bits equal.
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


def _bits_normal(rng, shape, scale=1.0):
    return oracle.f64_to_bf16_bits(rng.standard_normal(shape) * scale)


def _packed(ax, w):
    """A device weight [K, N] in the projections' packed layout."""
    K, N = w.shape
    wp = torch.empty_like(w)
    ax.pack_weight_m64(w, K, N, wp)
    return wp


def _linear(ax, a_bits, w_bits):
    K, N = w_bits.shape
    A, W = up(a_bits), _packed(ax, up(w_bits))
    C = torch.zeros((64, N), dtype=torch.int16, device=DEV)
    nb = ax.linear_m64_workspace_bytes(K, N)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    ax.linear_m64(A, W, K, N, C, ws)
    torch.cuda.synchronize()
    return down(C)


def _check_linear(got_bits, a_bits, w_bits, label):
    a, w = bf16_to_f64(a_bits), bf16_to_f64(w_bits)
    ref = a @ w
    got = bf16_to_f64(got_bits)
    ref_r = bf16_to_f64(oracle.f64_to_bf16_bits(ref))
    # float32 sums of exact bf16 products: error at most K 2^-24 sum |a w| (a deterministic bound);
    # then one bf16 rounding, at most 2^-8 of the value
    acc = w.shape[0] * 2.0 ** -24 * (np.abs(a) @ np.abs(w))
    bound = 2.0 ** -8 * (np.abs(ref) + acc) + acc
    ratio = np.abs(got - ref) / bound
    i = np.unravel_index(np.argmax(ratio), ratio.shape)
    same = float(np.mean(got == ref_r))
    print(f"{label}: equal to the rounded float64 product {same:.5f}, max_abs {np.abs(got - ref).max():.3e}, "
          f"worst/bound {ratio[i]:.3f} at {i} (got {got[i]!r}, ref {ref[i]!r})", flush=True)
    assert ratio.max() <= 1.0
    assert same > 0.99


@pytest.mark.parametrize("K,N", [(128, 64), (1536, 4096), (2048, 1536), (1536, 6144), (6144, 1536), (384, 192)])
def test_linear_m64_matches_float64_product(ax, K, N):
    rng = np.random.default_rng(K * 7 + N)
    a = _bits_normal(rng, (64, K))
    w = _bits_normal(rng, (K, N), 1.0 / np.sqrt(K))
    say(f"linear_m64 K={K} N={N}")
    _check_linear(_linear(ax, a, w), a, w, f"linear K={K} N={N}")


def test_linear_m64_structure(ax):
    # identity weights copy A (every column of the tile maps to its own output column), a single
    # nonzero weight row picks one A column: a transposed operand or a swizzle slip fails these
    rng = np.random.default_rng(3)
    K = N = 256
    a = _bits_normal(rng, (64, K))
    eye = oracle.f64_to_bf16_bits(np.eye(K))
    say("linear_m64 identity")
    assert np.array_equal(_linear(ax, a, eye), a)
    w = np.zeros((K, N))
    w[37, :] = np.arange(N) + 1.0
    got = bf16_to_f64(_linear(ax, a, oracle.f64_to_bf16_bits(w)))
    ref = bf16_to_f64(oracle.f64_to_bf16_bits(bf16_to_f64(a)[:, 37:38] * (np.arange(N) + 1.0)[None, :]))
    assert np.array_equal(got, ref)


def test_pack_weight_m64_layout(ax):
    # packed block (32-column block j, 16-row step s), lane l, element e holds weight row
    # 16 s + 8 (l // 32) + e, column 32 j + l % 32: the matrix-core operand of lane l, checked
    # element by element against that definition
    K, N = 256, 192
    w = np.arange(K * N, dtype=np.uint32).reshape(K, N).astype(np.uint16)
    say("pack_weight_m64 layout")
    got = down(_packed(ax, up(w))).reshape(N // 32, K // 16, 64, 8)
    j, s, l, e = np.meshgrid(*(np.arange(n) for n in got.shape), indexing="ij")
    ref = w[16 * s + 8 * (l // 32) + e, 32 * j + l % 32]
    assert np.array_equal(got, ref)


def test_linear_m64_rejects_bad_shapes(ax):
    x = torch.zeros(64 * 256, dtype=torch.int16, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    for K, N in ((100, 64), (128, 96), (0, 64)):
        with pytest.raises(RuntimeError):
            ax.linear_m64(x, x, K, N, x, ws)


class LayerBufs:
    def __init__(self, ax, w, x, cache, S, Smax, rope_delta=0):
        self.S, self.Smax = S, Smax
        self.w = {k: (_packed(ax, up(v)) if v.ndim == 2 else up(v)) for k, v in w.items()}
        self.x = up(x)
        self.Kc, self.Vc = up(cache["Kc"]), up(cache["Vc"])
        cos, sin = ax.rope_tables(S + rope_delta)
        self.cos = torch.from_numpy(cos).to(DEV)
        self.sin = torch.from_numpy(sin).to(DEV)
        self.out_g = Guarded(64 * 1536 * 2)
        self.out = self.out_g.t.view(torch.int16).view(64, 1536)
        nb = ax.expert_layer_workspace_bytes(S, Smax)
        assert nb > 0
        self.ws_g = Guarded(nb)
        self.ws = self.ws_g.t

    def run(self, ax):
        w = self.w
        ax.expert_layer(self.x, w["ln1"], w["wqkv"], w["qn"], w["kn"], w["wo"], w["ln2"], w["w1"], w["w3"], w["w2"],
                        self.cos, self.sin, 1e-6, self.Kc, self.Vc, self.S, self.Smax, self.out, self.ws)
        torch.cuda.synchronize()
        self.out_g.check("out")
        self.ws_g.check("workspace")
        if self.ws is self.ws_g.t:
            assert_status_clear(ax, self.ws)


def _ref(w, x, cache, S, Smax, rope_delta=0):
    return oracle.expert_layer(x, w["ln1"], w["wqkv"], w["qn"], w["kn"], w["wo"], w["ln2"], w["w1"], w["w3"],
                               w["w2"], cache["Kc"], cache["Vc"], S, Smax, rope_delta)


def _check_layer(b, ref, cache, label):
    got = bf16_to_f64(down(b.out))
    r = ref["x_out"]
    m = metrics(got, r)
    ratio = np.abs(got - r) / (0.05 + 2.0 ** -6 * np.abs(r))
    i = np.unravel_index(np.argmax(ratio), ratio.shape)
    print(f"{label}: max_abs={m['max_abs']:.3e} pcc={m['pcc']:.7f} rel_l2={m['rel_l2']:.3e} "
          f"equal={np.mean(got == r):.4f} worst/bound={ratio[i]:.3f} (got {got[i]!r}, ref {r[i]!r})", flush=True)
    assert ratio.max() <= 1.0, m
    assert m["pcc"] >= 0.9999, m
    assert m["rel_l2"] <= 1e-2, m
    Smax = b.Smax
    for name, t in (("Kc", b.Kc), ("Vc", b.Vc)):
        c = down(t)
        assert np.array_equal(c[:, :Smax - 64], cache[name][:, :Smax - 64]), name
        tail, rt = bf16_to_f64(c[:, Smax - 64:]), ref[name + "_new"][:, Smax - 64:]
        rtf = bf16_to_f64(rt)
        # the float32 sum over the 1536 qkv inputs may be off by up to 1536 2^-24 sum |n1 w| (~2e-3
        # here) before its rounding, which matters for values near zero; a k element whose rounding
        # fell the other way reaches its rotate_half partner (d +- 64) through RoPE
        part = np.roll(rtf, 64, axis=-1) if name == "Kc" else 0.0
        assert (np.abs(tail - rtf) <= 2.0 ** -6 * (np.abs(rtf) + np.abs(part)) + 2e-3).all(), name
        same = float(np.mean(c[:, Smax - 64:] == rt))
        print(f"  {name} tail bits equal: {same:.5f}", flush=True)
        assert same > 0.98, name


@pytest.mark.parametrize("S,Smax,seed", [(128, 256, 1), (0, 64, 2), (1000, 1100, 3)])
def test_expert_layer_matches_oracle(ax, S, Smax, seed):
    w = synth.layer_weights(100 + seed)
    x = synth.residual_inputs(200 + seed)
    cache = synth.layer_inputs(Smax, S, 300 + seed)
    say(f"expert_layer S={S} Smax={Smax} seed={seed}")
    b = LayerBufs(ax, w, x, cache, S, Smax)
    b.run(ax)
    torch.cuda.synchronize()
    _check_layer(b, _ref(w, x, cache, S, Smax), cache, f"layer S={S} Smax={Smax}")


def test_expert_layer_rope_delta_and_full_cache(ax):
    # the tables passed in decide the positions (S + rope_delta + i); a cache with no hidden rows
    S, Smax, delta = 448, 512, 7
    w = synth.layer_weights(51)
    x = synth.residual_inputs(52)
    cache = synth.layer_inputs(Smax, S, 53)
    say(f"expert_layer S={S} Smax={Smax} rope_delta={delta}")
    b = LayerBufs(ax, w, x, cache, S, Smax, rope_delta=delta)
    b.run(ax)
    torch.cuda.synchronize()
    ref = _ref(w, x, cache, S, Smax, delta)
    _check_layer(b, ref, cache, f"layer S={S} Smax={Smax} delta={delta}")
    # the same call with the tables of rope_delta 0 is measurably different (the offset is used)
    ref0 = _ref(w, x, cache, S, Smax, 0)
    assert np.abs(ref0["x_out"] - ref["x_out"]).max() > 0.05


def test_expert_layer_workspace_reuse(ax):
    # one workspace sized for the larger shape serves a smaller one next (no state is kept in it)
    w = synth.layer_weights(61)
    x = synth.residual_inputs(62)
    big = synth.layer_inputs(2048, 1900, 63)
    small = synth.layer_inputs(256, 64, 64)
    say("expert_layer workspace reuse 1900/2048 then 64/256")
    b1 = LayerBufs(ax, w, x, big, 1900, 2048)
    b1.run(ax)
    b2 = LayerBufs(ax, w, x, small, 64, 256)
    b2.ws = b1.ws
    b2.run(ax)
    torch.cuda.synchronize()
    _check_layer(b1, _ref(w, x, big, 1900, 2048), big, "layer reuse, big")
    _check_layer(b2, _ref(w, x, small, 64, 256), small, "layer reuse, small")


def test_expert_layer_headline_shape(ax):
    S, Smax = 4700, 8192
    w = synth.layer_weights(11)
    x = synth.residual_inputs(12)
    cache = synth.layer_inputs(Smax, S, 13)
    say(f"expert_layer S={S} Smax={Smax}")
    b = LayerBufs(ax, w, x, cache, S, Smax)
    b.run(ax)
    torch.cuda.synchronize()
    _check_layer(b, _ref(w, x, cache, S, Smax), cache, "layer headline")
    # a second call on the updated cache and the same input: the tail is rewritten with the
    # same rows, so the output repeats bit for bit
    first = down(b.out).copy()
    b.run(ax)
    torch.cuda.synchronize()
    assert np.array_equal(down(b.out), first)


def test_expert_layer_chained_equals_plain(ax):
    # three layers run one after another: the chained calls (each layer's first norm made by the
    # previous call's last launch) give the plain calls' x_out bit for bit, and the first layer
    # matches the oracle
    S, Smax = 300, 512
    ws_ = [synth.layer_weights(700 + i) for i in range(3)]
    x = synth.residual_inputs(710)
    caches = [synth.layer_inputs(Smax, S, 720 + i) for i in range(3)]
    say(f"expert_layer_chained S={S} Smax={Smax}, 3 layers")
    lay = [LayerBufs(ax, ws_[i], x, caches[i], S, Smax) for i in range(3)]
    # plain: x -> layer 0 -> layer 1 -> layer 2
    xs = [up(x)] + [torch.empty((64, 1536), dtype=torch.int16, device=DEV) for _ in range(3)]
    for i, b in enumerate(lay):
        w = b.w
        ax.expert_layer(xs[i], w["ln1"], w["wqkv"], w["qn"], w["kn"], w["wo"], w["ln2"], w["w1"], w["w3"],
                        w["w2"], b.cos, b.sin, 1e-6, b.Kc, b.Vc, S, Smax, xs[i + 1], b.ws)
    torch.cuda.synchronize()
    plain = [down(t).copy() for t in xs[1:]]
    # chained, on fresh caches, with guarded outputs and norm buffers
    lay = [LayerBufs(ax, ws_[i], x, caches[i], S, Smax) for i in range(3)]
    xg = [Guarded(64 * 1536 * 2) for _ in range(3)]
    ng = [Guarded(64 * 1536 * 2) for _ in range(2)]
    xo = [g.t.view(torch.int16).view(64, 1536) for g in xg]
    n1 = [g.t.view(torch.int16).view(64, 1536) for g in ng]
    for i, b in enumerate(lay):
        w = b.w
        n1_in = None if i == 0 else n1[(i - 1) % 2]
        ln1 = w["ln1"] if i == 0 else None  # not read when n1_in is given
        nxt = lay[i + 1].w["ln1"] if i < 2 else None
        n1_out = n1[i % 2] if i < 2 else None
        ax.expert_layer_chained(up(x) if i == 0 else xo[i - 1], n1_in, ln1, w["wqkv"], w["qn"], w["kn"], w["wo"],
                                w["ln2"], w["w1"], w["w3"], w["w2"], b.cos, b.sin, 1e-6, b.Kc, b.Vc, S, Smax, xo[i],
                                nxt, n1_out, b.ws)
        torch.cuda.synchronize()
    for i in range(3):
        xg[i].check(f"x_out {i}")
        assert np.array_equal(down(xo[i]), plain[i]), f"layer {i}"
    for g in ng:
        g.check("n1")
    for b in lay:
        assert_status_clear(ax, b.ws)
    ref = _ref(ws_[0], x, caches[0], S, Smax)
    got = bf16_to_f64(plain[0])
    assert metrics(got, ref["x_out"])["pcc"] >= 0.9999
    # the norm buffer a chained call hands on is the oracle's norm of its x_out, within a bf16 rounding
    n1_ref = oracle.rms_norm(bf16_to_f64(plain[1]), bf16_to_f64(ws_[2]["ln1"]), 1e-6)
    got_n1 = bf16_to_f64(down(n1[1]))
    assert (np.abs(got_n1 - n1_ref) <= 2.0 ** -8 * np.abs(n1_ref) + 1e-30).all()


def test_expert_layer_chained_rejects_bad_arguments(ax):
    S, Smax = 64, 128
    b = LayerBufs(ax, synth.layer_weights(730), synth.residual_inputs(731), synth.layer_inputs(Smax, S, 732), S, Smax)
    w = b.w
    n = torch.empty((64, 1536), dtype=torch.int16, device=DEV)

    def call(**kw):
        a = dict(x_in=b.x, n1_in=None, ln1=w["ln1"], ln1_next=None, n1_out=None, x_out=b.out)
        a.update(kw)
        ax.expert_layer_chained(a["x_in"], a["n1_in"], a["ln1"], w["wqkv"], w["qn"], w["kn"], w["wo"], w["ln2"],
                                w["w1"], w["w3"], w["w2"], b.cos, b.sin, 1e-6, b.Kc, b.Vc, S, Smax, a["x_out"],
                                a["ln1_next"], a["n1_out"], b.ws)

    for kw in (dict(ln1=None), dict(ln1_next=w["ln1"]), dict(n1_out=n), dict(ln1_next=w["ln1"], n1_out=b.x),
               dict(ln1_next=w["ln1"], n1_out=b.out), dict(x_out=b.x)):
        with pytest.raises(RuntimeError):
            call(**kw)
    call(ln1_next=w["ln1"], n1_out=n)  # valid
    torch.cuda.synchronize()


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("layer", [0, 63])
def test_layer_benchmark_inputs_match_oracle(ax, layer):
    # the benchmark's own inputs: device-seeded weights of this layer (packed as the benchmark
    # packs them), the layer's cache, the first residual; copied back and checked against the oracle
    S, Smax = 4700, 8192
    say(f"layer benchmark inputs, layer {layer}")
    w = synth.device_layer_weights(layer, DEV)
    Kc, Vc = (t.contiguous() for t in synth.device_cache(Smax, S, layer, DEV))
    g = torch.Generator(device=DEV)
    g.manual_seed(11000)
    x = torch.randn((64, 1536), generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    host = {k: _bits(v) for k, v in w.items()}
    cache = {"Kc": _bits(Kc), "Vc": _bits(Vc)}
    xb = _bits(x)
    packed = {k: (_packed(ax, v) if v.dim() == 2 else v) for k, v in w.items()}
    cos, sin = (torch.from_numpy(t).to(DEV) for t in ax.rope_tables(S))
    out = torch.zeros((64, 1536), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(ax.expert_layer_workspace_bytes(S, Smax), dtype=torch.uint8, device=DEV)
    ax.expert_layer(x, packed["ln1"], packed["wqkv"], packed["qn"], packed["kn"], packed["wo"], packed["ln2"],
                    packed["w1"], packed["w3"], packed["w2"], cos, sin, 1e-6, Kc, Vc, S, Smax, out, ws)
    torch.cuda.synchronize()
    ref = _ref(host, xb, cache, S, Smax)
    got = bf16_to_f64(_bits(out))
    m = metrics(got, ref["x_out"])
    print(f"layer {layer}: max_abs={m['max_abs']:.3e} pcc={m['pcc']:.7f} rel_l2={m['rel_l2']:.3e}", flush=True)
    assert m["pcc"] >= 0.9999 and m["rel_l2"] <= 1e-2, m
    assert (np.abs(got - ref["x_out"]) <= 0.05 + 2.0 ** -6 * np.abs(ref["x_out"])).all()


def test_layer_graph_replay_equals_eager(ax):
    # the layer's nine launches captured in one graph, replayed three times with eager work in
    # between: every replay equals the eager result bit for bit
    S, Smax = 1000, 2048
    w = synth.layer_weights(41)
    x = synth.residual_inputs(42)
    cache = synth.layer_inputs(Smax, S, 43)
    say("layer graph capture / replay x3")
    b = LayerBufs(ax, w, x, cache, S, Smax)
    b.run(ax)
    torch.cuda.synchronize()
    eager = down(b.out).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    wt = b.w
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            ax.expert_layer(b.x, wt["ln1"], wt["wqkv"], wt["qn"], wt["kn"], wt["wo"], wt["ln2"], wt["w1"], wt["w3"],
                            wt["w2"], b.cos, b.sin, 1e-6, b.Kc, b.Vc, S, Smax, b.out, b.ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        b.out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(down(b.out), eager), f"replay {rep}"
        torch.randn(1 << 20, device=DEV).sum().item()   # eager work between replays
