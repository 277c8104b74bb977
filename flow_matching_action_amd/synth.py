"""Seeded synthetic inputs for the expert-attention step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the HIP path and the fp64 oracle can take their
inputs from it. All tensors are bf16 bit patterns (uint16), the format the
pages keep the KV cache and the q/k/v heads in (page
code/alpamayo_tt/EXPERT_NOTES.md, table "Layouts").

Recipe (single-layer workloads): numpy ``Generator(PCG64(seed))``, draws of
``standard_normal(dtype=float32)`` rounded to bf16 (nearest-even, by torch's
CPU cast), in this order: K cache, V cache, q, own k, own v, then the two
RMSNorm gammas as 1 + 0.1 * N(0, 1). Cache rows [S, Smax-64) (rows the mask
hides; the pages' tests fill them with 7.0) are then overwritten with 7.0,
exactly representable in bf16 (0x40E0). Rows [Smax-64, Smax) keep their random
draws: they are scratch that the tail write replaces.

fp8 caches (e4m3 codes + one float32 scale per (kv head, row)): the cache
values are N(0, 1) draws before quantisation. Each row gets a random
power-of-two scale 2^-e, e uniform in {4, 5, 6}, and its codes are torch's
nearest-even cast of x * 2^e (clipped to +-448) to float8_e4m3fn, so that
code * scale ~ x. These are input recipes, not the per-row max rule that the
layer applies to its own rows: this module holds no quantiser of the method.
Hidden rows hold the code of 7.0 with scale 1.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

N_Q_HEADS = 16
N_KV_HEADS = 8
N_TOK = 64
HEAD_DIM = 128
BF16_SEVEN = 0x40E0
E4M3_SEVEN = 0x4E   # 1.75 * 2^2


@dataclass(frozen=True)
class LayerWorkload:
    """One single-layer workload: cache length, valid rows, RoPE offset, seed."""
    name: str
    Smax: int
    S: int
    seed: int
    rope_delta: int = 0
    filler: float = 7.0


# The single-layer workloads (the Smax=8192 / S=4700 one is the headline; the
# Smax=256 one is small enough for the oracle to run in well under a second).
SMALL = LayerWorkload("layer Smax=256 S=128", 256, 128, 1)
HEADLINE = LayerWorkload("layer Smax=8192 S=4700", 8192, 4700, 2)
SHORT_CACHE = LayerWorkload("layer Smax=5120 S=4700", 5120, 4700, 3)
FULL_CACHE = LayerWorkload("layer Smax=8192 S=8128", 8192, 8128, 5)
WORKLOADS = {w.name: w for w in (SMALL, HEADLINE, SHORT_CACHE, FULL_CACHE)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), nearest-even, via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def layer_inputs(Smax: int, S: int, seed: int, rope_delta: int = 0, filler: float | None = 7.0,
                 n_kv: int = N_KV_HEADS, n_q: int = N_Q_HEADS, n_tok: int = N_TOK,
                 d: int = HEAD_DIM) -> dict:
    """Inputs of one layer as bf16 bits: Kc, Vc [n_kv,Smax,d], q [n_q,n_tok,d], k, v [n_kv,n_tok,d], gq, gk [d]."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def draw(*shape):
        return rng.standard_normal(shape, dtype=np.float32)

    Kc = f32_to_bf16_bits(draw(n_kv, Smax, d))
    Vc = f32_to_bf16_bits(draw(n_kv, Smax, d))
    q = f32_to_bf16_bits(draw(n_q, n_tok, d))
    k = f32_to_bf16_bits(draw(n_kv, n_tok, d))
    v = f32_to_bf16_bits(draw(n_kv, n_tok, d))
    gq = f32_to_bf16_bits(1.0 + 0.1 * draw(d))
    gk = f32_to_bf16_bits(1.0 + 0.1 * draw(d))
    if filler is not None and Smax - n_tok > S:
        fb = f32_to_bf16_bits(np.array([filler], np.float32))[0]
        Kc[:, S:Smax - n_tok, :] = fb
        Vc[:, S:Smax - n_tok, :] = fb
    return {"Kc": Kc, "Vc": Vc, "q": q, "k": k, "v": v, "gq": gq, "gk": gk,
            "S": S, "Smax": Smax, "rope_delta": rope_delta}


def workload_inputs(w: LayerWorkload) -> dict:
    return layer_inputs(w.Smax, w.S, w.seed, w.rope_delta, w.filler)


def f32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 array -> e4m3 codes (uint8): torch's CPU cast to float8_e4m3fn after clipping to +-448."""
    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def layer_inputs_fp8(Smax: int, S: int, seed: int, rope_delta: int = 0, filler: float | None = 7.0,
                     n_kv: int = N_KV_HEADS, n_q: int = N_Q_HEADS, n_tok: int = N_TOK,
                     d: int = HEAD_DIM) -> dict:
    """Inputs of one layer with an fp8 cache: Kc8, Vc8 [n_kv,Smax,d] uint8 e4m3 codes, Ks, Vs
    [n_kv,Smax] float32 scales; q, k, v, gq, gk as bf16 bits (as ``layer_inputs``).

    Draw order: K cache values, V cache values, q, own k, own v, the two gammas, then the
    scale exponents of the K rows and of the V rows.
    """
    rng = np.random.Generator(np.random.PCG64(seed))

    def draw(*shape):
        return rng.standard_normal(shape, dtype=np.float32)

    Kx = draw(n_kv, Smax, d)
    Vx = draw(n_kv, Smax, d)
    q = f32_to_bf16_bits(draw(n_q, n_tok, d))
    k = f32_to_bf16_bits(draw(n_kv, n_tok, d))
    v = f32_to_bf16_bits(draw(n_kv, n_tok, d))
    gq = f32_to_bf16_bits(1.0 + 0.1 * draw(d))
    gk = f32_to_bf16_bits(1.0 + 0.1 * draw(d))
    ek = rng.integers(4, 7, size=(n_kv, Smax))
    ev = rng.integers(4, 7, size=(n_kv, Smax))
    Kc8 = f32_to_e4m3_codes(Kx * np.exp2(ek).astype(np.float32)[..., None])
    Vc8 = f32_to_e4m3_codes(Vx * np.exp2(ev).astype(np.float32)[..., None])
    Ks = np.exp2(-ek).astype(np.float32)
    Vs = np.exp2(-ev).astype(np.float32)
    if filler is not None and Smax - n_tok > S:
        fc = f32_to_e4m3_codes(np.array([filler], np.float32))[0]
        for c8, sc in ((Kc8, Ks), (Vc8, Vs)):
            c8[:, S:Smax - n_tok, :] = fc
            sc[:, S:Smax - n_tok] = 1.0
    return {"Kc8": Kc8, "Ks": Ks, "Vc8": Vc8, "Vs": Vs, "q": q, "k": k, "v": v, "gq": gq, "gk": gk,
            "S": S, "Smax": Smax, "rope_delta": rope_delta}


def workload_inputs_fp8(w: LayerWorkload) -> dict:
    return layer_inputs_fp8(w.Smax, w.S, w.seed, w.rope_delta, w.filler)


# ---- the 64-layer x 10-step sequence, generated on the device ------------------------------------
# 64 distinct caches (2.1 GB at Smax 8192, far beyond the 256 MB Infinity Cache), fresh q / own k / own v
# for every (step, layer). Seeds: cache l -> 4000 + l, q/k/v of (step s, layer l) -> 5000 + 64 s + l,
# gammas of layer l -> 6000 + l.

def _dev_normal_bf16(shape, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def device_cache(Smax: int, S: int, layer: int, device, filler: float = 7.0):
    """K and V cache of one layer on the device (bf16 tensors [8, Smax, 128]); hidden rows = filler."""
    kv = _dev_normal_bf16((2, N_KV_HEADS, Smax, HEAD_DIM), 4000 + layer, device)
    if Smax - N_TOK > S:
        kv[:, :, S:Smax - N_TOK, :] = filler
    return kv[0], kv[1]


def device_cache_fp8(Smax: int, S: int, layer: int, device, filler: float = 7.0):
    """fp8 K and V cache of one layer on the device: codes (uint8 [8, Smax, 128]) and scales
    (float32 [8, Smax]) of each, by the recipe of ``layer_inputs_fp8`` (seed 8000 + layer)."""
    g = torch.Generator(device=device)
    g.manual_seed(8000 + layer)
    x = torch.randn((2, N_KV_HEADS, Smax, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    e = torch.randint(4, 7, (2, N_KV_HEADS, Smax), generator=g, device=device).to(torch.float32)
    codes = (x * torch.exp2(e)[..., None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    scales = torch.exp2(-e)
    if Smax - N_TOK > S:
        codes[:, :, S:Smax - N_TOK, :] = E4M3_SEVEN
        scales[:, :, S:Smax - N_TOK] = 1.0
    return codes[0], scales[0], codes[1], scales[1]


def decode_inputs(Smax: int, pos: int, seed: int, rope_delta: int = 0, n_kv: int = N_KV_HEADS,
                  n_q: int = 64, d: int = HEAD_DIM) -> dict:
    """Inputs of one text-model decode step as bf16 bits: Kc, Vc [n_kv,Smax,d], q [n_q,d] (64 query
    heads of the one new token), k, v [n_kv,d], gq, gk [d]. Draw order: K cache, V cache, q, k, v, the
    two gammas (1 + 0.1 N(0,1)). Rows [pos, Smax) of the caches hold 7.0: row pos is replaced by the
    step's own k/v, the rows after it are not yet written."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def draw(*shape):
        return rng.standard_normal(shape, dtype=np.float32)

    Kc = f32_to_bf16_bits(draw(n_kv, Smax, d))
    Vc = f32_to_bf16_bits(draw(n_kv, Smax, d))
    q = f32_to_bf16_bits(draw(n_q, d))
    k = f32_to_bf16_bits(draw(n_kv, d))
    v = f32_to_bf16_bits(draw(n_kv, d))
    gq = f32_to_bf16_bits(1.0 + 0.1 * draw(d))
    gk = f32_to_bf16_bits(1.0 + 0.1 * draw(d))
    Kc[:, pos:] = BF16_SEVEN
    Vc[:, pos:] = BF16_SEVEN
    return {"Kc": Kc, "Vc": Vc, "q": q, "k": k, "v": v, "gq": gq, "gk": gk, "pos": pos, "Smax": Smax,
            "rope_delta": rope_delta}


def device_decode_qkv(step: int, layer: int, device):
    """q [64,128], k and v [8,128] (bf16 tensors) of one text-model decode step (seed 9000 + 64 step + layer)."""
    t = _dev_normal_bf16((64 + 2 * N_KV_HEADS, HEAD_DIM), 9000 + 64 * step + layer, device)
    return t[:64], t[64:64 + N_KV_HEADS], t[64 + N_KV_HEADS:]


def device_layer_weights(layer: int, device, hidden: int = 1536, qkv: int = 4096, attn: int = 2048,
                         mlp: int = 6144) -> dict:
    """Weights of one expert decoder layer on the device (bf16 tensors, input-major), the recipe of
    ``layer_weights`` drawn with torch's device generator (seed 10000 + layer); qn and kn are the
    gammas of ``device_gammas(layer)``."""
    g = torch.Generator(device=device)
    g.manual_seed(10000 + layer)

    def draw(*shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)

    def mat(i, o):
        return (draw(i, o) / float(np.sqrt(i))).to(torch.bfloat16).contiguous()

    qn, kn = device_gammas(layer, device)
    return {"ln1": (1.0 + 0.1 * draw(hidden)).to(torch.bfloat16), "wqkv": mat(hidden, qkv),
            "qn": qn.contiguous(), "kn": kn.contiguous(), "wo": mat(attn, hidden),
            "ln2": (1.0 + 0.1 * draw(hidden)).to(torch.bfloat16), "w1": mat(hidden, mlp), "w3": mat(hidden, mlp),
            "w2": mat(mlp, hidden)}


def layer_weights(seed: int, hidden: int = 1536, qkv: int = 4096, attn: int = 2048, mlp: int = 6144) -> dict:
    """Random weights of one expert decoder layer as bf16 bits, stored input-major ([in, out]):
    ln1, ln2 [hidden] = 1 + 0.1 N(0,1); wqkv [hidden, qkv], wo [attn, hidden], w1 and w3 [hidden, mlp],
    w2 [mlp, hidden] = N(0,1) / sqrt(in), so that every product keeps unit scale; qn, kn [128] as the
    other gammas. Draw order: ln1, wqkv, qn, kn, wo, ln2, w1, w3, w2."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def draw(*shape):
        return rng.standard_normal(shape, dtype=np.float32)

    def mat(i, o):
        return f32_to_bf16_bits(draw(i, o) / np.float32(np.sqrt(i)))

    return {"ln1": f32_to_bf16_bits(1.0 + 0.1 * draw(hidden)), "wqkv": mat(hidden, qkv),
            "qn": f32_to_bf16_bits(1.0 + 0.1 * draw(128)), "kn": f32_to_bf16_bits(1.0 + 0.1 * draw(128)),
            "wo": mat(attn, hidden), "ln2": f32_to_bf16_bits(1.0 + 0.1 * draw(hidden)),
            "w1": mat(hidden, mlp), "w3": mat(hidden, mlp), "w2": mat(mlp, hidden)}


def residual_inputs(seed: int, n_tok: int = N_TOK, hidden: int = 1536) -> np.ndarray:
    """The residual stream entering a layer, [n_tok, hidden] bf16 bits of N(0,1) draws."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return f32_to_bf16_bits(rng.standard_normal((n_tok, hidden), dtype=np.float32))


def device_qkv(step: int, layer: int, device):
    """q [16,64,128], own k and v [8,64,128] (bf16 tensors) of one (step, layer)."""
    t = _dev_normal_bf16((N_Q_HEADS + 2 * N_KV_HEADS, N_TOK, HEAD_DIM), 5000 + 64 * step + layer, device)
    return t[:N_Q_HEADS], t[N_Q_HEADS:N_Q_HEADS + N_KV_HEADS], t[N_Q_HEADS + N_KV_HEADS:]


def device_gammas(layer: int, device):
    """q and k RMSNorm gammas [128] (bf16 tensors) of one layer: 1 + 0.1 * N(0, 1)."""
    g = torch.Generator(device=device)
    g.manual_seed(6000 + layer)
    t = 1.0 + 0.1 * torch.randn((2, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    t = t.to(torch.bfloat16)
    return t[0], t[1]
