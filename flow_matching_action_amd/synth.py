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
