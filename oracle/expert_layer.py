"""fp64 oracle of one whole action-expert decoder layer with given weights (test infrastructure).

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; the product path never touches it.

What it computes follows page ``code/alpamayo_tt/EXPERT_NOTES.md``, section "Layouts" (the
per-layer op list and the weight-shape table), and page ``code/alpamayo_tt/expert.py``,
``TTExpert.layer``: the residual x is RMS-normed and projected to q, k and v heads (16 + 8 + 8 of
width 128, in that column order of the fused weight); the attention step of ``expert_attn_layer``
runs on them; its heads are concatenated, projected back to the residual width and added to x;
that sum is RMS-normed again and goes through the SwiGLU MLP (silu of one projection times
another, then the down projection), whose result is added once more. Shapes: residual
[64, 1536]; the fused qkv weight [1536, 4096]; the output projection [2048, 1536]; the two MLP
up projections [1536, 6144] and the down projection [6144, 1536]; every weight is stored
input-major ([in, out], the transpose of the HF layout), as the pages keep them.

Reading: every op hands a bf16 tensor to the next, as ttnn ops do
(the pages' activations are bf16 throughout), so the oracle rounds to bf16 at each op boundary
of the list above and computes inside each op in float64: the residual inputs of the adds, the
normed activations, qkv, the attention output, o, g = silu(n2 w1), u = n2 w3, m = g u, d.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_bits_to_f64, f64_to_bf16_bits
from .expert_attn import EPS, N_KV_HEADS, N_Q_HEADS, expert_attn_layer, rms_norm

HIDDEN = 1536
QKV = 4096
ATTN_OUT = N_Q_HEADS * 128
MLP = 6144


def _bf(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 and return them as float64 (an op's bf16 output)."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def expert_layer(x, ln1, wqkv, qn, kn, wo, ln2, w1, w3, w2, Kc, Vc, S: int, Smax: int, rope_delta: int = 0,
                 eps: float = EPS) -> dict:
    """One decoder layer: x [64, 1536] and every weight as bf16 bits; caches [8, Smax, 128] bits.
    The residual RMSNorms are ``rms_norm`` over the 1536 columns (eps as for the heads).

    Returns ``x_out`` [64, 1536] float64 (bf16 values), the intermediate bf16 tensors (as float64)
    ``n1``, ``qkv``, ``attn`` ([64, 2048], heads concatenated), ``x2``, ``n2``, ``m``, and the
    updated caches ``Kc_new``/``Vc_new`` (bits).
    """
    x = bf16_bits_to_f64(x)
    w = {k: bf16_bits_to_f64(v) for k, v in dict(ln1=ln1, wqkv=wqkv, wo=wo, ln2=ln2, w1=w1, w3=w3, w2=w2).items()}
    n1 = _bf(rms_norm(x, w["ln1"], eps))
    qkv = _bf(n1 @ w["wqkv"])                                   # [64, 4096]
    t = x.shape[0]
    q = qkv[:, :N_Q_HEADS * 128].reshape(t, N_Q_HEADS, 128).transpose(1, 0, 2)             # [16, 64, 128]
    k = qkv[:, N_Q_HEADS * 128:(N_Q_HEADS + N_KV_HEADS) * 128].reshape(t, N_KV_HEADS, 128).transpose(1, 0, 2)
    v = qkv[:, (N_Q_HEADS + N_KV_HEADS) * 128:].reshape(t, N_KV_HEADS, 128).transpose(1, 0, 2)
    att = expert_attn_layer(f64_to_bf16_bits(q), f64_to_bf16_bits(k), f64_to_bf16_bits(v), qn, kn, Kc, Vc, S, Smax,
                            rope_delta, eps)
    a = _bf(att["out"]).transpose(1, 0, 2).reshape(t, N_Q_HEADS * 128)                      # concat heads
    o = _bf(a @ w["wo"])
    x2 = _bf(x + o)
    n2 = _bf(rms_norm(x2, w["ln2"], eps))
    g = _bf(silu(n2 @ w["w1"]))
    u = _bf(n2 @ w["w3"])
    m = _bf(g * u)
    d = _bf(m @ w["w2"])
    x3 = _bf(x2 + d)
    return {"x_out": x3, "n1": n1, "qkv": qkv, "attn": a, "x2": x2, "n2": n2, "m": m,
            "Kc_new": att["Kc_new"], "Vc_new": att["Vc_new"]}
