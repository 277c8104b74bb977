"""fp64 oracle of the text model's single-token decode attention step (test infrastructure).

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; the product path never touches it.

What is computed, and where the pages define it (page ``code/alpamayo_tt/text.py``,
``TTTextModel._layer_decode`` and ``_decode_inputs_host``): one new token at cache position
``pos`` of a Qwen3-VL text layer with 64 query heads and 8 kv heads of width 128 -

* per-head RMSNorm of q and k with the ``qn``/``kn`` gammas (``_norm_sharded``);
* HF rotate_half RoPE of both at position ``pos + rope_delta`` (``rotary_embedding_hf`` with the
  tables of ``text_cos_sin`` for that one position);
* the roped k and the raw v written into cache row ``pos`` (``paged_update_cache`` with
  ``update_idxs_tensor = pos``);
* attention of each query head h over cache rows ``[0, pos]`` of kv head ``h // 8`` with scale
  ``head_dim ** -0.5`` (``scaled_dot_product_attention_decode`` with ``cur_pos_tensor = pos``:
  a decode step sees every position up to and including its own).

Readings (also in the design notes): the cache stores the roped k rounded to bf16 (the cache
dtype), everything else stays float64; the tables are the exact float64 values; rows past
``pos`` are never part of the result.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_bits_to_f64, f64_to_bf16_bits
from .expert_attn import EPS, HEAD_DIM, ROPE_THETA, apply_rope, rms_norm, rope_tables

N_Q_HEADS_TEXT = 64
N_KV_HEADS_TEXT = 8


def decode_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, pos: int, scale: float) -> np.ndarray:
    """Attention of one token per query head over cache rows [0, pos].

    q [Hq, D]; K, V [Hkv, N, D] with N > pos; query head h reads kv head h // (Hq / Hkv).
    Returns [Hq, D] float64.
    """
    hq = q.shape[0]
    rep = hq // K.shape[0]
    out = np.empty((hq, V.shape[-1]), dtype=np.float64)
    for h in range(hq):
        g = h // rep
        sc = (K[g, :pos + 1] @ q[h]) * scale
        w = np.exp(sc - sc.max())
        out[h] = (w / w.sum()) @ V[g, :pos + 1]
    return out


def text_decode_attn(q_in, k_in, v_in, gamma_q, gamma_k, Kc, Vc, pos: int, rope_delta: int = 0,
                     eps: float = EPS, theta: float = ROPE_THETA) -> dict:
    """One decode step's attention, from bf16 bit patterns to the float64 output.

    q_in [64, D], k_in and v_in [8, D], gamma_q and gamma_k [D], Kc and Vc [8, Smax, D]: uint16
    bf16 bits. Returns ``out`` [64, D] float64, the float64 ``q_roped`` and ``k_roped``, and the
    updated caches ``Kc_new``/``Vc_new`` (bits; only row ``pos`` differs from the inputs).
    """
    Kc = np.asarray(Kc, dtype=np.uint16)
    Vc = np.asarray(Vc, dtype=np.uint16)
    smax, d = Kc.shape[1], Kc.shape[2]
    if not 0 <= pos < smax:
        raise ValueError("need 0 <= pos < Smax")
    q = bf16_bits_to_f64(q_in)
    k = bf16_bits_to_f64(k_in)
    cos, sin = rope_tables(pos + rope_delta, 1, d, theta)
    q_roped = apply_rope(rms_norm(q, bf16_bits_to_f64(gamma_q), eps), cos, sin)
    k_roped = apply_rope(rms_norm(k, bf16_bits_to_f64(gamma_k), eps), cos, sin)
    Kc_new = Kc.copy()
    Vc_new = Vc.copy()
    Kc_new[:, pos, :] = f64_to_bf16_bits(k_roped)
    Vc_new[:, pos, :] = np.asarray(v_in, dtype=np.uint16)
    out = decode_attention(q_roped, bf16_bits_to_f64(Kc_new), bf16_bits_to_f64(Vc_new), pos, d ** -0.5)
    return {"out": out, "q_roped": q_roped, "k_roped": k_roped, "Kc_new": Kc_new, "Vc_new": Vc_new}
