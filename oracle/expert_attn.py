"""fp64 oracle of one expert layer's attention step (test infrastructure).

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; the product path never touches it.

What is computed, and where the pages define it:

* per-head RMSNorm of q and of the expert's own k, eps 1e-6 - page
  ``code/alpamayo_tt/expert.py``, ``TTExpert.layer`` (the two ``rms_norm``
  calls with the ``qn``/``kn`` gammas); eps and the per-head width in page
  ``code/alpamayo_tt/EXPERT_NOTES.md``, section "Layouts";
* HF rotate_half RoPE with theta 5e6 at positions ``i + rope_delta + S`` - page
  ``code/alpamayo_tt/expert.py``, ``TTExpert.set_context`` and ``TTExpert.layer``
  (``rotary_embedding_hf``); theta and positions in EXPERT_NOTES.md, "Layouts";
* own roped K and raw V written into cache rows ``[Smax-64, Smax)`` in the
  cache dtype - ``TTExpert.layer`` (``typecast`` + ``fill_cache`` at
  ``update_idx = Smax - 64``) and EXPERT_NOTES.md, section "Attention over the
  VLM cache: masking approach";
* additive mask, 0 on ``[0, S)`` and on ``[Smax-64, Smax)``, -1e9 elsewhere -
  ``TTExpert.build_mask`` and the ``MASK_MIN`` constant of expert.py;
* non-causal GQA attention over the whole cache, q head h reading kv head
  ``h // 2``, scale ``head_dim ** -0.5`` - ``TTExpert.attention_core`` and the
  ``scale`` set in ``TTExpert.__init__``; the head folding in the expert.py
  module docstring and in EXPERT_NOTES.md, "masking approach".

Readings taken where the pages leave a step open (each also listed in the
design notes of the repository):

* No intermediate rounding: norm and RoPE stay in float64; the only rounding
  is the store of the roped own k into the bf16 cache (the cache holds the
  cache dtype).
* cos/sin are exact float64 values of the plain definition (the pages upload
  bf16 tables; here no table precision is modelled).
* RoPE is plain 1-D RoPE with the duplicated-half (rotate_half) table layout.
* Hidden rows ``[S, Smax-64)`` may hold any finite value; the explicit
  additive mask is applied over the whole cache exactly as stated.
"""
from __future__ import annotations

import numpy as np

from .codecs import E4M3_MAX, bf16_bits_to_f64, e4m3_bits_to_f64, f64_to_bf16_bits, f64_to_e4m3_bits

# Model constants of the action expert (page code/alpamayo_tt/EXPERT_NOTES.md,
# table "Layouts": q/k/v heads [1,16,64,128] and [1,8,64,128]; cos/sin at theta
# 5e6; the mask value is MASK_MIN of page code/alpamayo_tt/expert.py).
N_Q_HEADS = 16
N_KV_HEADS = 8
N_TOK = 64
HEAD_DIM = 128
EPS = 1e-6
ROPE_THETA = 5e6
MASK_MIN = -1e9


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float = EPS) -> np.ndarray:
    """RMSNorm over the last axis: gamma * x / sqrt(mean(x^2) + eps).

    Page code/alpamayo_tt/expert.py, ``TTExpert.layer``: q and k heads are
    normalised per head (width head_dim) with the ``qn``/``kn`` gammas.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def rope_tables(pos0: int, n_tok: int = N_TOK, head_dim: int = HEAD_DIM,
                theta: float = ROPE_THETA) -> tuple[np.ndarray, np.ndarray]:
    """cos and sin tables [n_tok, head_dim] for positions pos0 + i.

    Page code/alpamayo_tt/expert.py, ``TTExpert.set_context`` builds the tables
    for the positions of the 64 expert tokens; EXPERT_NOTES.md ("Layouts") names
    them HF rotate_half tables at positions i + rope_delta + S with theta 5e6.
    Frequency j (0 <= j < head_dim/2) is theta^(-2j/head_dim); the angle of
    token i is position * frequency; the second half of each row repeats the
    first half (rotate_half layout).
    """
    half = head_dim // 2
    pos = np.arange(n_tok, dtype=np.float64) + float(pos0)
    inv_freq = np.array([theta ** (-(2.0 * j) / head_dim) for j in range(half)], dtype=np.float64)
    ang = np.outer(pos, inv_freq)
    cos = np.concatenate([np.cos(ang), np.cos(ang)], axis=-1)
    sin = np.concatenate([np.sin(ang), np.sin(ang)], axis=-1)
    return cos, sin


def rotate_half(x: np.ndarray) -> np.ndarray:
    """[x1, x2] -> [-x2, x1] over the last axis (HF rotate_half)."""
    half = x.shape[-1] // 2
    return np.concatenate([-x[..., half:], x[..., :half]], axis=-1)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """x * cos + rotate_half(x) * sin, tables broadcast over heads.

    Page code/alpamayo_tt/expert.py, ``TTExpert.layer`` (``rotary_embedding_hf``
    on the normed q and k, prefill mode: token i uses table row i).
    """
    return x * cos + rotate_half(x) * sin


def build_mask(S: int, Smax: int, n_rows: int = 2 * N_TOK, n_tok: int = N_TOK) -> np.ndarray:
    """Additive mask [n_rows, Smax]: 0 on [0, S) and [Smax - n_tok, Smax), else MASK_MIN.

    Page code/alpamayo_tt/expert.py, ``TTExpert.build_mask`` (rows = folded
    query rows, 128 in the decode mode); ``set_context`` requires S <= Smax - 64.
    """
    if S > Smax - n_tok:
        raise ValueError(f"S={S} > Smax-{n_tok}: the last {n_tok} cache rows are expert scratch")
    m = np.full((n_rows, Smax), MASK_MIN, dtype=np.float64)
    m[:, :S] = 0.0
    m[:, Smax - n_tok:] = 0.0
    return m


def place_tail(cache: np.ndarray, rows: np.ndarray, n_tok: int = N_TOK) -> np.ndarray:
    """Copy of cache [Hkv, Smax, D] with rows [Smax - n_tok, Smax) replaced by rows [Hkv, n_tok, D].

    Page code/alpamayo_tt/expert.py, ``TTExpert.layer`` (``fill_cache`` at
    ``update_idx = Smax - 64``, batch index 0). Every other row is unchanged.
    """
    out = np.array(cache, copy=True)
    smax = out.shape[1]
    out[:, smax - n_tok:, :] = rows
    return out


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, mask: np.ndarray | None,
              scale: float) -> np.ndarray:
    """Non-causal GQA softmax attention with an additive mask.

    q [Hq, T, D]; K, V [Hkv, N, D]; mask [T', N] broadcast over heads with
    T' >= T (row t of q head h uses mask row (h % rep) * T + t, which for this
    method's mask is the same for every row). q head h reads kv head h // rep,
    rep = Hq / Hkv (page code/alpamayo_tt/expert.py, ``attention_core``).
    Returns [Hq, T, D] float64.
    """
    hq, t, d = q.shape
    hkv = K.shape[0]
    rep = hq // hkv
    out = np.empty((hq, t, V.shape[-1]), dtype=np.float64)
    for h in range(hq):
        g = h // rep
        sc = (q[h] @ K[g].T) * scale
        if mask is not None:
            r0 = (h % rep) * t
            sc = sc + mask[r0:r0 + t] if mask.shape[0] >= r0 + t else sc + mask[:t]
        sc = sc - sc.max(axis=-1, keepdims=True)
        w = np.exp(sc)
        w = w / w.sum(axis=-1, keepdims=True)
        out[h] = w @ V[g]
    return out


def attention_partial(q: np.ndarray, K: np.ndarray, V: np.ndarray, keys: np.ndarray,
                      scale: float) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Unnormalised attention over a subset of key rows (one split).

    Returns (m, l, o): m [Hq, T] row max of the scaled scores over ``keys``,
    l = sum exp(score - m), o [Hq, T, D] = sum exp(score - m) * V. This is the
    per-split quantity of the flash-decode kernel that the pages use, which
    splits the key sequence across cores and reduces the parts (page
    code/alpamayo_tt/EXPERT_NOTES.md, "masking approach", decode kernel).
    """
    hq, t, _ = q.shape
    rep = hq // K.shape[0]
    m = np.empty((hq, t))
    l = np.empty((hq, t))
    o = np.empty((hq, t, V.shape[-1]))
    for h in range(hq):
        g = h // rep
        sc = (q[h] @ K[g][keys].T) * scale
        m[h] = sc.max(axis=-1)
        e = np.exp(sc - m[h][:, None])
        l[h] = e.sum(axis=-1)
        o[h] = e @ V[g][keys]
    return m, l, o


def lse_combine(parts: list[tuple[np.ndarray, np.ndarray, np.ndarray]]) -> np.ndarray:
    """Combine split partials: out = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c, M = max_c m_c."""
    M = np.max(np.stack([p[0] for p in parts]), axis=0)
    num = sum(np.exp(m - M)[..., None] * o for m, _, o in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    return num / den[..., None]


def expert_attn_layer(q_in, k_in, v_in, gamma_q, gamma_k, Kc, Vc, S: int, Smax: int,
                      rope_delta: int = 0, eps: float = EPS, theta: float = ROPE_THETA) -> dict:
    """One layer's attention step, from bf16 bit patterns to the float64 output.

    Inputs are uint16 bf16 bit arrays: q_in [Hq, 64, D], k_in/v_in [Hkv, 64, D],
    gamma_q/gamma_k [D], Kc/Vc [Hkv, Smax, D]. The steps follow
    ``TTExpert.layer`` up to the attention output (page
    code/alpamayo_tt/expert.py): q/k RMSNorm, RoPE at positions S + rope_delta
    + i, own k/v cast to the cache dtype and written to rows [Smax-64, Smax),
    attention over the whole cache under the 0/-1e9 mask.

    Returns a dict with ``out`` [Hq, 64, D] float64, the float64 ``q_roped`` and
    ``k_roped``, the cache tail bits ``k_tail_bits``/``v_tail_bits`` [Hkv, 64, D]
    and the updated caches ``Kc_new``/``Vc_new`` (bits).
    """
    q_in = np.asarray(q_in, dtype=np.uint16)
    n_tok = q_in.shape[1]
    d = q_in.shape[-1]
    if Kc.shape[1] != Smax or Vc.shape[1] != Smax:
        raise ValueError("cache length does not match Smax")
    if S < 0 or S > Smax - n_tok:
        raise ValueError(f"need 0 <= S <= Smax - {n_tok}")
    q = bf16_bits_to_f64(q_in)
    k = bf16_bits_to_f64(k_in)
    gq = bf16_bits_to_f64(gamma_q)
    gk = bf16_bits_to_f64(gamma_k)
    cos, sin = rope_tables(S + rope_delta, n_tok, d, theta)
    q_roped = apply_rope(rms_norm(q, gq, eps), cos, sin)
    k_roped = apply_rope(rms_norm(k, gk, eps), cos, sin)
    k_tail_bits = f64_to_bf16_bits(k_roped)
    v_tail_bits = np.asarray(v_in, dtype=np.uint16).copy()
    Kc_new = place_tail(np.asarray(Kc, dtype=np.uint16), k_tail_bits, n_tok)
    Vc_new = place_tail(np.asarray(Vc, dtype=np.uint16), v_tail_bits, n_tok)
    rep = q.shape[0] // Kc.shape[0]
    mask = build_mask(S, Smax, rep * n_tok, n_tok)
    out = attention(q_roped, bf16_bits_to_f64(Kc_new), bf16_bits_to_f64(Vc_new), mask, d ** -0.5)
    return {"out": out, "q_roped": q_roped, "k_roped": k_roped, "k_tail_bits": k_tail_bits,
            "v_tail_bits": v_tail_bits, "Kc_new": Kc_new, "Vc_new": Vc_new}


# ---- fp8 cache variant ---------------------------------------------------------------------------
# The pages offer an 8-bit cache (bfp8, a block floating-point format: page code/alpamayo_tt/expert.py,
# TTExpert.__init__, the kv_cache dtype map; page code/alpamayo_tt/EXPERT_NOTES.md, the decode row for
# the bfp8 cache in the attention timing table). Here the cache rows are e4m3 codes with one float32
# scale per (kv head, row): value = e4m3(code) * scale. The own rows that the layer writes into the
# tail are quantised with the per-row rule below (the reading taken for the tail write of such a
# cache: the cache stores the cache dtype, page code/alpamayo_tt/expert.py, TTExpert.layer, the
# typecast before fill_cache).

def quantize_rows_e4m3(x_f32) -> tuple[np.ndarray, np.ndarray]:
    """Per-row e4m3 quantisation: (codes [..., D] uint8, scales [...] float32).

    scale = max_j |x_j| / 448 (float32 division, nearest-even), or 1.0 for an
    all-zero row; code_j = e4m3 rounding (nearest, ties to even, saturating) of
    the float32 quotient x_j / scale. Both divisions are done in float32, the
    precision in which the kernel takes the same decisions, so the codes are
    defined bit for bit.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    return f64_to_e4m3_bits(y.astype(np.float64)), scale


def dequantize_rows_e4m3(codes, scales) -> np.ndarray:
    """value = e4m3(code) * scale in float64 (exact: a 4-bit by 24-bit significand product)."""
    return e4m3_bits_to_f64(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def expert_attn_layer_fp8(q_in, k_in, v_in, gamma_q, gamma_k, Kc8, Ks, Vc8, Vs, S: int, Smax: int,
                          rope_delta: int = 0, eps: float = EPS, theta: float = ROPE_THETA) -> dict:
    """One layer's attention step over an e4m3 cache with per-row float32 scales.

    As ``expert_attn_layer`` (page code/alpamayo_tt/expert.py, ``TTExpert.layer``), except for the
    cache format: Kc8/Vc8 [Hkv, Smax, D] uint8 e4m3 codes, Ks/Vs [Hkv, Smax] float32 scales. The own
    roped k (rounded to bf16, the activation format) and the own bf16 v are quantised row by row
    with ``quantize_rows_e4m3`` into rows [Smax-64, Smax); attention then reads the dequantised
    cache under the same 0/-1e9 mask.

    Returns ``out`` [Hq, 64, D] float64, ``q_roped``, ``k_roped``, the tail codes and scales
    (``k_tail_codes``, ``k_tail_scales``, ``v_tail_codes``, ``v_tail_scales``) and the updated
    caches ``Kc8_new``, ``Ks_new``, ``Vc8_new``, ``Vs_new``.
    """
    q_in = np.asarray(q_in, dtype=np.uint16)
    n_tok = q_in.shape[1]
    d = q_in.shape[-1]
    if Kc8.shape[1] != Smax or Vc8.shape[1] != Smax or Ks.shape[1] != Smax or Vs.shape[1] != Smax:
        raise ValueError("cache length does not match Smax")
    if S < 0 or S > Smax - n_tok:
        raise ValueError(f"need 0 <= S <= Smax - {n_tok}")
    q = bf16_bits_to_f64(q_in)
    k = bf16_bits_to_f64(k_in)
    gq = bf16_bits_to_f64(gamma_q)
    gk = bf16_bits_to_f64(gamma_k)
    cos, sin = rope_tables(S + rope_delta, n_tok, d, theta)
    q_roped = apply_rope(rms_norm(q, gq, eps), cos, sin)
    k_roped = apply_rope(rms_norm(k, gk, eps), cos, sin)
    k_bf16 = bf16_bits_to_f64(f64_to_bf16_bits(k_roped)).astype(np.float32)
    v_bf16 = bf16_bits_to_f64(v_in).astype(np.float32)
    k_codes, k_scales = quantize_rows_e4m3(k_bf16)
    v_codes, v_scales = quantize_rows_e4m3(v_bf16)
    Kc8_new = place_tail(np.asarray(Kc8, dtype=np.uint8), k_codes, n_tok)
    Vc8_new = place_tail(np.asarray(Vc8, dtype=np.uint8), v_codes, n_tok)
    Ks_new = np.array(Ks, dtype=np.float32, copy=True)
    Vs_new = np.array(Vs, dtype=np.float32, copy=True)
    Ks_new[:, Smax - n_tok:] = k_scales
    Vs_new[:, Smax - n_tok:] = v_scales
    rep = q.shape[0] // Kc8.shape[0]
    mask = build_mask(S, Smax, rep * n_tok, n_tok)
    K = dequantize_rows_e4m3(Kc8_new, Ks_new)
    V = dequantize_rows_e4m3(Vc8_new, Vs_new)
    out = attention(q_roped, K, V, mask, d ** -0.5)
    return {"out": out, "q_roped": q_roped, "k_roped": k_roped,
            "k_tail_codes": k_codes, "k_tail_scales": k_scales,
            "v_tail_codes": v_codes, "v_tail_scales": v_scales,
            "Kc8_new": Kc8_new, "Ks_new": Ks_new, "Vc8_new": Vc8_new, "Vs_new": Vs_new}
