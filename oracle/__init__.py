"""Plain fp64 CPU oracle of the expert-layer attention step (test infrastructure).

This package is test infrastructure only. It may be imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py`` and
by nothing else: the product path (``flow_matching_action_amd``) never imports,
links or runs anything here, and this package imports nothing from it.

Everything is written from the pages' description of the method (page
``code/alpamayo_tt/expert.py`` and page ``code/alpamayo_tt/EXPERT_NOTES.md``),
in NumPy float64, with no blocking, fusion or reordering beyond the plain
definition. Its bf16 and e4m3 codecs are its own.
"""
from .codecs import E4M3_MAX, bf16_bits_to_f64, e4m3_bits_to_f64, f64_to_bf16_bits, f64_to_e4m3_bits
from .expert_attn import (
    HEAD_DIM, N_KV_HEADS, N_Q_HEADS, N_TOK, EPS, ROPE_THETA, MASK_MIN,
    rms_norm, rope_tables, rotate_half, apply_rope, build_mask, place_tail,
    attention, attention_partial, lse_combine, expert_attn_layer,
    quantize_rows_e4m3, dequantize_rows_e4m3, expert_attn_layer_fp8,
)
from .text_decode import N_KV_HEADS_TEXT, N_Q_HEADS_TEXT, decode_attention, text_decode_attn
from .expert_layer import HIDDEN, MLP, QKV, expert_layer, silu

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "e4m3_bits_to_f64", "f64_to_e4m3_bits", "E4M3_MAX",
    "HEAD_DIM", "N_KV_HEADS", "N_Q_HEADS", "N_TOK", "EPS", "ROPE_THETA", "MASK_MIN",
    "rms_norm", "rope_tables", "rotate_half", "apply_rope", "build_mask", "place_tail",
    "attention", "attention_partial", "lse_combine", "expert_attn_layer",
    "quantize_rows_e4m3", "dequantize_rows_e4m3", "expert_attn_layer_fp8",
    "N_Q_HEADS_TEXT", "N_KV_HEADS_TEXT", "decode_attention", "text_decode_attn",
    "HIDDEN", "QKV", "MLP", "expert_layer", "silu",
]
