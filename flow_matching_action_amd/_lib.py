"""ctypes binding of libax.so: argument marshalling only.

Every function here has the name of the C entry point it forwards to (without
the ``ax_`` prefix), takes torch tensors where the C function takes device
pointers, passes torch's current HIP stream unless one is given, and raises
``AxError`` on a nonzero return code. All computation happens in the library's
HIP kernels; there is no fallback of any kind: if the library is missing the
import fails.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libax.so")

AX_OK = 0
AX_E_NULL = -1
AX_E_SHAPE = -2
AX_E_ALIGN = -3
AX_E_WORKSPACE = -4
AX_E_UNSUPPORTED = -5
AX_E_ARG = -6
AX_STATUS_WAIT_EXPIRED = 1

N_Q_HEADS, N_KV_HEADS, N_TOK, HEAD_DIM = 16, 8, 64, 128


class AxError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn}: {msg} (code {code})")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m flow_matching_action_amd.build`")
    return ctypes.CDLL(_LIB_PATH)


lib = _load()
_P = ctypes.c_void_p
_I = ctypes.c_int
lib.ax_abi_version.restype = _I
lib.ax_abi_version.argtypes = []
lib.ax_strerror.restype = ctypes.c_char_p
lib.ax_strerror.argtypes = [_I]
lib.ax_debug_set_wait_limit.restype = _I
lib.ax_debug_set_wait_limit.argtypes = [_I]
lib.ax_rope_tables.restype = _I
lib.ax_rope_tables.argtypes = [_I, _I, _I, ctypes.c_double, _P, _P]
lib.ax_qk_norm_rope.restype = _I
lib.ax_qk_norm_rope.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P]
lib.ax_cache_tail_write.restype = _I
lib.ax_cache_tail_write.argtypes = [_P, _P, _P, _P, _I, _P]
lib.ax_qk_norm_rope_tail.restype = _I
lib.ax_qk_norm_rope_tail.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _I, _P]
lib.ax_expert_attn_workspace_bytes.restype = ctypes.c_size_t
lib.ax_expert_attn_workspace_bytes.argtypes = [_I, _I]
lib.ax_expert_attn.restype = _I
lib.ax_expert_attn.argtypes = [_P, _P, _P, _P, _P, _I, _I, _P, _P, ctypes.c_size_t, _P]
lib.ax_expert_layer_attn.restype = _I
lib.ax_expert_layer_attn.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _I, _I, _P, _P,
                                     ctypes.c_size_t, _P]
lib.ax_expert_layer_attn_noalloc.restype = _I
lib.ax_expert_layer_attn_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _I, _I, _P, _P]
lib.ax_expert_layer_attn_split.restype = _I
lib.ax_expert_layer_attn_split.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _I, _I, _P,
                                           ctypes.c_size_t, _P]
lib.ax_expert_attn_combine.restype = _I
lib.ax_expert_attn_combine.argtypes = [_P, ctypes.c_size_t, _I, _I, _P, _P]
lib.ax_expert_attn_fp8_workspace_bytes.restype = ctypes.c_size_t
lib.ax_expert_attn_fp8_workspace_bytes.argtypes = [_I, _I]
lib.ax_cache_tail_write_fp8.restype = _I
lib.ax_cache_tail_write_fp8.argtypes = [_P, _P, _P, _P, _P, _P, _I, _P]
lib.ax_expert_attn_fp8.restype = _I
lib.ax_expert_attn_fp8.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, ctypes.c_size_t, _P]
lib.ax_expert_layer_attn_fp8.restype = _I
lib.ax_expert_layer_attn_fp8.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P, _I, _I, _P,
                                         _P, ctypes.c_size_t, _P]
lib.ax_expert_layer_attn_fp8_split.restype = _I
lib.ax_expert_layer_attn_fp8_split.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P, _I,
                                               _I, _P, ctypes.c_size_t, _P]
lib.ax_expert_attn_fp8_combine.restype = _I
lib.ax_expert_attn_fp8_combine.argtypes = [_P, ctypes.c_size_t, _I, _I, _P, _P]
lib.ax_text_decode_workspace_bytes.restype = ctypes.c_size_t
lib.ax_text_decode_workspace_bytes.argtypes = [_I, _I]
lib.ax_text_decode_attn.restype = _I
lib.ax_text_decode_attn.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _I, _I, _P, _P,
                                    ctypes.c_size_t, _P]
lib.ax_expert_layer_workspace_bytes.restype = ctypes.c_size_t
lib.ax_expert_layer_workspace_bytes.argtypes = [_I, _I]
lib.ax_expert_layer.restype = _I
lib.ax_expert_layer.argtypes = [_P] * 12 + [ctypes.c_float, _P, _P, _I, _I, _P, _P, ctypes.c_size_t, _P]
lib.ax_expert_layer_chained.restype = _I
lib.ax_expert_layer_chained.argtypes = [_P] * 13 + [ctypes.c_float, _P, _P, _I, _I, _P, _P, _P, _P, ctypes.c_size_t,
                                                    _P]
lib.ax_pack_weight_m64.restype = _I
lib.ax_pack_weight_m64.argtypes = [_P, _I, _I, _P, _P]
lib.ax_linear_m64_workspace_bytes.restype = ctypes.c_size_t
lib.ax_linear_m64_workspace_bytes.argtypes = [_I, _I]
lib.ax_linear_m64.restype = _I
lib.ax_linear_m64.argtypes = [_P, _P, _I, _I, _P, _P, ctypes.c_size_t, _P]
lib.ax_copy_words.restype = _I
lib.ax_copy_words.argtypes = [_P, _P, ctypes.c_size_t, _P]

EXPORTS = ("ax_abi_version", "ax_strerror", "ax_debug_set_wait_limit", "ax_rope_tables",
           "ax_expert_layer_attn_noalloc", "ax_qk_norm_rope", "ax_cache_tail_write",
           "ax_qk_norm_rope_tail", "ax_expert_attn_workspace_bytes", "ax_expert_attn",
           "ax_expert_layer_attn", "ax_expert_layer_attn_split", "ax_expert_attn_combine",
           "ax_expert_attn_fp8_workspace_bytes", "ax_cache_tail_write_fp8", "ax_expert_attn_fp8",
           "ax_expert_layer_attn_fp8", "ax_expert_layer_attn_fp8_split", "ax_expert_attn_fp8_combine",
           "ax_text_decode_workspace_bytes", "ax_text_decode_attn", "ax_expert_layer_workspace_bytes",
           "ax_expert_layer", "ax_expert_layer_chained", "ax_pack_weight_m64", "ax_linear_m64_workspace_bytes", "ax_linear_m64",
           "ax_copy_words")


def _check(fn: str, code: int) -> None:
    if code != AX_OK:
        raise AxError(fn, code, lib.ax_strerror(code).decode())


def _ptr(t) -> int | None:
    """Device pointer of a tensor (None -> NULL). Only the address is passed: the library checks the rest."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def abi_version() -> int:
    return lib.ax_abi_version()


def strerror(code: int) -> str:
    return lib.ax_strerror(code).decode()


def debug_set_wait_limit(polls: int) -> None:
    """Polls before a bounded in-workgroup wait gives up, for later launches (0 = the default)."""
    _check("ax_debug_set_wait_limit", lib.ax_debug_set_wait_limit(int(polls)))


def workspace_status(ws) -> int:
    """The status word (first 4 bytes) of an attention workspace tensor; synchronises the device."""
    torch.cuda.synchronize()
    return int(ws[:4].view(torch.int32).item())


def rope_tables(pos0: int, n_tok: int = N_TOK, head_dim: int = HEAD_DIM, theta: float = 5e6):
    """Host RoPE tables (cos, sin), float32 numpy arrays [n_tok, head_dim // 2], from the C library."""
    cos = np.empty((n_tok, head_dim // 2), np.float32)
    sin = np.empty((n_tok, head_dim // 2), np.float32)
    _check("ax_rope_tables", lib.ax_rope_tables(pos0, n_tok, head_dim, theta,
                                                cos.ctypes.data_as(_P), sin.ctypes.data_as(_P)))
    return cos, sin


def qk_norm_rope(q_in, k_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, q_out, k_out, stream=None):
    _check("ax_qk_norm_rope", lib.ax_qk_norm_rope(
        _ptr(q_in), _ptr(k_in), _ptr(gamma_q), _ptr(gamma_k), _ptr(rope_cos), _ptr(rope_sin), float(eps),
        _ptr(q_out), _ptr(k_out), _stream(stream)))


def cache_tail_write(k_roped, v, Kc, Vc, Smax: int, stream=None):
    _check("ax_cache_tail_write", lib.ax_cache_tail_write(
        _ptr(k_roped), _ptr(v), _ptr(Kc), _ptr(Vc), int(Smax), _stream(stream)))


def qk_norm_rope_tail(q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, q_out, Kc, Vc, Smax: int,
                      stream=None):
    _check("ax_qk_norm_rope_tail", lib.ax_qk_norm_rope_tail(
        _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(gamma_q), _ptr(gamma_k), _ptr(rope_cos), _ptr(rope_sin),
        float(eps), _ptr(q_out), _ptr(Kc), _ptr(Vc), int(Smax), _stream(stream)))


def expert_attn_workspace_bytes(S: int, Smax: int) -> int:
    return int(lib.ax_expert_attn_workspace_bytes(int(S), int(Smax)))


def expert_attn(q_roped, k_own, v_own, Kc, Vc, S: int, Smax: int, out, ws, stream=None):
    _check("ax_expert_attn", lib.ax_expert_attn(
        _ptr(q_roped), _ptr(k_own), _ptr(v_own), _ptr(Kc), _ptr(Vc), int(S), int(Smax), _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def expert_layer_attn_noalloc(q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, Kc, Vc, S: int,
                              Smax: int, out, stream=None):
    _check("ax_expert_layer_attn_noalloc", lib.ax_expert_layer_attn_noalloc(
        _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(gamma_q), _ptr(gamma_k), _ptr(rope_cos), _ptr(rope_sin),
        float(eps), _ptr(Kc), _ptr(Vc), int(S), int(Smax), _ptr(out), _stream(stream)))


def expert_layer_attn(q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, Kc, Vc, S: int, Smax: int,
                      out, ws, stream=None):
    _check("ax_expert_layer_attn", lib.ax_expert_layer_attn(
        _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(gamma_q), _ptr(gamma_k), _ptr(rope_cos), _ptr(rope_sin),
        float(eps), _ptr(Kc), _ptr(Vc), int(S), int(Smax), _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def expert_layer_attn_split(q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, Kc, Vc, S: int,
                            Smax: int, ws, stream=None):
    _check("ax_expert_layer_attn_split", lib.ax_expert_layer_attn_split(
        _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(gamma_q), _ptr(gamma_k), _ptr(rope_cos), _ptr(rope_sin),
        float(eps), _ptr(Kc), _ptr(Vc), int(S), int(Smax), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def expert_attn_combine(ws, S: int, Smax: int, out, stream=None):
    _check("ax_expert_attn_combine", lib.ax_expert_attn_combine(
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, int(S), int(Smax), _ptr(out),
        _stream(stream)))


def _nbytes(t) -> int:
    return t.numel() * t.element_size() if t is not None else 0


def expert_attn_fp8_workspace_bytes(S: int, Smax: int) -> int:
    return int(lib.ax_expert_attn_fp8_workspace_bytes(int(S), int(Smax)))


def cache_tail_write_fp8(k_roped, v, Kc8, Ks, Vc8, Vs, Smax: int, stream=None):
    _check("ax_cache_tail_write_fp8", lib.ax_cache_tail_write_fp8(
        _ptr(k_roped), _ptr(v), _ptr(Kc8), _ptr(Ks), _ptr(Vc8), _ptr(Vs), int(Smax), _stream(stream)))


def expert_attn_fp8(q_roped, k_own, v_own, Kc8, Ks, Vc8, Vs, S: int, Smax: int, out, ws, stream=None):
    _check("ax_expert_attn_fp8", lib.ax_expert_attn_fp8(
        _ptr(q_roped), _ptr(k_own), _ptr(v_own), _ptr(Kc8), _ptr(Ks), _ptr(Vc8), _ptr(Vs), int(S), int(Smax),
        _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream)))


def expert_layer_attn_fp8(q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, Kc8, Ks, Vc8, Vs, S: int,
                          Smax: int, out, ws, stream=None):
    _check("ax_expert_layer_attn_fp8", lib.ax_expert_layer_attn_fp8(
        _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(gamma_q), _ptr(gamma_k), _ptr(rope_cos), _ptr(rope_sin),
        float(eps), _ptr(Kc8), _ptr(Ks), _ptr(Vc8), _ptr(Vs), int(S), int(Smax), _ptr(out), _ptr(ws), _nbytes(ws),
        _stream(stream)))


def expert_layer_attn_fp8_split(q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, Kc8, Ks, Vc8, Vs,
                                S: int, Smax: int, ws, stream=None):
    _check("ax_expert_layer_attn_fp8_split", lib.ax_expert_layer_attn_fp8_split(
        _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(gamma_q), _ptr(gamma_k), _ptr(rope_cos), _ptr(rope_sin),
        float(eps), _ptr(Kc8), _ptr(Ks), _ptr(Vc8), _ptr(Vs), int(S), int(Smax), _ptr(ws), _nbytes(ws),
        _stream(stream)))


def expert_attn_fp8_combine(ws, S: int, Smax: int, out, stream=None):
    _check("ax_expert_attn_fp8_combine", lib.ax_expert_attn_fp8_combine(
        _ptr(ws), _nbytes(ws), int(S), int(Smax), _ptr(out), _stream(stream)))


def text_decode_workspace_bytes(pos: int, Smax: int) -> int:
    return int(lib.ax_text_decode_workspace_bytes(int(pos), int(Smax)))


def text_decode_attn(q_in, k_in, v_in, gamma_q, gamma_k, rope_cos, rope_sin, eps, Kc, Vc, pos: int, Smax: int, out,
                     ws, stream=None):
    _check("ax_text_decode_attn", lib.ax_text_decode_attn(
        _ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(gamma_q), _ptr(gamma_k), _ptr(rope_cos), _ptr(rope_sin),
        float(eps), _ptr(Kc), _ptr(Vc), int(pos), int(Smax), _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream)))


def expert_layer_workspace_bytes(S: int, Smax: int) -> int:
    return int(lib.ax_expert_layer_workspace_bytes(int(S), int(Smax)))


def expert_layer(x_in, ln1, wqkv, q_norm_w, k_norm_w, wo, ln2, w1, w3, w2, rope_cos, rope_sin, eps, Kc, Vc, S: int,
                 Smax: int, x_out, ws, stream=None):
    _check("ax_expert_layer", lib.ax_expert_layer(
        _ptr(x_in), _ptr(ln1), _ptr(wqkv), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(wo), _ptr(ln2), _ptr(w1), _ptr(w3),
        _ptr(w2), _ptr(rope_cos), _ptr(rope_sin), float(eps), _ptr(Kc), _ptr(Vc), int(S), int(Smax), _ptr(x_out),
        _ptr(ws), _nbytes(ws), _stream(stream)))


def expert_layer_chained(x_in, n1_in, ln1, wqkv, q_norm_w, k_norm_w, wo, ln2, w1, w3, w2, rope_cos, rope_sin, eps,
                         Kc, Vc, S: int, Smax: int, x_out, ln1_next, n1_out, ws, stream=None):
    _check("ax_expert_layer_chained", lib.ax_expert_layer_chained(
        _ptr(x_in), _ptr(n1_in), _ptr(ln1), _ptr(wqkv), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(wo), _ptr(ln2),
        _ptr(w1), _ptr(w3), _ptr(w2), _ptr(rope_cos), _ptr(rope_sin), float(eps), _ptr(Kc), _ptr(Vc), int(S),
        int(Smax), _ptr(x_out), _ptr(ln1_next), _ptr(n1_out), _ptr(ws), _nbytes(ws), _stream(stream)))


def pack_weight_m64(W, K: int, N: int, W_packed, stream=None):
    _check("ax_pack_weight_m64", lib.ax_pack_weight_m64(_ptr(W), int(K), int(N), _ptr(W_packed), _stream(stream)))


def linear_m64_workspace_bytes(K: int, N: int) -> int:
    return int(lib.ax_linear_m64_workspace_bytes(int(K), int(N)))


def linear_m64(A, W, K: int, N: int, C, ws, stream=None):
    _check("ax_linear_m64", lib.ax_linear_m64(_ptr(A), _ptr(W), int(K), int(N), _ptr(C), _ptr(ws), _nbytes(ws),
                                              _stream(stream)))


def copy_words(src, dst, n_words16: int, stream=None):
    _check("ax_copy_words", lib.ax_copy_words(_ptr(src), _ptr(dst), int(n_words16), _stream(stream)))
