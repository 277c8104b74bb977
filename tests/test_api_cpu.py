"""C-ABI checks that need no GPU: exports, error codes of the host-side validation, host RoPE tables.

Validation happens on the host before any device call, so the rejected calls
below never touch a device (the pointers are fake, 16-byte aligned integers).
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle
from flow_matching_action_amd import ax

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ax.h")
FAKE = 0x10000   # aligned, never dereferenced
MIS = 0x10008    # 8-byte aligned only


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ax_[a-z0-9_]+)\s*\(", src)))


def test_header_and_library_agree():
    names = declared_symbols()
    assert len(names) >= 9
    for n in names:
        assert hasattr(ax.lib, n), f"libax.so does not export {n}"
    assert sorted(ax.EXPORTS) == names


def test_abi_version_and_strerror():
    assert ax.abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert ax.strerror(code)
    assert "unknown" in ax.strerror(-99)


def test_rope_tables_match_oracle():
    for pos0 in (0, 1, 4700, 8128, 65472):
        cos, sin = ax.rope_tables(pos0)
        ref_c, ref_s = oracle.rope_tables(pos0)
        assert np.array_equal(ref_c[:, :64], ref_c[:, 64:])
        ulp = np.spacing(np.abs(ref_c[:, :64]).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(cos - ref_c[:, :64]) <= ulp)
        ulp = np.spacing(np.abs(ref_s[:, :64]).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(sin - ref_s[:, :64]) <= ulp)
    c, s = ax.rope_tables(0)
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)   # row 0 is position 0


def test_rope_tables_rejects_bad_arguments():
    buf = np.empty(64 * 64, np.float32)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    assert ax.lib.ax_rope_tables(0, 64, 128, 5e6, None, p) == ax.AX_E_NULL
    assert ax.lib.ax_rope_tables(0, 64, 127, 5e6, p, p) == ax.AX_E_SHAPE
    assert ax.lib.ax_rope_tables(0, 0, 128, 5e6, p, p) == ax.AX_E_SHAPE
    assert ax.lib.ax_rope_tables(0, 64, 128, 0.0, p, p) == ax.AX_E_ARG
    assert ax.lib.ax_rope_tables(-1, 64, 128, 5e6, p, p) == ax.AX_E_ARG


def test_workspace_bytes():
    assert ax.expert_attn_workspace_bytes(128, 256) > 0
    assert ax.expert_attn_workspace_bytes(4700, 8192) >= ax.expert_attn_workspace_bytes(128, 256)
    assert ax.expert_attn_workspace_bytes(0, 64) > 0
    assert ax.expert_attn_workspace_bytes(193, 256) == 0      # S > Smax - 64
    assert ax.expert_attn_workspace_bytes(-1, 256) == 0
    assert ax.expert_attn_workspace_bytes(0, 63) == 0
    assert ax.expert_attn_workspace_bytes(0, (1 << 20) + 64) == 0


def _layer(q=FAKE, k=FAKE, v=FAKE, gq=FAKE, gk=FAKE, c=FAKE, s=FAKE, eps=1e-6, Kc=FAKE, Vc=FAKE, S=128,
           Smax=256, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return ax.lib.ax_expert_layer_attn(q, k, v, gq, gk, c, s, eps, Kc, Vc, S, Smax, out, ws, ws_bytes, None)


def test_layer_validation_codes():
    assert _layer(q=None) == ax.AX_E_NULL
    assert _layer(out=None) == ax.AX_E_NULL
    assert _layer(Kc=MIS) == ax.AX_E_ALIGN
    assert _layer(S=193) == ax.AX_E_SHAPE
    assert _layer(S=-1) == ax.AX_E_SHAPE
    assert _layer(Smax=32, S=0) == ax.AX_E_SHAPE
    assert _layer(eps=float("nan")) == ax.AX_E_ARG
    assert _layer(eps=-1.0) == ax.AX_E_ARG
    assert _layer(ws_bytes=16) == ax.AX_E_WORKSPACE
    assert _layer(ws=FAKE + 16) == ax.AX_E_WORKSPACE      # not 256-byte aligned


def test_attn_validation_codes():
    f = ax.lib.ax_expert_attn
    assert f(FAKE, FAKE, None, FAKE, FAKE, 128, 256, FAKE, FAKE, 1 << 30, None) == ax.AX_E_NULL
    assert f(FAKE, MIS, MIS, FAKE, FAKE, 128, 256, FAKE, FAKE, 1 << 30, None) == ax.AX_E_ALIGN
    assert f(FAKE, None, None, FAKE, FAKE, 300, 256, FAKE, FAKE, 1 << 30, None) == ax.AX_E_SHAPE
    assert f(FAKE, None, None, FAKE, FAKE, 128, 256, FAKE, FAKE, 100, None) == ax.AX_E_WORKSPACE
    g = ax.lib.ax_qk_norm_rope
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1e-6, FAKE, FAKE, None) == ax.AX_E_NULL
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, float("inf"), FAKE, FAKE, None) == ax.AX_E_ARG
    t = ax.lib.ax_cache_tail_write
    assert t(FAKE, FAKE, FAKE, None, 256, None) == ax.AX_E_NULL
    assert t(FAKE, FAKE, FAKE, FAKE, 63, None) == ax.AX_E_SHAPE
    assert ax.lib.ax_copy_words(None, FAKE, 1, None) == ax.AX_E_NULL


def test_split_and_combine_validation_codes():
    sp = ax.lib.ax_expert_layer_attn_split

    def split(q=FAKE, Kc=FAKE, S=128, Smax=256, eps=1e-6, ws=FAKE, ws_bytes=1 << 30):
        return sp(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, eps, Kc, FAKE, S, Smax, ws, ws_bytes, None)

    assert split(q=None) == ax.AX_E_NULL
    assert split(Kc=MIS) == ax.AX_E_ALIGN
    assert split(S=193) == ax.AX_E_SHAPE
    assert split(eps=float("nan")) == ax.AX_E_ARG
    assert split(ws_bytes=16) == ax.AX_E_WORKSPACE
    assert split(ws=FAKE + 16) == ax.AX_E_WORKSPACE
    cb = ax.lib.ax_expert_attn_combine
    assert cb(None, 1 << 30, 128, 256, FAKE, None) == ax.AX_E_NULL
    assert cb(FAKE, 1 << 30, 128, 256, None, None) == ax.AX_E_NULL
    assert cb(FAKE, 1 << 30, 128, 256, MIS, None) == ax.AX_E_ALIGN
    assert cb(FAKE, 1 << 30, -1, 256, FAKE, None) == ax.AX_E_SHAPE
    assert cb(FAKE, 8, 128, 256, FAKE, None) == ax.AX_E_WORKSPACE


def _gpu_present() -> bool:
    import torch
    return torch.cuda.is_available()


def test_no_device_is_reported_not_launched():
    if _gpu_present():
        pytest.skip("a GPU is present: the valid call would launch")
    assert _layer() == ax.AX_E_UNSUPPORTED


def test_fp8_workspace_bytes():
    assert ax.expert_attn_fp8_workspace_bytes(128, 256) > 0
    assert ax.expert_attn_fp8_workspace_bytes(8128, 8192) > 0
    assert ax.expert_attn_fp8_workspace_bytes(193, 256) == 0
    assert ax.expert_attn_fp8_workspace_bytes(0, 63) == 0


def test_bf16_workspace_holds_one_partial_row_per_range_and_query_row():
    # the 256-byte status word block, then, with 15 cache key ranges of 10 blocks + the own-token
    # range at S = 4700, per (kv head, range, folded query row): 128 float16 of O and a 16-byte
    # record (m and l in float32, 4 exponents in int16)
    per_row = 128 * 2 + 16
    assert ax.expert_attn_workspace_bytes(4700, 8192) == 256 + 16 * 8 * 128 * per_row
    assert ax.expert_attn_workspace_bytes(4700, 5120) == 256 + 16 * 8 * 128 * per_row   # rows read, not Smax
    assert ax.expert_attn_workspace_bytes(0, 64) == 256 + 1 * 8 * 128 * per_row         # the own range alone
    # ranges never exceed 10 blocks: long caches take more ranges
    assert ax.expert_attn_workspace_bytes(65472, 65536) >= 256 + (65472 // 320 + 1) * 8 * 128 * per_row


def test_debug_wait_limit_rejects_negative():
    assert ax.lib.ax_debug_set_wait_limit(-1) == ax.AX_E_ARG
    assert ax.lib.ax_debug_set_wait_limit(0) == ax.AX_OK   # back to the default


def test_fp8_validation_codes():
    lf = ax.lib.ax_expert_layer_attn_fp8

    def layer(q=FAKE, Kc=FAKE, Ks=FAKE, Vs=FAKE, S=128, Smax=256, eps=1e-6, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return lf(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, eps, Kc, Ks, FAKE, Vs, S, Smax, out, ws, ws_bytes, None)

    assert layer(q=None) == ax.AX_E_NULL
    assert layer(Ks=None) == ax.AX_E_NULL
    assert layer(out=None) == ax.AX_E_NULL
    assert layer(Vs=MIS) == ax.AX_E_ALIGN
    assert layer(out=MIS) == ax.AX_E_ALIGN
    assert layer(S=193) == ax.AX_E_SHAPE
    assert layer(eps=float("nan")) == ax.AX_E_ARG
    assert layer(ws_bytes=16) == ax.AX_E_WORKSPACE
    assert layer(ws=FAKE + 16) == ax.AX_E_WORKSPACE
    sp = ax.lib.ax_expert_layer_attn_fp8_split
    assert sp(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, FAKE, None, FAKE, FAKE, 128, 256, FAKE, 1 << 30,
              None) == ax.AX_E_NULL
    assert sp(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, FAKE, FAKE, FAKE, FAKE, 128, 256, FAKE, 16,
              None) == ax.AX_E_WORKSPACE
    at = ax.lib.ax_expert_attn_fp8
    assert at(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 128, 256, FAKE, FAKE, 1 << 30, None) == ax.AX_E_NULL
    assert at(FAKE, MIS, MIS, FAKE, FAKE, FAKE, FAKE, 128, 256, FAKE, FAKE, 1 << 30, None) == ax.AX_E_ALIGN
    assert at(FAKE, None, None, FAKE, FAKE, FAKE, FAKE, 300, 256, FAKE, FAKE, 1 << 30, None) == ax.AX_E_SHAPE
    tw = ax.lib.ax_cache_tail_write_fp8
    assert tw(FAKE, FAKE, FAKE, None, FAKE, FAKE, 256, None) == ax.AX_E_NULL
    assert tw(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 63, None) == ax.AX_E_SHAPE
    cb = ax.lib.ax_expert_attn_fp8_combine
    assert cb(FAKE, 8, 128, 256, FAKE, None) == ax.AX_E_WORKSPACE
    assert cb(FAKE, 1 << 30, 128, 256, None, None) == ax.AX_E_NULL


def test_text_decode_validation_codes():
    assert ax.text_decode_workspace_bytes(0, 1) > 0
    assert ax.text_decode_workspace_bytes(4700, 8192) > 0
    assert ax.text_decode_workspace_bytes(8192, 8192) == 0      # pos must be < Smax
    assert ax.text_decode_workspace_bytes(-1, 64) == 0
    f = ax.lib.ax_text_decode_attn

    def call(q=FAKE, Kc=FAKE, pos=100, Smax=256, eps=1e-6, ws=FAKE, ws_bytes=1 << 30, c=FAKE):
        return f(q, FAKE, FAKE, FAKE, FAKE, c, FAKE, eps, Kc, FAKE, pos, Smax, FAKE, ws, ws_bytes, None)

    assert call(q=None) == ax.AX_E_NULL
    assert call(c=None) == ax.AX_E_NULL
    assert call(Kc=MIS) == ax.AX_E_ALIGN
    assert call(pos=256) == ax.AX_E_SHAPE
    assert call(pos=-1) == ax.AX_E_SHAPE
    assert call(Smax=(1 << 20) + 1, pos=0) == ax.AX_E_SHAPE
    assert call(eps=float("inf")) == ax.AX_E_ARG
    assert call(ws_bytes=8) == ax.AX_E_WORKSPACE
    assert call(ws=FAKE + 16) == ax.AX_E_WORKSPACE


def test_expert_layer_workspace_and_validation_codes():
    assert ax.expert_layer_workspace_bytes(4700, 8192) > ax.expert_attn_workspace_bytes(4700, 8192)
    assert ax.expert_layer_workspace_bytes(193, 256) == 0
    assert ax.linear_m64_workspace_bytes(1536, 4096) == 2 * 64 * 4096 * 4     # 2 splits of 768 rows
    assert ax.linear_m64_workspace_bytes(100, 64) == 0
    assert ax.linear_m64_workspace_bytes(128, 96) == 0
    f = ax.lib.ax_expert_layer
    big = 1 << 30

    def layer(**kw):
        a = dict(x=FAKE, ln1=FAKE, wqkv=FAKE, qn=FAKE, kn=FAKE, wo=FAKE, ln2=FAKE, w1=FAKE, w3=FAKE, w2=FAKE,
                 cos=FAKE, sin=FAKE, eps=1e-6, Kc=FAKE, Vc=FAKE, S=128, Smax=256, out=FAKE, ws=FAKE, ws_bytes=big)
        a.update(kw)
        return f(*a.values(), None)

    assert layer(w2=None) == ax.AX_E_NULL
    assert layer(out=None) == ax.AX_E_NULL
    assert layer(S=193) == ax.AX_E_SHAPE
    assert layer(eps=float("nan")) == ax.AX_E_ARG
    assert layer(ws_bytes=16) == ax.AX_E_WORKSPACE
    assert layer(ws=FAKE + 16) == ax.AX_E_WORKSPACE
    pk = ax.lib.ax_pack_weight_m64
    assert pk(None, 128, 64, FAKE, None) == ax.AX_E_NULL
    assert pk(FAKE, 100, 64, FAKE, None) == ax.AX_E_SHAPE
    g = ax.lib.ax_linear_m64
    assert g(None, FAKE, 128, 64, FAKE, FAKE, big, None) == ax.AX_E_NULL
    assert g(FAKE, FAKE, 100, 64, FAKE, FAKE, big, None) == ax.AX_E_SHAPE
    assert g(FAKE, FAKE, 128, 96, FAKE, FAKE, big, None) == ax.AX_E_SHAPE
    assert g(FAKE, FAKE, 128, 64, FAKE, FAKE, 16, None) == ax.AX_E_WORKSPACE
    # Valid arguments pass validation and would launch on the fake pointers where a device exists:
    # only without one may they be called, to see them reported as unsupported.
    if not _gpu_present():
        assert layer() == ax.AX_E_UNSUPPORTED
        assert pk(FAKE, 128, 64, FAKE, None) == ax.AX_E_UNSUPPORTED
        assert g(FAKE, FAKE, 128, 64, FAKE, FAKE, big, None) == ax.AX_E_UNSUPPORTED


def test_expert_layer_chained_validation_codes():
    f = ax.lib.ax_expert_layer_chained
    X, XO, N1, N2 = 0x100000, 0x200000, 0x300000, 0x400000  # aligned, 1 MiB apart, never dereferenced

    def layer(**kw):
        a = dict(x=X, n1_in=None, ln1=FAKE, wqkv=FAKE, qn=FAKE, kn=FAKE, wo=FAKE, ln2=FAKE, w1=FAKE, w3=FAKE,
                 w2=FAKE, cos=FAKE, sin=FAKE, eps=1e-6, Kc=FAKE, Vc=FAKE, S=128, Smax=256, out=XO, ln1_next=None,
                 n1_out=None, ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return f(*a.values(), None)

    assert layer(wqkv=None) == ax.AX_E_NULL
    assert layer(ln1=None) == ax.AX_E_NULL                   # no n1_in: the first norm needs ln1
    assert layer(ln1_next=FAKE) == ax.AX_E_NULL              # ln1_next without n1_out
    assert layer(n1_out=N2) == ax.AX_E_NULL                  # n1_out without ln1_next
    assert layer(n1_in=MIS) == ax.AX_E_ALIGN
    assert layer(ln1_next=FAKE, n1_out=N2 + 8) == ax.AX_E_ALIGN
    assert layer(out=X + 4096) == ax.AX_E_ARG                # x_out overlaps x_in
    assert layer(ln1_next=FAKE, n1_out=XO + 1024) == ax.AX_E_ARG
    assert layer(ln1_next=FAKE, n1_out=X) == ax.AX_E_ARG
    assert layer(n1_in=N1, ln1_next=FAKE, n1_out=N1 + 16) == ax.AX_E_ARG
    assert layer(S=193) == ax.AX_E_SHAPE
    assert layer(eps=float("nan")) == ax.AX_E_ARG
    assert layer(ws_bytes=16) == ax.AX_E_WORKSPACE
    if not _gpu_present():  # valid arguments would launch on the fake pointers where a device exists
        assert layer() == ax.AX_E_UNSUPPORTED
        assert layer(n1_in=N1, ln1=None, ln1_next=FAKE, n1_out=N2) == ax.AX_E_UNSUPPORTED
