"""ax_expert_layer_attn_noalloc (the entry point for callers that cannot allocate) against
ax_expert_layer_attn on the same inputs: output and cache update bit for bit, on two calls in a
row, the second with a smaller shape (the static scratch keeps the first call's contents), and
the rejection of shapes whose partials do not fit the scratch.
"""
import numpy as np
import pytest
import torch

from flow_matching_action_amd import synth

from gpu_util import Guarded, Layer, down, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ax():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from flow_matching_action_amd import ax as lib
    return lib


def test_noalloc_equals_workspace_entry_point(ax):
    for S, Smax, seed in ((4700, 8192, 601), (700, 1024, 602)):
        inp = synth.layer_inputs(Smax, S, seed=seed)
        say(f"expert_layer_attn with a workspace, S={S} Smax={Smax}")
        ref = Layer(inp, ax)
        ref_bits = ref.run(ax)
        say(f"expert_layer_attn_noalloc, S={S} Smax={Smax}")
        b = Layer(inp, ax)
        out_g = Guarded(16 * 64 * 128 * 2)
        out = out_g.t.view(torch.int16).view(16, 64, 128)
        ax.expert_layer_attn_noalloc(b.q, b.k, b.v, b.gq, b.gk, b.cos, b.sin, 1e-6, b.Kc, b.Vc, S, Smax, out)
        torch.cuda.synchronize()
        out_g.check("out")
        assert np.array_equal(down(out), ref_bits), (S, Smax)
        assert np.array_equal(down(b.Kc), down(ref.Kc)) and np.array_equal(down(b.Vc), down(ref.Vc)), (S, Smax)


def test_noalloc_rejects_shapes_beyond_its_scratch(ax):
    inp = synth.layer_inputs(256, 128, seed=603)
    b = Layer(inp, ax)
    # S = 18880 fits (59 cache key ranges + the own one), S = 18881 needs one more: rejected on
    # the host, nothing launched
    fits = ax.expert_attn_workspace_bytes(18880, 20480)
    over = ax.expert_attn_workspace_bytes(18881, 20480)
    assert fits <= 16 << 20 < over
    code = ax.lib.ax_expert_layer_attn_noalloc(b.q.data_ptr(), b.k.data_ptr(), b.v.data_ptr(), b.gq.data_ptr(),
                                               b.gk.data_ptr(), b.cos.data_ptr(), b.sin.data_ptr(), 1e-6,
                                               b.Kc.data_ptr(), b.Vc.data_ptr(), 18881, 20480, b.out.data_ptr(),
                                               None)
    assert code == ax.AX_E_WORKSPACE
