"""MI355X (gfx950) expert-attention step of the Alpamayo2-Super action expert.

The compute lives in ``libax.so`` (hand-written HIP kernels behind the C ABI of
``include/ax.h``); ``flow_matching_action_amd.ax`` is its ctypes binding and
``flow_matching_action_amd.synth`` the seeded input generators. Importing
``ax`` fails if the library has not been built.
"""
from . import synth  # noqa: F401


def __getattr__(name):
    if name == "ax":
        from . import _lib
        return _lib
    raise AttributeError(name)
