"""MI355X-native Kimi Delta Attention (KDA) forward: chunkwise prefill, packed
varlen prefill and the fused decode step, as hand-written HIP kernels for
gfx950 behind the C ABI in include/kda.h.

``from gated_delta_rule_06_amd import kda`` loads the library (and raises if it
is not built); ``gated_delta_rule_06_amd.inputs`` holds the seeded synthetic
input generator and needs no library.
"""
import importlib

__all__ = ["kda", "inputs", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
