"""MI355X (gfx950) forward pass of a top-k routed MoE SwiGLU FFN layer.

The work happens in hand-written HIP kernels behind a C ABI (``include/moe.h``,
``libmoe_mi355x.so``).  ``mixture_experts_layer_sum_amd.moe`` is the thin
Python binding over it; ``synth`` draws seeded synthetic inputs.
"""
__all__ = ["moe", "synth"]


def __getattr__(name):
    if name in ("moe", "synth"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
