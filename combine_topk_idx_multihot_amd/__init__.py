"""MI355X-native MoE token dispatch / combine into the expanded layout (one GPU's share).

The compute path lives in ``libmoe_mi355x.so`` (hand-written HIP for gfx950 behind a
C ABI declared in ``include/moe_mi355x.h``); ``binding`` marshals torch tensors into
that ABI and loads the library on first use, failing loudly if it is missing.
``inputs`` draws seeded synthetic workloads and carries no dispatch arithmetic.
"""

__all__ = ["binding", "inputs"]


def __getattr__(name):
    if name in ("binding", "inputs"):
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
