"""MI355X-native paged split-KV GQA/MQA decode attention.

The compute path is the C-ABI library ``libpa_decode.so`` (hand-written HIP for
gfx950, built from ``csrc/``); ``binding`` wraps its three entry points with the
same names for PyTorch device tensors.  ``synth`` draws seeded synthetic inputs.
The binding is imported on first use so that ``synth`` can be used without a GPU.
"""
__all__ = ["binding", "synth"]


def __getattr__(name):
    if name == "binding":
        from . import binding as _b
        return _b
    raise AttributeError(name)
