"""MI355X-native paged split-KV GQA/MQA decode attention.

The compute path is the C-ABI library ``lib/libpa_decode.so`` (hand-written HIP for
gfx950, built from ``csrc/`` by ``build.py``); ``binding`` wraps its entry points
with the same names for PyTorch device tensors.  ``synth`` draws seeded synthetic
inputs.  Submodules are imported explicitly (``from mqa_split_kv_amd import
binding``), so ``synth`` can be used on a machine without a GPU.
"""
