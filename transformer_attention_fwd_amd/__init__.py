"""MI355X-native forward attention (GroupQueryAttention / MultiHeadAttention /
ai.onnx Attention) on hand-written HIP kernels for gfx950.

Importing the package loads nothing native.  ``transformer_attention_fwd_amd.olk``
loads ``libolk.so`` (the C-ABI library built from ``csrc/``) and raises if it is
missing: there is no CPU fallback.  ``workloads`` holds the seeded input
generators shared by tests and the benchmark.
"""

__all__ = ["olk", "workloads"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
