"""Exact split-KV softmax attention decoding for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libattn_decode.so`` built from the HIP
sources under ``csrc/``; ``binding`` only marshals torch tensors into it.
``inputs`` holds the seeded synthetic workloads.  The binding is imported on
first use so that the input generator can be used without the library.
"""
_BINDING_NAMES = ("AttnError", "decode", "decode_bifurcated", "decode_energy", "library_path",
                  "load_library", "plan", "workspace_bytes")

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
