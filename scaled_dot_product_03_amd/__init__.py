"""Flash-attention forward for AMD Instinct MI355X (gfx950).

The compute lives in ``libsdpa03.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/sdpa03.h``).  This package holds the thin ctypes
binding (``scaled_dot_product_03_amd.binding``), the build step
(``scaled_dot_product_03_amd.build``) and the seeded synthetic input
generator (``scaled_dot_product_03_amd.inputs``).

The binding is imported lazily so that the input generator can be used
without loading the shared library.
"""

__all__ = [
    "attn_fwd",
    "attn_fwd_compact_varlen",
    "attn_fwd_padded_varlen",
    "SdpaError",
]


def __getattr__(name):
    if name in __all__:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
