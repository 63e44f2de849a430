"""MI355X-native fused scaled-dot-product attention forward with vision-transformer bias.

The compute path is the C-ABI library ``libattn.so`` (hand-written HIP for
gfx950); :mod:`scaled_dot_product_16_amd.binding` marshals torch tensors into
its descriptors.  Importing this package loads nothing; the first call of
:func:`fwd` loads the library and raises if it is missing.
"""

__all__ = ["fwd", "check", "TableBias", "RelposBias", "AdditiveBias", "ShiftMask",
           "AdditiveMask", "Window"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
