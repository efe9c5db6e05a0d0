"""MI355X-native GR-KAN (Group-Rational KAN) safe Pade activation.

The compute path is the HIP library ``libgrkan.so`` (hand-written gfx950
kernels behind a C ABI declared in ``include/grkan.h``); the names below are
its thin Python binding.  Importing this package loads nothing: the library
is loaded on first use and a missing or unloadable library raises.
"""
__all__ = [
    "grkan_forward",
    "grkan_backward",
    "grkan_backward_workspace_size",
    "grkan_status_string",
    "GRKANFunction",
    "GRKANError",
    "grkan_query_launch",
    "grkan_pau_forward",
    "grkan_pau_backward",
    "grkan_pau_backward_workspace_size",
    "grkan_pau_query_launch",
    "grkan_pau_supported",
    "load_library",
]


def __getattr__(name):
    if name in __all__:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
