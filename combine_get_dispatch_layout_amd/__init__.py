"""MI355X-native MoE dispatch layout, token pack, handle reuse and combine.

The compute path is the HIP library ``libmoedx.so`` (hand-written gfx950
kernels behind a C ABI); this package holds its Python binding.  Importing the
package does not load the library; the first use of an API name does, and
raises if the library has not been built.
"""

_API = ("Buffer", "EventOverlap", "capi")


def __getattr__(name):
    if name in ("Buffer", "EventOverlap"):
        from . import buffer
        return getattr(buffer, name)
    if name == "capi":
        from . import _capi
        return _capi
    raise AttributeError(name)
