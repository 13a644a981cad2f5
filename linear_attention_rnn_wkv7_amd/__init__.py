"""MI355X-native WKV7 (RWKV-7) recurrence: forward scan and reverse scan.

The compute lives in libwkv7.so (hand-written HIP for gfx950 behind a C ABI,
include/wkv7.h); ``api`` is a thin torch binding of it.  Importing the
package does not load the library; the first call does, and raises if it
has not been built.
"""
__all__ = ["wkv7_forward", "wkv7_backward", "wkv7_checkpoint_bytes",
           "wkv7_backward_workspace_bytes"]


def __getattr__(name):
    if name in __all__:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
