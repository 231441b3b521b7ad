"""MI355X (gfx950) fused scaled-dot-product attention forward.

The compute path is the HIP library built from csrc/ (libattn_fwd.so); the
Python layer only marshals arguments.  Importing this package does not load
the library: `attn_fwd` and friends load it on first use and raise if it is
missing -- there is no fallback implementation.
"""


def __getattr__(name):
    if name in ("attn_fwd", "attn_fwd_raw", "load_library", "library_path", "Status",
                "MASK_MODES", "DTYPE_CODES", "abi_version", "status_str"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
