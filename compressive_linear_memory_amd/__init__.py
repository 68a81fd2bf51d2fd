"""Infini-attention segment kernel for MI355X (gfx950): HIP kernels behind a C ABI.

`attn_fwd` / `attn_bwd` are thin ctypes wrappers over libinfini; importing the
package does not load the library (so the input generators can be used on
machines without a GPU).
"""


def __getattr__(name):
    if name in ("attn_fwd", "attn_bwd", "lib", "Problem", "InfiniError", "workspace_bytes"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
