"""MI355X-native selective state-space scan (Mamba S6): prefill scan and decode step.

The compute path is the C-ABI library ``libssmscan.so`` (hand-written HIP kernels for gfx950);
``ssm_scan_fwd`` and ``ssm_scan_step`` below marshal torch tensors into it. Importing the package
does not load the library; the first call does, and fails loudly when it is missing.
"""
__version__ = "0.1.0"

__all__ = ["ssm_scan_fwd", "ssm_scan_step", "library_path"]


def __getattr__(name):
    if name in __all__:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
