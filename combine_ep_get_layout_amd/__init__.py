"""MI355X-native MoE token dispatch / combine on simulated ranks.

The compute path is the HIP library ``libep.so`` (built from ``csrc/``)
behind a C ABI; ``ep`` is its thin ctypes binding.  Importing the package
loads nothing; ``combine_ep_get_layout_amd.ep`` loads the library on first
use and raises if it has not been built.
"""
__all__ = ["ep", "inputs"]
