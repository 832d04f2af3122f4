"""BeaconKV eviction step for MI355X (gfx950).

The compute path is the C-ABI library ``libbkv.so`` built from the HIP
sources in ``csrc/`` (declared in ``include/bkv.h``); ``lib`` is its thin
Python binding.  ``configs`` holds the workload shapes and ``synth`` the seeded
input generator.  Importing the package does not load the library; the first
call through ``lib`` does, and fails loudly if it has not been built.
"""
from .configs import EVICT_CONFIGS, EvictConfig, STREAM, StreamConfig  # noqa: F401
