"""MI355X-native SSD / 2Mamba sequence mixer.

The compute path is the HIP library ``libssd.so`` behind the C ABI declared in
``include/ssd.h``; ``mamba_ssd_sequence_amd.ssd`` is its thin Python binding.
Importing this package does not load the library: ``inputs`` (seeded synthetic
inputs) is usable without a GPU.
"""

__all__ = ["inputs", "ssd"]
