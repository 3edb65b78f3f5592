"""MI355X-native Mamba-2 mixer layer: decode step and chunked prefill.

The compute path is the HIP library ``libm2.so`` (sources in ``csrc/``, C ABI in
``include/m2.h``). ``m2`` is its thin ctypes binding; ``synth`` draws the seeded
synthetic workloads. Importing this package loads nothing; ``from
full_duplex_speech_mamba2_amd import m2`` loads the library and fails loudly if
it is missing.
"""
__all__ = ["m2", "synth"]
