"""kvsel: MI355X-native KV-cache score-and-evict (R-KV) and threshold cut (ReFreeKV).

The compute path is the HIP library ``libkvsel.so`` built from ``csrc/``; the
Python side (``decode_eviction_amd.kvsel``) only marshals arguments to its
C-ABI.  ``decode_eviction_amd.synth`` draws the seeded synthetic inputs.
Submodules are imported on demand so that importing the generators never
loads the GPU library.
"""
