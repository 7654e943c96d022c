"""CPU oracle for the KV score-and-evict step — TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 numpy implementations of the two selection rules:
``oracle.rkv`` (R-KV joint importance + redundancy top-B and compaction) and
``oracle.refreekv`` (ReFreeKV sink + reverse-recency threshold cut).

Only tests/, ``__graft_entry__.smoke()`` and the cpu_baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(decode_eviction_amd/csrc) and imports nothing from it; both sides are fed by
the input generators in ``decode_eviction_amd.synth``, which hold none of the
method's arithmetic.

Pins (tests/test_oracle_*.py) tie every function to something other than
itself: brute-force subset search, library routines (scipy softmax, sklearn
cosine similarity), closed forms and invariants.
"""

from . import refreekv, rkv  # noqa: F401
