"""CPU fp64 oracle for single-step decode attention over a shrunk KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
imports it and shares no code with it.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
algebraic identities stated on the pages, brute force in 40-digit decimal
arithmetic, and library routines (torch CPU fp64 attention, torch's float8
decoder).  RoPE (``rope``) is the one part whose *flavour* the pages leave
open; its invariants are pinned, its pair layout and base are a reading
(parity unpinned for the flavour and base).  The decode kernels never rotate;
the GPU cache append rotates the new key under the same reading, so its
parity test cannot catch a different flavour or base.
"""
from .attention import *  # noqa: F401,F403
from .cache import *  # noqa: F401,F403
from .projection import *  # noqa: F401,F403
