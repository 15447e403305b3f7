"""MI355X (gfx950) decode attention over a shrunk KV cache: absorbed MLA, GLA, MLRA, GQA, MQA, GTA.

The compute lives in ``liblatent_decode.so`` (hand-written HIP kernels behind
the C ABI of ``include/latent_decode.h``); this package is its ctypes binding.
"""
from .binding import *  # noqa: F401,F403
