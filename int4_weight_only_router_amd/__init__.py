"""int4_weight_only_router_amd -- MI355X (gfx950) W4A16 MoE layer hot path.

A thin ctypes binding over libmoe_w4a16.so.  Every function has the name of
the C entry point it forwards to (see include/moe_w4a16.h) and does argument
marshalling only: torch CUDA tensors become device pointers, the stream
defaults to torch's current stream.  All arithmetic runs in the HIP kernels;
there is no CPU fallback, and importing fails loudly when the library is
missing and cannot be built.
"""
from ._abi import *  # noqa: F401,F403
from ._abi import __all__  # noqa: F401
