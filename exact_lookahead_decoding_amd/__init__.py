"""MI355X-native exact Lookahead decoding: the packed lookahead + verification step.

The hot path lives in HIP kernels behind the C ABI of include/la.h
(csrc/, built into _lib/liblookahead.so by `build`); `la` is the thin
Python binding used by the tests and the benchmark.
"""
__all__ = ["build", "la"]
