"""MI355X-native hot path of DistFlashAttn: blockwise exact causal attention
over token chunks (partial O + LSE per chunk pair, LSE merge, backward from
the saved O and LSE) on the token-level load-balanced schedule.

The compute lives in hand-written gfx950 HIP kernels behind the C ABI
declared in ``include/dfa.h`` (``libdfa.so``); ``long_context_exact_amd.dfa``
is the thin ctypes binding with the same entry-point names.  Importing this
package loads nothing; the library is opened on first use and a missing or
unloadable library raises instead of falling back to anything else.
"""

__version__ = "0.1.0"
