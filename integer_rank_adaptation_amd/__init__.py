"""MI355X-native IntLoRA integer merge and integer linear layer.

The compute lives in ``libintlora.so`` (hand-written HIP kernels for gfx950 behind a
C ABI declared in ``include/intlora.h``); ``binding`` is a thin ctypes layer over it
and ``ops`` allocates outputs with torch and calls it.  The library is loaded on the
first call, so the input generators (``synth``) work on machines without it; any
compute call without the built library raises.
"""
