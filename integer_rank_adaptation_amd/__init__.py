"""MI355X-native IntLoRA integer merge and integer linear layer.

The compute lives in ``libintlora.so`` (hand-written HIP kernels for gfx950 behind a
C ABI declared in ``include/intlora.h``); ``binding`` is a thin ctypes layer over it.
The binding is imported lazily so that the input generators (``synth``) can be used on
machines without the library; any compute call without the library raises.
"""

__all__ = ["binding", "synth"]


def __getattr__(name):
    if name == "binding":
        from . import binding

        return binding
    raise AttributeError(name)
