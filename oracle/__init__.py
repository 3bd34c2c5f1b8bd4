"""Test infrastructure: the CPU reference for attention forward,
backward and decode.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use
this package. The GPU library never imports, links or calls it, and it
shares no code with the GPU library.
"""
from .attention import attention, attention_rows  # noqa: F401
from .backward import attention_backward  # noqa: F401
from .decode import decode_attention  # noqa: F401
