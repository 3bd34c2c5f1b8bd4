"""Test infrastructure: the CPU reference for attention forward
(16-bit and FP8 inputs), backward and decode.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use
this package. The GPU library never imports, links or calls it, and it
shares no code with the GPU library.
"""
from .attention import attention, attention_rows  # noqa: F401
from .backward import attention_backward  # noqa: F401
from .decode import decode_attention  # noqa: F401
from .fp8 import attention_fp8, e4m3_decode, e4m3_encode  # noqa: F401
