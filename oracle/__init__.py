"""CPU oracle for ProxyAttn block-sparse prefill attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library or its binding.
"""
from . import proxyattn  # noqa: F401
