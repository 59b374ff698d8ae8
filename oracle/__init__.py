"""fp64 CPU oracle for tree-structured GDN speculative verification.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library or its Python
binding, and it does not import them.
"""
from .gdn_oracle import *          # noqa: F401,F403
from .gdn_oracle import __all__    # noqa: F401
