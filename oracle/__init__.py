"""CPU oracle for the LSA selection path: test infrastructure only.

Only the tests, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package. The HIP library and its Python binding
never do.
"""
from . import brute, lsa_oracle  # noqa: F401
