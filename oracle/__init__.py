"""CPU oracle of the rotated W4A4 hot path -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and this
package imports nothing from the product path.

Pinned by ``tests/test_oracle_*.py`` against closed forms, invariants,
hand-worked examples (``tests/golden/``) and brute force.
"""
from .reference import *  # noqa: F401,F403
from .reference import __all__  # noqa: F401
