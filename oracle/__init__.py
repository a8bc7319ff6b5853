"""CPU oracle for PISA block-sparse attention: TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of the
bench may import this package. The product path (the HIP library and its
Python binding) never imports, calls or links anything here.
"""

from .pisa_oracle import *  # noqa: F401,F403
from .pisa_oracle import __all__  # noqa: F401
