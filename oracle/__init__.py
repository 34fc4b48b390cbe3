"""CPU oracle for permute_layout.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only code allowed to import this package.  The product
library never loads it, and it imports nothing from the product.

* ``permute``     -- the plain C loop (``oracle_permute.c``) through ctypes;
* ``permute_py``  -- the same definition in pure Python, for small cases;
* ``address``     -- the address rule of one coordinate;
* ``plan_oracle`` -- the host-side steps of the method (shard, P, XOR k).
"""

from .runner import address, build, library_path, permute, permute_py, swizzle  # noqa: F401
from . import plan_oracle  # noqa: F401
