"""fp64 CPU oracle for block-top-k sparse paged decode.

TEST INFRASTRUCTURE: imported only by the test suite, the smoke check and the
benchmark's CPU-baseline leg.  The GPU library never imports it.
"""

from .block_topk import *  # noqa: F401,F403
from .block_topk import __all__ as _exact_all
from .radix_topk import *  # noqa: F401,F403
from .radix_topk import __all__ as _radix_all
from .quest import *  # noqa: F401,F403
from .quest import __all__ as _quest_all

__all__ = list(_exact_all) + list(_radix_all) + list(_quest_all)
