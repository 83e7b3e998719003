"""Plain, slow, float64 CPU oracle of GPTQ layer-wise weight quantization.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the product path never
does, and it shares no code with the HIP library.
"""
from .gptq import *  # noqa: F401,F403
from .gptq import __all__ as _gptq_all
from .w4a16 import *  # noqa: F401,F403
from .w4a16 import __all__ as _w4a16_all
from .awq import *  # noqa: F401,F403
from .awq import __all__ as _awq_all
from .chain import *  # noqa: F401,F403
from .chain import __all__ as _chain_all

__all__ = list(_gptq_all) + list(_w4a16_all) + list(_awq_all) + list(_chain_all)
