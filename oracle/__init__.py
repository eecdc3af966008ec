"""CPU oracle (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never uses it; the two
share no code.
"""
from .kvq_oracle import *  # noqa: F401,F403
from .kvq_oracle import (INT8_SYM, INT4_ASYM, INT2_ASYM, INT8_CHANNEL, FP8_E4M3, INT4_INLINE, MODES, BITS,  # noqa: F401
                         LEVELS, META_FLOATS)
