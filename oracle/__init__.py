"""Plain fp64 CPU oracle for one packed chunked-prefill + decode attention step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code, header, table or helper with the HIP
library under ``chunked_prefill_mixed_amd/``; the two meet only through the
seeded synthetic inputs.

Every function is pinned by ``tests/test_oracle_pins.py`` against things the
oracle itself does not compute (brute force, closed forms, a library routine,
the worked numbers the pages print).  No function here is "parity unpinned".
"""

from .step import (  # noqa: F401
    BLOCK_SIZE,
    POLICIES,
    adaptive_chunk,
    BudgetError,
    Request,
    advance,
    append,
    attention,
    bf16_bits_to_f64,
    schedule,
    softmax_weights,
)
