"""Plain FP64 CPU oracle for the fused Matryoshka contrastive loss.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, helpers, tables or constants); the two meet only
in the seeded input generator, which holds none of the method's arithmetic.
"""

from .contrastive import (  # noqa: F401
    INFONCE,
    INFONCE_ROWS,
    ONESET_EDGES,
    ONESET_SIGLIP,
    SIGLIP,
    KIND_NAMES,
    bf16_bits_to_f64,
    contrastive_fwd_bwd,
    logsumexp,
    prefix_normalise,
    sigmoid,
    softplus,
)
