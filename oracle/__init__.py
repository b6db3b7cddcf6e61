"""Plain fp64 CPU oracle for masked attention (forward, backward, block tables).

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library, its C ABI or
the Python binding in ``masked_attention_backward_amd``) imports, links or calls
this package.  It may be used only by ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``.

It shares no code with the GPU path: the only thing both sides use is the seeded
input generator, which holds none of the method's arithmetic.

Every function with a pin is checked by ``tests/test_oracle_*.py`` against
something other than itself (central finite differences, torch fp64 autograd
through ``scaled_dot_product_attention`` / ``softmax``, closed forms, invariants,
brute force on tiny masks and hand-worked fixtures under ``tests/golden/``).
No oracle function is "parity unpinned".
"""

from .attention import (  # noqa: F401
    window_visibility,
    block_visibility,
    sink_attention_forward,
    sink_attention_backward,
    sink_attention_backward_sampled,
    packed_window_visibility,
    sink_attention_forward_varlen,
    sink_attention_backward_varlen,
    blocksparse_attention_forward,
    blocksparse_attention_backward,
    blocksparse_attention_backward_sampled,
    softmax_probabilities,
)
from .tables import build_block_tables, block_mask_popcount  # noqa: F401
