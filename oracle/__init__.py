"""Reference decoder on the CPU: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never import it.
"""

from .decoder import (  # noqa: F401
    Oracle,
    forward_full,
    greedy_token,
    round_f32_to_bf16,
    to_storage,
    weight_f64,
)
