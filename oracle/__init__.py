"""CPU float64 oracle for exact disentangled (C2P/P2C) self-attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run anything in this package.
The product path (the HIP library and its Python binding) never imports it and
shares no code with it.
"""
from .df_oracle import (  # noqa: F401
    att_and_rows, bucket_exact, delta, p2c_rows, P2C_CONVENTIONS, rel_luts, sequences, scores,
    forward, backward, forward_rows, dq_rows,
)
from . import philox  # noqa: F401
from .proj import qkv_projection, qkv_projection_backward  # noqa: F401
from .pack import pack_padded, unpack_packed  # noqa: F401
