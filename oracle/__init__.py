"""fp64 CPU oracle for the Gecko SCA + AWM forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path. It
shares no code with the HIP library or its binding.
"""

from .gecko_oracle import (  # noqa: F401
    HeadStream,
    affine,
    awm_head,
    chunk_ranges,
    feature_softmax,
    forward,
    forward_head,
    sca_chunk,
    sca_head,
)
from .cema_oracle import cema, cema_multiplier  # noqa: F401
from .tdn_oracle import tdn  # noqa: F401
from .gecko_grad_oracle import AFFINE, forward_torch_head, grad, grad_head, lse_head  # noqa: F401
