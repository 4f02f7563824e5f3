"""Float64 CPU oracle for the MLP training step.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path.
All functions are pinned by ``tests/test_oracle.py``.
"""
from .mlp_oracle import (backward, forward, gamma, layer_error_factors,  # noqa: F401
                         mask_band, sgd, softmax_xent, train_step)
