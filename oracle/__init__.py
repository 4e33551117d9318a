"""Float64 CPU oracle for differential attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library.
"""

from .diffattn_oracle import (  # noqa: F401
    attention,
    diff_attention,
    diff_attention_backward,
    diff_attention_backward_dq_rows,
    diff_attention_decode,
    diff_attention_decode_ragged,
    diff_attention_rows,
    diff_attention_v2,
    diff_attention_v2_decode,
    head_rmsnorm,
    lambda_init_schedule,
    reparam_lambda,
    reparam_lambda_backward,
    score_maps,
    signed_map,
)
