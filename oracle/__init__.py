"""Float64 CPU oracle of DSpark's per-round token path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  The product path (the HIP library and its Python binding) never
touches it and shares no code with it.

Modules:
  philox      Philox4x64-10 (Salmon et al., SC'11) and the stream layout.
  dspark_ref  draft (Markov and RNN heads), verify, survival, the confidence
              head and the prefix scheduler in plain float64 numpy.

Every function is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, brute-force enumeration, Monte Carlo laws or
library routines.  None is "parity unpinned".
"""

from . import philox  # noqa: F401
from .dspark_ref import (  # noqa: F401
    EXEMPT_RADIUS,
    acceptance_rate,
    admit_top,
    confidence,
    draft_logits,
    first_argmax,
    inverse_cdf,
    markov_bias,
    markov_draft,
    position_logits,
    residual_law,
    residual_sample,
    rnn_draft,
    round_to_bf16,
    schedule,
    schedule_capacity,
    softmax,
    survival,
    target_logits,
    verify,
    weights_as_f64,
)
