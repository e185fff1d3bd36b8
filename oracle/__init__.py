"""Plain CPU oracle of the DSpark draft -> schedule -> verify round.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never calls it, shares no code with it and never falls back to it.
"""

from .dspark_oracle import (  # noqa: F401
    FLAG_EPS,
    widen_weights,
    markov_bias,
    draft_distribution,
    inverse_cdf,
    draft,
    schedule,
    schedule_async,
    schedule_threshold,
    accept_rates,
    verify,
    run_round,
    row_flags,
    sts_calibrate,
    ece,
    sts_fit,
    to_storage,
    rnn_state_update,
    draft_rnn,
)
