"""KDA oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct CPU evaluation of the Kimi Delta Attention
recurrence in float64.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  It shares no code with the HIP path (``gated_delta_rule_95_amd``)
and never imports it; the two meet only through the seeded generators in
``synth``.

What it computes (Kimi K3 architecture walkthrough, mhpq.cn/news/56770,
section "KDA 到底在算什么", state-update equation): per (sequence, head),
with a d_k x d_v state S whose rows are key channels,

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    o_t = S_t^T q_t,        alpha_t = exp(g_t)  (one factor per key channel)

Modules
  recurrence  token-by-token fp64 recurrence (NumPy) and the decode step
  clib        the same recurrence in plain C (OpenMP over chains), for size
  transition  brute-force product of explicit d_k x d_k transition matrices
  chunked     fp64 chunked (WY/UT) form with 16-token tile re-referencing,
              used to check the chunk algebra before it is trusted on the GPU
  spec        speculative-decoding verify / replay, as compositions of the
              recurrence
  prologue    the lower-bounded gate, beta's sigmoid and q/k L2
              normalisation ahead of the recurrence
  backward    reverse-mode gradients of the recurrence (dq, dk, dv, dg,
              dbeta, dS0)

Every function is pinned (``tests/test_oracle_pins.py``, ``tests/test_oracle_spec.py``,
``tests/test_oracle_prologue.py``, ``tests/test_oracle_backward.py``) against facts that
do not come from the oracle itself (closed forms, a hand-derived example,
retrieval identities, brute force, invariants); none is "parity unpinned".
"""
from .recurrence import kda_recurrent, kda_recurrent_varlen, kda_decode_step  # noqa: F401
from .transition import kda_transition_bruteforce  # noqa: F401
from .chunked import kda_chunked  # noqa: F401
from .spec import kda_spec_verify, kda_spec_commit, kda_spec_step  # noqa: F401
from .prologue import kda_gate, kda_prologue, kda_gated_recurrent  # noqa: F401
from .backward import kda_recurrent_vjp, kda_recurrent_vjp_varlen  # noqa: F401
