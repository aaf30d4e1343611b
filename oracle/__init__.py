"""CPU oracle for the OSDN forward pass and its Gated DeltaNet-2 generalisation.

This package is TEST INFRASTRUCTURE. Only the test suite, the smoke check and
the CPU-baseline leg of the benchmark may import it. The HIP library never
calls it, and it shares no code, header, table or helper with the HIP path.

Sources (cited by page title and section; the pages are web summaries of the
two papers):

* [OSDN-it]  "Riepilogo Tecnico: OSDN: Miglioramento della Regola Delta con
  Precondizionamento Online Provabile nell'Attenzione Lineare"
  (gist.science/it/paper/2605.13473).
* [OSDN-de]  "OSDN: Improving Delta Rule with Provable Online Preconditioning
  in Linear Attention", its "Technische Zusammenfassung" part
  (gist.science/de/paper/2605.13473). Its sections mirror [OSDN-it].
* [GDN2-it]  "Riepilogo Tecnico: Gated DeltaNet-2"
  (gist.science/it/paper/2605.22791).

Modules:

* ``recurrence``  fp64 NumPy token-by-token recurrences (OSDN, phase 1 alone,
  GDN-2, OSDN on a per-channel-decay backbone), the surrogate h_t, by definition and in closed form, and the
  residual contraction ratios with their geometric mean q_geo.
* ``backward``  the fp64 reverse-mode adjoints of the OSDN token recurrence
  (the gradients of every input, the preconditioner learner's included), of
  OSDN on a per-channel-decay backbone and of GDN-2 (gate-aware: decay,
  erase and write gates), pinned by central differences of ``osdn_ref``,
  ``osdn_gated_ref`` and ``gdn2_ref`` in ``tests/test_oracle_backward.py``.
* ``exact``     the same recurrences in exact rational arithmetic
  (``fractions.Fraction``) plus an independent closed-form unrolling of the
  state as a sum of products of transition matrices, for tiny inputs.

Every function is pinned by a CPU test in ``tests/test_oracle_pins.py``
against something other than itself (closed forms, invariants, special cases,
exact arithmetic). Values the pages print for trained models (recall,
perplexity, q_geo) cannot be reproduced without weights and datasets: those are
"parity unpinned" and are not used.
"""

from .recurrence import (  # noqa: F401
    osdn_ref,
    precond_scan_ref,
    residual_ratio_ref,
    osdn_gated_ref,
    deltanet_ref,
    gdn2_ref,
    h_closed_form,
    h_by_definition,
    grad_h_closed_form,
    regression_loss,
)
from .backward import (  # noqa: F401
    osdn_backward_ref,
    osdn_gated_backward_ref,
    gdn2_backward_ref,
)
