"""Float64 CPU oracle for the generalized gated delta rule.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``gated_delta_rule_17_amd``) and imports nothing from it.

Sources (the four web pages the method is taken from; cited by title and
section):

* [QD]   "Q-Delta: Beyond Key-Value Associative State Evolution"
         (papernotes.org summary, ICML 2026).
* [GDN2] "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention"
         (papernotes.org summary, NeurIPS 2026).
* [KDA]  "You could have come up with Kimi Delta Attention" (Chinese
         translation of the Doubleword blog post).
* [CH11] "Chapter 11  Gated DeltaNet: understanding the recurrence from a
         matrix state" (book chapter, book.ozine.me).

Modules
-------
``recurrence``   the plain token-by-token recurrence in the unified form
                 (the oracle proper; every GPU parity test compares with it).
``page_forms``   each variant written in its own page's orientation and step
                 order, plus the product expansion and linear-attention brute
                 force; used only to pin ``recurrence``.
``chunk_mirror`` the chunkwise WY form with absorbed decay, written literally
                 in float64, and its backward in the chunk form's own terms;
                 pinned against ``recurrence`` and ``backward``.
``backward``     reverse mode through the token loop: the gradients of every
                 input for a given output and final-state cotangent; pinned
                 by finite differences of ``recurrence``.
``epilogue``     RMSNorm of each head's readout, then the SiLU output gate;
                 pinned by torch's rms_norm and silu and by closed forms.

Every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` or ``tests/test_oracle_backward.py`` against
something other than itself (a worked
example from [CH11], closed forms, page-form reductions, a stability identity
from [QD], finite-difference gradients).  No function is parity-unpinned.
"""

from .recurrence import gdr_recurrence, gdr_step, VARIANTS, variant_kinds  # noqa: F401
from .backward import gdr_recurrence_vjp  # noqa: F401
from .epilogue import output_norm_gate  # noqa: F401
