"""CPU oracle for the ReplaySSM decode path -- TEST INFRASTRUCTURE ONLY.

Plain NumPy in float64. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
HIP library and its Python binding never import it, and it imports nothing from
them: the two sides share no code. Only the seeded input generators
(``hybrid_model_ssm_amd.synth``, which hold none of the method's arithmetic)
feed both.

Sources. The method is described in words on four web pages:

* "ReplaySSM Caches Inputs Instead of State to Speed Up Hybrid-Model Decoding"
  (an NVIDIA Developer post summary), sections "Why SSM layers slow down hybrid
  models" and "How ReplaySSM works";
* "ReplaySSM" (the project README), the list of three benefits (reduced memory
  traffic, cheap rollback, separate state precisions);
* "ReplaySSM (a vLLM research fork)" (an older README), section "Core
  implementation files", which names the entry points.

The pages print no equations. The recurrences written here are the standard
Mamba2 selective state update and the standard gated delta rule, which is what
"conventional decoding" on the first page runs; the replay formulas are derived
from them (see each function's docstring).

Modules:

* ``oracle.mamba2`` -- conventional recurrence, replay form, speculative cursor
  model.
* ``oracle.gdn`` -- gated delta rule, conventional and replay form.
* ``oracle.readcopy`` -- the low-precision read copies of the checkpoint (bf16,
  fp16, and E4M3 fp8 with row scales).

Every function's pins (closed forms, invariants, brute force) live in
``tests/test_oracle_*.py``. Functions with no such pin would be marked "parity
unpinned" here; at present every function has at least one pin.
"""

from . import gdn, mamba2, readcopy  # noqa: F401
