"""Float64 CPU oracle of the per-layer KronQ solver.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library never
calls it, and nothing here calls the GPU library: the two share no code, no
tables and no constants. Both take their inputs from ``synth`` (random draws
only).

Every function cites the passage of the KronQ pages (or of the Hessian-guided
PTQ page used for identities) that it follows:

* "KronQ: LLM Quantization via Kronecker-Factored Hessian" — paper review page
  (romaanj.github.io), sections Background, Problem, Prior limitations, Goal,
  Method, Key idea, Limitations, "Where this paper sits".
* KronQ abstract and the authors' reply on the Hugging Face paper page.
* "A Unified Hessian-Guided Framework for Post-Training Quantization" (hub.valency.io),
  sections Background (quantization scales, transformations), Modeling the Hessian
  matrices (Table 1), and the appendix on the quantization loss decomposition.
* The H_Z-PTQ page's "Weight scales and rounding" section and experimental settings
  (the Hessian-aware scale search and the trace-sorted block order).

Parity unpinned: the choice of principal square root for non-diagonal H_G (a
reading; any factor S with S^T S = H_G gives the same loss reduction), the
bit-allocation rule (a reading of "upgrade ordering"), and GPTAQ's own column-wise
drift update (not on the pages; ``kronq.drift_target`` is a least-squares reading of
the drift correction, pinned to that reading's algebra, not to GPTAQ).
"""
from . import hadamard, kronq, alloc  # noqa: F401
