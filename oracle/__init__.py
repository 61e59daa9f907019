"""CPU oracle for the VerKV hot path: PoissonComp and KVFetch.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(the HIP library and its Python binding) never imports, links or calls it,
and shares no code, tables or constants with it.

Everything here is plain numpy in float64 (Python integers where a sum must be
exact), written step by step from "Verify Before You Fetch: Reliable KV Cache
Compression for LLM Inference" (Jha, Kumar, Chowdhury, Agrawal, Desai):

* ``oracle.philox``   -- Philox4x32-10, the counter-based generator that draws
  the Poisson sample (Salmon et al., "Parallel Random Numbers: As Easy as
  1, 2, 3", SC'11).
* ``oracle.compress`` -- PoissonComp (Algorithm 1, §4.1, eq. 3).
* ``oracle.decode``   -- KVFetch (Algorithm 2, §4.2: Definition 2 / eq. 5,
  Theorem 1 / eq. 6, Lemma 1 / eq. 7, eqs. 9-10, Theorem 2), the binary
  shrinkage of Appendix A.2, the corrected attention output (§3, eq. 1) and
  the Dense baselines of §5 (exact attention over the whole cache).

Parity status of each function is stated in its docstring; every function is
pinned by ``tests/test_oracle_*.py`` against closed forms, brute force or
library routines, except where a docstring says "parity unpinned".
"""

from . import philox, compress, decode  # noqa: F401
