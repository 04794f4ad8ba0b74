"""CPU oracle for the chunked gated delta-rule operator (float64).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU path
(``chunked_gated_delta_06_amd``) never imports it and shares no code with it.

Two independent evaluations of the same operator live here:

* ``recurrent`` -- the plain per-token recurrence (PyTorch CPU ops, float64),
  its autograd backward, and a hand-derived reverse recurrence;
* ``chunked``   -- a separate chunk-wise WY evaluation (NumPy, float64) that
  follows the chunk-parallel form quoted on the coverage-matrix page
  ("FLA operator-kernel correctness testing and coverage matrix", section 2,
  the DeltaNet chunk form S^r = P^r S^0 + H^r with P^r in WY form), plus the
  brute-force chunk enumeration for varlen batches.

``metrics`` holds the error ratio the contributor guide's ``assert_close``
uses (RMS of the difference over RMS of the reference).

Readings of the pages that the oracle adopts (the pages leave them open):
  * the state S is K x V and is left-multiplied by the transition, so
    S_t = (I - b_t k_t k_t^T) D_t S_{t-1} + b_t k_t v_t^T and o_t = scale S_t^T q_t
    (the page's ``P^r S^0`` orientation); D_t = diag(exp(g_t)) decays first;
  * the output uses the updated state (inclusive of token t);
  * value head j reads q/k head j // (HV/H);
  * the in-kernel L2 norm is x / sqrt(sum(x^2) + 1e-6).
"""
