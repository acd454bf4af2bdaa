"""CPU oracle for the low-rank block predictor (test infrastructure only).

This package is a plain, slow, obviously-correct NumPy/Python re-statement of what
the block predictor computes, written from the ``predictor.rs`` page (module doc,
``project_q``, ``project_kv_block``, ``score_blocks``) and, for tie handling, the
``qsa_select.rs`` page (host per-row top-k).  It works in float64 and rounds once
to bfloat16 where the method stores bfloat16.

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product library never calls into it, and it
shares no code, tables or helpers with the HIP path: it has its own bf16 codec,
its own projection generator and its own layouts.

Parity status per function (what pins it is listed in each module docstring):

* ``bf16.encode`` / ``bf16.decode``                 pinned (exact rationals, exhaustive)
* ``prng.splitmix64`` / ``prng.projection``         pinned (published SplitMix64 vector,
                                                    distribution tests); the pages'
                                                    own generator is not shown, so
                                                    equality with *their* P is
                                                    parity unpinned
* ``predictor.project``                             pinned (exact rationals, P = I,
                                                    hand-worked examples)
* ``predictor.score_blocks``                        pinned (hand values, brute force
                                                    q^T P P^T k, P = I logits, invariants)
* ``predictor.rank_victims``                        pinned (sorted() on tiny inputs,
                                                    permutation validity, planted blocks)
* ``predictor.select_victims``                      pinned (sorted() truncated to k)
* ``predictor.score_rows``                          pinned (pure-Python brute force per cell,
                                                    max over rows equals score_blocks,
                                                    causal mask by hand)
* ``predictor.keep_sets``                           pinned (sorted() with the page's
                                                    comparator, hand-worked example)
"""

from . import bf16, prng, predictor  # noqa: F401
