"""Oracle for draft-tree verification: plain, slow, obviously correct CPU code.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call this
package: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it. It shares no code with the HIP library (no kernels, headers, helpers or
constant tables) and imports nothing from it.

What it computes, and where the pages define it:

* ``tree``       -- ancestor sets of a flattened prefix tree (DARTree paper,
                    Preliminaries > Tree Verification and DDTree: each node sees
                    the verified context and its root-to-node path).
* ``attention``  -- tree attention in float64 with an explicit dense
                    ancestor-only mask (same passage; DDTree abstract: one target
                    forward with an ancestor-only attention mask).
* ``argmax``     -- the target's greedy prediction per node, lowest index on
                    ties (DARTree paper, Preliminaries > Speculative Sampling,
                    the T = 0 rule).
* ``sample``     -- the target's sample per node at temperature T > 0 for
                    exact target-sample matching (DARTree paper, Preliminaries >
                    Speculative Sampling, the DFlash rule; Experimental Setup >
                    Evaluation Details at T = 1), drawn by Gumbel-max from
                    Philox4x32-10 uniforms.
* ``walk``       -- the accepted root-to-leaf path and the bonus token (same
                    passage, plus the bonus-token sentence of Speculative
                    Sampling and the definition of tau in Experimental Setup).
* ``commit``     -- the accepted path's keys and values copied into the KV
                    cache rows that follow the verified prefix (Speculative
                    Sampling: every round commits the accepted prefix and a
                    bonus token; Figure 3: accepted tokens and features leave
                    tree verification).
* ``dartree``    -- DARTree's construction: per-depth top-K candidates with
                    log-softmax values, depth-wise fixed-width expansion scored
                    by eq. 5 (Algorithm 1), and deferred top-B pruning with the
                    best-first heap it equals (eq. 6, Lemma 1, Appendix C).
* ``build_tree`` -- the DDTree best-first heap (DARTree paper, Figure 3
                    caption) and the top-mass optimum it reaches (Tree
                    Verification and DDTree, eq. 4 and the mass decomposition
                    after it; Lemma 1 with its proof in Appendix C).

Parity pins: every function here is checked by tests/test_oracle_*.py against
something other than itself (library routines, closed forms, brute force,
hand-worked fixtures under tests/golden/). No function is left unpinned.
"""

from . import tree, attention, argmax, sample, walk, commit, build_tree, dartree  # noqa: F401
