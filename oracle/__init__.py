"""CPU oracle for the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously
correct definition that the GPU library is checked against.  Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it;
the library and its Python binding never do, and it shares no code with
them.

Sources (web pages; cited by title and section):
  [SD]  "Speculative decoding on RDNA" (hipfire 0.4.1 explainer)
  [TREE] "One RDNA4 verify pass has slack for about two dozen speculative tokens"
  [PR]  "feat(dflash): developer-only online draft tuning" (hipfire PR #820)

Stages and the passage each follows:
  gemv.gemv_rows        [SD] §02 (multi-row verify projections), §01
  penalty.*             [SD] §04 figure "the penalty history of verify row i"
  topk.topk_row(s)      [SD] §03 "how hipfire does it" (64-wide pool, tie order);
                        [PR] "Code map" (batched top-K; ties, NaN, -inf)
  policy.policy_row     [SD] §03 "how hipfire does it" (temperature, top-k,
                        min-p, top-p; same pool, tie order and summation)
  policy.draw           [SD] §03 (one request-seeded random stream)
  accept.*              [SD] §01 figure and text, §02, §03 steps 1-4, §06;
                        [TREE] "Spend the budget on a tree"
  tree_attention.*      [TREE] "Spend the budget on a tree" (tree attention
                        mask), "Where the tree earns its keep" (KV scratch
                        slots, only the accepted branch kept)

Every function's pin (what checks it against something other than itself)
is in tests/test_oracle_*.py.  Parity unpinned: none of the functions here;
the sampler policy's stage semantics are pinned only by constructed closed
forms, since the pages print no numbers for it.
"""

from . import accept, gemv, penalty, pipeline, policy, topk, tree_attention  # noqa: F401
