"""Reference oracle for batched speculative verification -- TEST INFRASTRUCTURE.

A plain, slow, CPU-only statement of what the verification path computes,
written from the source pages:

* ``verify``  -- the target-model forward pass over the stacked draft chunks
  (fp64 arithmetic on the exact decodes of the stored bf16 / int4 / fp32 inputs);
* ``accept``  -- rejection-sampling acceptance, residual / bonus resampling and
  the KV-length commit (the fp32 / integer / fp64 decisions the library makes);
* ``plan``    -- the compute-slack budget, expected-tokens formulas, the step
  roofline model, the crossover batch and draft-length planning (fp64).

Only the tests, the smoke entry point and the benchmark's CPU-baseline leg may
import this package.  The library never calls it; it shares no code, headers,
tables or helpers with the HIP implementation.

Every function names the page passage it follows.  Page short names used below:

* [slack]  "Speculative Decoding and Batching Compete for the Same Compute
  Slack on RDNA4" (zolotukhin.ai, 2026-07-26)
* [tax]    "Speculative Decoding at High Batch Size: Where the 3x Speedup
  Turns Into a Tax" (techfordev.netlify.app)
* [static] "Why Static Batching Wastes an RX 9070 XT Agent Swarm and
  Continuous Batching Wins It Back" (zolotukhin.ai, 2026-07-30)
* [primer] the speculative-decoding primer at splicedso.github.io/learn

Parity status: the verify pass is pinned by self-consistency and textbook
special cases (no page prints logits); acceptance is pinned by exhaustive
enumeration of the lossless property and by the primer's worked example;
the planner is pinned by the values the pages print.
"""
