"""CPU oracle for heavy-hitter KV-cache eviction fused into decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import or run anything in this package.  The GPU library
never imports it, links it or falls back to it, and this package imports
nothing from the GPU library: the two share no code.  Both sides take their
inputs from the seeded generators in ``workloads``, which hold none of the
method's arithmetic.

Everything here is plain numpy in float64 on the exact storage-dtype input
values (upcast), written step by step in the order the pages state the
method:

* ``attention`` - softmax attention (textbook definition).
* ``h2o``       - H2O heavy-hitter scoring, prefill selection and the greedy
                  per-step eviction with a recent window; also the
                  Scissorhands fixed-budget reading (same loop).
* ``fastgen``   - FastGen's per-head policies: full cache, local window,
                  special+punctuation tokens, frequency (H2O) + local.
* ``hashevict`` - HashEvict's sign sketches, Hamming ranking, prompt replay
                  and pre-attention replacement.
* ``persistence`` - the persistence-of-importance reading of [SH]: pivotal
                  bits (weight >= 1/|A|) over a history window, eviction of
                  the lowest count outside the recent window.
* ``adaptive``  - FastGen's profiling step: the per-head composite chosen by
                  recovered attention over the last prompt rows.
* ``quant``     - the 4-bit cache format (groups of 32, float32 scale and
                  rounding) that [SH] combines with eviction; the H2O and
                  persistence loops take what a cache slot reads back.
* ``lockstep``  - replays a unit against a GPU run's logs with the near-tie
                  acceptance band, and measures the score and output errors.

Sources (cited per function):
  [H2O]  review page of "H2O: Heavy-Hitter Oracle for Efficient Generative
         Inference of Large Language Models" (nubint.ai), sections
         "研究の動機と目的" (motivation), "提案手法" (proposed method).
  [FG]   review page of "Model Tells You What to Discard: Adaptive KV Cache
         Compression for LLMs" (FastGen, nubint.ai): Abstract, "提案手法",
         Figure 2 caption.
  [SH]   summary page of "Scissorhands: Exploiting the Persistence of
         Importance Hypothesis for LLM KV Cache Compression at Test Time"
         (fugumt.com): Abstract.
  [HE]   summary page of "HashEvict: A Pre-Attention KV Cache Eviction
         Strategy using Locality-Sensitive Hashing" (jarxiv.com): 要約 and
         the original abstract.

Parity pins: every function is pinned by a CPU test against a textbook
routine, a closed form, an invariant or brute force (tests/test_oracle_*.py).
Parity unpinned: the H2O score trajectory for generic inputs beyond those
invariants, the brute-force checks and one trajectory worked by hand in exact
fractions (distinct keys, two evictions) -- the pages print no worked example; the
persistence rule itself is a reading of a one-sentence hypothesis, so its
pins (closed forms on constructed inputs, invariants, a replay of recorded
weights) check the oracle against that reading, not against the page; the
4-bit format is likewise a reading (the page names no format), pinned by
exact grids, brute-force nearest grid points and the rounding bound.
"""
