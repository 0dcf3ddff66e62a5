"""Oracle for the routed-MoE layer served from a per-layer cache of hot experts.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The library never imports or calls it
and shares no code with it; the two meet only through the seeded inputs of the
`synth` package.

What it computes (plain, slow, fp64 unless stated):

* q4        -- decoding of 18-byte / 32-weight Q4_0 blocks.
* routing   -- router logits in one fixed fp32 summation order, top-k with ties
               to the lower expert id, softmax gating weights.
* expert    -- the SwiGLU expert MLP on dequantised weights.
* layer     -- the full layer over all routed experts: the cache moves where an
               expert is computed, not what the layer computes ("How it works",
               llama.cpp + MoE expert cache: every expert is computed exactly
               once, on the GPU or on the CPU).
* lru       -- the per-layer slot table as a step-by-step LRU simulator
               (longhaul.md, "Longhaul MoE loading": fixed budget, LRU per layer,
               experts of the batch protected, duplicates loaded once, staged
               execution when the batch needs more experts than there are slots).

Parity pins live in tests/test_oracle_*.py.  Functions without one are marked
"parity unpinned" in their docstring.
"""
