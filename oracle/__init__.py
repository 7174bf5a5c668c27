"""Plain CPU oracle for one Medusa verify iteration -- TEST INFRASTRUCTURE ONLY.

This package is a slow, obviously-correct NumPy (float64) restatement of what
the Medusa decode iteration computes, written from the method as described on
the page "大模型推理 memory bandwidth bound (5) - Medusa" (section 一, the method:
Medusa heads, tree attention, typical acceptance; section 二, the code walk-through:
generate_medusa_buffers, generate_candidates, tree_decoding, evaluate_posterior,
update_inference_inputs) with the decoder shape left open by the pages filled in
as a pre-norm LLaMA-style block.

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from here.  The HIP product path never imports,
links or calls this package, and this package imports nothing from the product
path: both sides only share the seeded input generators in ``workloads``.

Modules
-------
numerics    bfloat16 round-to-nearest-even, SiLU, first-index argmax (fp64)
tree        static sparse-tree buffers from rank-path choices
heads       Medusa residual heads, top-K and the root argmax
candidates  flat candidate list -> tree tokens, positions, cartesian paths
attention   tree attention of T tree queries over a KV prefix + tree KV
decoder     pre-norm decoder forward over a batch of new tokens, plain greedy decode
posterior   greedy and typical ("fast") acceptance with longest-path choice
update      KV compaction / token append after acceptance
loop        whole Medusa generation loop and the plain greedy baseline
calib       tree calibration: expected accepted length, the best tree of n
            nodes from per-(depth, rank) acceptance, teacher-forced head hits

Every function that has no independent pin says "parity unpinned" in its
docstring; all others are pinned by ``tests/test_oracle_*.py``.
"""
