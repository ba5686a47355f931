"""Plain, slow CPU oracle for tree-packed attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
anything in this package; only the tests, the graft smoke check and the bench's
CPU-baseline leg do. It shares no code with the HIP library: it is written from
the pages' definitions (trie packing and depth positions on the "Trie packing"
visualization page and in "Tree Training" §3.1-3.2; the compressed prefix tree
of the Claw-R1 "Prefix Tree Merge" page) in float64 NumPy.

Modules
-------
pack       trie insert, chain compression, preorder DFS, depth positions,
           subtree ends, path counts g, weights g/K, occurrence maps
attention  per-branch causal attention with RoPE (forward and backward), a
           dense-mask packed formulation for tiny inputs, and per-row /
           per-key ancestor-chain formulations for sampled checks
logprob    log-softmax gather, weighted loss and the scatter-added gradient
           on shared logit rows; occurrence-form and unique-form entries
tiles      (q-tile, k-tile) classification counts from subtree ends
ssm        tree-routed gated delta rule (per-token recurrence, its reverse
           mode, the per-branch and chunked forms) and the tree causal conv1d
partition  the partition planner's cut and pack, with a brute-force minimum
"""
from . import pack, attention, logprob, tiles, ssm, partition  # noqa: F401
