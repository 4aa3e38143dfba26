"""CPU oracle for the DDTree tree-verify step -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct NumPy code in fp64.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The HIP library never calls into it and it never calls into the
HIP library; the two share no code.  Inputs come from ``synth`` (seeded
random numbers only).

What the step computes (sources)
--------------------------------
* The step verifies a budget-sized draft token tree with the target in one
  pass, replacing chain verification (lucebox-hub README, "02 · DFlash
  DDtree ...", "Algorithms used": DDTree tree-structured verify).
* Its linear-attention layers need tree-aware causal conv and tree-aware
  gated delta-net kernels whose state can be rolled back to the accepted
  node (same section, "Implemented here": ssm_conv_tree,
  gated_delta_net_tree, gated_delta_net_tree_persist).
* Acceptance is greedy (temperature 0) against the target's argmax, computed
  on device and validated (codehub lucebox-hub@main, "Run the Server",
  "Making requests"; "GPU draft top-K & verify-argmax (DFlash)").
* Attention is full attention over the KV cache, optionally paged
  (codehub lucebox-hub@main, "Server flags", --fa-window default 0;
  Luce-Org/lucebox README, "Inference Engine Optimizations").
* Ahead of the step (a widening of it): the draft model's top-K tokens and
  log-sum-exp per draft position are read from the device logits (codehub
  lucebox-hub@main, "GPU draft top-K & verify-argmax (DFlash)"), and
  DDTree builds the budget-N tree from them (draft.py states the reading).
* A second widening fuses a linear-attention layer's input stage into the
  delta-net: tree conv, SiLU, split into q | k | v and L2 normalisation of
  q and k (the Gated DeltaNet layer), the pages' idea being fewer launches
  per forward (lucebox-hub README, "01 · Megakernel"); fused.py states the
  readings.
* Under sampling (temperature > 0, the model card's top_p and top_k when a
  request gives none: codehub lucebox-hub@main, "Making requests") each
  node's verify sample replaces its argmax in the walk; sample.py states
  the reading of that acceptance rule, which the pages do not give.

The pages give names and roles, not formulas.  The recurrence is the
standard gated delta rule (Yang, Kautz, Hatamizadeh, "Gated Delta Networks",
2024): S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t.
The defining property of tree verification is that every tree node sees
exactly the sequence ``committed context ++ its root-to-node path``; every
function here computes a node's result by processing that explicit
sequence.  Readings of the pages' gaps are listed in each module.

Parity status: every function is pinned by tests/test_oracle_*.py against
closed forms, library routines (torch CPU conv1d / softmax attention,
numpy argmax and stable sort, scipy logsumexp), hand-worked golden cases or
brute force on tiny inputs.
"""
from .tree import validate_tree, depth, root_path, ancestor_mask, conv_window, TreeError  # noqa: F401
from .conv import tree_conv  # noqa: F401
from .gdn import gdn_chain, tree_gdn, tree_gdn_recurrent  # noqa: F401
from .attn import tree_attn, gather_cache, dequant_q8  # noqa: F401
from .walk import argmax_rows, accept_walk  # noqa: F401
from .commit import commit_gdn_state, commit_conv_prefix, commit_kv  # noqa: F401
from .draft import draft_topk, log_probs, build_tree, build_tree_brute  # noqa: F401
from .fused import qkv_split_norm, tree_conv_gdn, L2_EPS  # noqa: F401
from .sample import filtered_dist, sample_row, sample_tokens  # noqa: F401
