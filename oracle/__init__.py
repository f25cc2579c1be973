"""CPU fp64 oracle for the contextually sparse decoder-layer step.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check of the package
entry point and the CPU-baseline leg of the bench may import this package. The
HIP library and its Python binding never import, call or link anything here,
and nothing here imports them.

Every function is the plain, slow definition of what the step computes, in
float64 (fp16/fp32 inputs convert to float64 exactly). Sparse selections are
applied as masks over the dense computation ("dense with mask"): a term whose
mask is 0 is multiplied by an exact zero.

Sources (the pages this follows):
* "DejaVu Guide: Contextual Sparsity for LLM Inference" (a blog guide):
  sections "Mathematical Formulation of Lookahead Predictors" (the two top-k
  mask equations), "Head-Pruned Attention Dispatch", "The Synchronous
  Prediction Dilemma" (the FFN equation), "Step-by-Step Implementation"
  (predictor, sparse MLP and layer sketch), "Blocked Channel Sparsity" and
  "Mathematical Modeling"; predictor targets in ``train.py``.
* "Deja Vu: How Contextual Sparsity Accelerates LLM Inference by 6x" (a blog
  summary): "What Is Contextual Sparsity?" (sparsity levels, online phase; the
  offline phase that trains the predictors, ``train.py``).

Pinned by tests/test_oracle_*.py against closed forms, invariants, brute force
on tiny inputs and the printed worked example; each function's docstring
names its pins.
"""
from .dejavu import (  # noqa: F401
    predict, topk, topk_order_key, rmsnorm, qkv_all_heads, attention, mlp, layer,
    masks_from_sets, block_scores, expand_blocks, RMS_EPS,
)
from .train import (  # noqa: F401
    layer_labels, sigmoid, bce_logits, predictor_loss_grad, train_predictor, recall,
)
