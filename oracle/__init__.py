"""CPU oracle of the LTE sparse-attention layer and of the linear-attention layer
of the hybrid -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the HIP path never does.
"""
from .lte_oracle import (  # noqa: F401
    LayerCache, all_ends, attention, attention_on_set, cnn_logits, cnn_logits_seq, cnn_scores,
    prefill, retained_set, retention_ends, sigmoid_to_f32, visible_indices, visible_set,
)
from .linear_oracle import linear_recurrent, linear_step  # noqa: F401,E402
