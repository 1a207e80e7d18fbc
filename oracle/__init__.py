"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .lce_oracle import *  # noqa: F401,F403
from .lce_oracle import (linear_cross_entropy, softmax_cross_entropy,  # noqa: F401
                         rows_forward, rows_grad_x, columns_grad_w_b,
                         target_masks, corrected_targets, row_weights, logits,
                         logsumexp_rows, row_losses, reduce_loss, dlogits,
                         linear_grads, argmax_rows)
