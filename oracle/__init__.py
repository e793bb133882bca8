"""CPU oracle (test infrastructure only; never used by the product path)."""
from .kl_oracle import (  # noqa: F401
    teacher_log_probs,
    student_log_softmax,
    row_terms,
    logit_grad,
    loss_from_logits,
    kl_dense,
    kl_rows,
)
from .topk_oracle import topk_rows  # noqa: F401,E402
