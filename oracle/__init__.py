"""CPU oracle for the fused chunked KL loss — TEST INFRASTRUCTURE, not product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package. The product path
(``chunked_kl_loss_amd``) never imports it and shares no code with it.

See ``oracle.kl`` for the definitions and their sources.
"""
from .kl import (  # noqa: F401
    teacher_distribution,
    student_log_softmax,
    forward,
    backward,
    loss_and_grads,
    dense_kl_loss,
    sampled_rows,
    dw_rows,
    logits_forward,
    logits_backward,
    logits_sampled_rows,
    kept_positions,
    IGNORE_ID,
    jsd_forward,
    jsd_backward,
    jsd_loss_and_grads,
    ALT_LOSSES,
    alt_forward,
    alt_backward,
    alt_loss_and_grads,
    topk_rkl_forward,
    topk_rkl_backward,
    topk_rkl_loss_and_grads,
    topk_rkl_sampled,
)
