"""CPU oracle for the fused LM-head + GRPO-family policy loss (TEST INFRASTRUCTURE).

Plain, slow, fp64 numpy. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path never does.

Sources it follows (the pages):
  * Liger-Kernel PR #1320 "Add GMPO to fused linear GRPO loss", Summary and
    "The implementation" bullets: advantage-dependent one-sided clipping of the
    per-token log-ratio in log space [-eps_low, +eps_high]; exp of the masked
    mean per completion; per-sample reduction; K3 KL (optionally bias
    corrected, reading R19); clipping metric;
    chunking; input/weight/bias gradients.
  * Liger-Kernel PR #1558 "support top_entropy_quantile", Details bullets:
    entropy H = log_z - sum_exp_z / sum_exp; batch-global threshold
    quantile(active entropies, 1 - q); the mask multiplies the policy term
    before the KL penalty.
  * Tinker "GSPO" page, the sequence ratio, the GSPO-token ratio and the GSPO
    objective equations, and "Choosing clipping thresholds".
  * The token-level clipped losses GRPO, BNPO and DAPO, which Liger PR #1558
    (Testing) and PR #1320 (Testing) name without printing them: the Tinker
    page's clipped objective with a per-token ratio (readings R15-R17).

Every function in ``core`` states the passage it follows and, where the pages
are silent, the reading it takes.
"""
from .core import (  # noqa: F401
    logits,
    forward_rows,
    quantile_linear_f32,
    entropy_quantile_mask,
    policy_loss,
    backward,
    grad_h_rows,
    grad_w_rows,
    run,
    finalize_metrics,
    token_normaliser,
    LossConfig,
    METRIC_NAMES,
    GMPO,
    GSPO_TOKEN,
    GRPO,
    BNPO,
    DAPO,
    PPO_CLIP_LOSSES,
)
