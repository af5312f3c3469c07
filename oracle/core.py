"""fp64 CPU oracle of the fused LM-head + GMPO / GSPO-token policy loss.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py; never by the product path.

Notation (rows are tokens, sequences are contiguous runs of T rows):
  z[t,v]  = (h_t . W_v + b_v) / tau                 logits, never stored whole
  lse_t   = log sum_v exp z[t,v]
  lp_t    = z[t, y_t] - lse_t                       target log-prob
  H_t     = lse_t - sum_v p[t,v] z[t,v]             entropy, p = softmax(z)
  lr_t    = lp_t - old_t                            log importance ratio
  M_i     = completion tokens of sequence i         (loss mask)
  R_i     = ratio tokens of sequence i              (defaults to M_i)
  n_i = max(1,|M_i|),  nt_i = max(1,|R_i|),  A_i = per-sequence advantage.

Readings taken where the pages are silent:
  R1  GMPO clip (Liger PR #1320, "The implementation", bullets 1 and 7): for
      A_i>0 the log-ratio is clipped from above only, c = min(lr, eps_high);
      for A_i<0 from below only, c = max(lr, -eps_low); this is PPO's
      pessimistic min taken in log space.
  R2  A_i = 0: the policy term and its gradient are exactly zero and the
      sequence ratio is not evaluated (it is reported as 1).
  R3  Ties at a bound are not clipped (strict predicate), so the gradient
      flows at equality, as autograd of min(x, clamp(x)) gives.
  R4  Clip predicates are decided in fp32: lr32 = fp32(fp32(lp) - old32)
      against fp32(eps). Clipped tokens take the fp32 bound as their value;
      everything else is fp64. GSPO bounds are fp32(1 - eps_low) and
      fp32(1 + eps_high); the sequence ratio is compared to them in fp64.
  R5  Per-sample reduction: masked mean over M_i per sequence, then the mean
      over all B sequences of the batch (global B, so outer chunking does not
      change the result).
  R6  The entropy mask multiplies the per-token policy term of every loss
      type, GMPO included (PR #1558, Details: the policy loss function
      applies the mask after its loss-type branch, for every type).
  R7  KL is K3, exp(ref - lp) - (ref - lp) - 1, reduced like the policy term
      and not multiplied by the entropy mask.
  R8  The clip metric is token-level over the loss tokens M and does not
      depend on the entropy mask; for GSPO the sequence predicate is broadcast
      to its tokens. The GSPO sequence clip fraction is two-sided.
  R9  Quantile: torch.quantile's linear interpolation on the fp32 active
      entropies at probability 1 - q, mask = active & H >= thr. No active
      token gives an all-false mask and a NaN threshold. q = 1 turns the mask
      off entirely. Past torch's 2^24-entry cap (PR #1558: a sort fallback)
      the rank is still fp32(p) * fp32(n - 1) rounded to fp32, and both order
      statistics are clamped to n - 1.
  R10 old_logp absent means on-policy (lr = 0); ratio_mask absent means R = M.
  R15 GRPO, BNPO and DAPO (named as loss types by Liger PR #1558, Testing,
      and PR #1320, Testing; their formulas are not printed): the token-level
      clipped surrogate of the Tinker GSPO page's objective with the token
      ratio rho_t = exp(lr_t) in place of the sequence ratio,
      policy_t = -min(rho_t A_i, clip(rho_t, 1-eps_low, 1+eps_high) A_i),
      over the completion tokens M (the ratio mask plays no part).
  R16 Their normalisations: GRPO the per-sample reduction of R5; BNPO the sum
      over every completion token of the batch divided by the number of those
      tokens; DAPO the same sum divided by a caller-given global token count
      (for gradient accumulation over several calls), defaulting to the
      batch's own count, where it equals BNPO.
  R17 Their clip predicate is decided on exp(lr32) in fp64 against
      fp32(1-eps_low) and fp32(1+eps_high); a clipped token takes the bound's
      value and no gradient.
  R18 Per-token advantages (Tinker GSPO page, "Input tensors": advantages
      of shape (N,); "Building a datum" zeroes them off the completion): the
      objective's min(s_t A_t, clip(s_t) A_t) takes each token's own A_t, so
      the clip binds per token by the sign of A_t. Defined for GSPO-token and
      the token-level clipped losses; GMPO's clip direction and geometric
      mean belong to the sequence, so it keeps per-sequence advantages.
  R19 Bias-corrected KL (Liger PR #1320, "The implementation" and
      "Testing" name the option; no formula is printed): the K3 term of
      every token is multiplied by that token's importance ratio
      rho_t = exp(lp_t - old_t), unclipped and differentiated through, so
      that its average over tokens drawn from the sampling policy is an
      estimate of KL(pi_theta || pi_ref) rather than of the same divergence
      weighted by the sampler. Without old log-probs rho_t = exp(lp - lp)
      with the second lp held constant, as for the policy terms: the value
      is plain K3 but the gradient keeps the ratio's own derivative, so it
      is lp_t - ref_t. The mean_kl metric reports the corrected term.
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction
from typing import Optional

import numpy as np

METRIC_NAMES = (
    "clip_fraction",
    "seq_log_ratio_mean",
    "clipped_seq_fraction",
    "mean_kl",
    "entropy_threshold",
    "entropy_kept_fraction",
    "active_tokens",
    "clipped_tokens",
)

GMPO = "gmpo"
GSPO_TOKEN = "gspo_token"
GRPO = "grpo"
BNPO = "bnpo"
DAPO = "dapo"
PPO_CLIP_LOSSES = (GRPO, BNPO, DAPO)


@dataclass(frozen=True)
class LossConfig:
    B: int
    T: int
    loss_type: str = GMPO
    eps_low: float = 0.4
    eps_high: float = 0.4
    beta: float = 0.0
    temperature: float = 1.0
    top_entropy_quantile: float = 1.0
    reduction: str = "seq_mean"      # "seq_mean" (per-sample) or "token_sum"; GMPO / GSPO only
    chunk_sequences: int = 0         # 0 = whole batch
    global_tokens: int = 0           # DAPO normaliser; 0 = the batch's completion tokens
    kl_bias_correction: bool = False  # R19: KL term = rho_t * K3

    @staticmethod
    def from_spec(spec) -> "LossConfig":
        return LossConfig(B=spec.B, T=spec.T, loss_type=spec.loss_type, eps_low=spec.eps_low,
                          eps_high=spec.eps_high, beta=spec.beta, temperature=spec.temperature,
                          top_entropy_quantile=spec.top_entropy_quantile,
                          reduction=spec.reduction, chunk_sequences=spec.chunk_sequences,
                          global_tokens=getattr(spec, "global_tokens", 0),
                          kl_bias_correction=getattr(spec, "kl_bias_correction", False))


# ---------------------------------------------------------------------------
# LM head forward: logits, log-sum-exp, target log-prob, entropy
# ---------------------------------------------------------------------------

def logits(h, W, b, tau: float) -> np.ndarray:
    """z = (h W^T + b) / tau in fp64 (the LM-head logits; PR #1558 tests divide
    by a temperature)."""
    z = np.asarray(h, np.float64) @ np.asarray(W, np.float64).T
    if b is not None:
        z = z + np.asarray(b, np.float64)[None, :]
    return z / tau


def forward_rows(h, W, b, tau: float, targets, chunk: int = 256) -> dict:
    """Exact full-vocabulary softmax statistics per row (no streaming).

    lse = m + log sum exp(z - m); lp = z_y - lse; H = lse - sum p z, which is
    the quantity PR #1558 accumulates as log_z - sum_exp_z / sum_exp.
    """
    W64 = np.asarray(W, np.float64)
    b64 = None if b is None else np.asarray(b, np.float64)
    h = np.asarray(h)
    N = h.shape[0]
    tg = np.asarray(targets, np.int64)
    lse = np.empty(N)
    lp = np.empty(N)
    ent = np.empty(N)
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        z = logits(h[r0:r1], W64, b64, tau)
        m = z.max(axis=1)
        e = np.exp(z - m[:, None])
        s = e.sum(axis=1)
        l = m + np.log(s)
        p = e / s[:, None]
        lse[r0:r1] = l
        lp[r0:r1] = z[np.arange(r1 - r0), tg[r0:r1]] - l
        ent[r0:r1] = l - (p * z).sum(axis=1)
    return {"lse": lse, "logp": lp, "entropy": ent}


# ---------------------------------------------------------------------------
# Batch-global entropy quantile and mask (PR #1558)
# ---------------------------------------------------------------------------

def _fma32(a, b, c) -> np.float32:
    """fp32 fused multiply-add, rounded once (exact rational arithmetic)."""
    return np.float32(float(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))))


def quantile_linear_f32(x32, prob: float) -> np.float32:
    """torch.quantile(x, prob, interpolation='linear') on an fp32 vector.

    Definition: sort ascending; rank = prob * (n - 1) in fp32; interpolate
    between the order statistics floor(rank) and ceil(rank) with weight
    w = rank - floor(rank). The interpolation is a single-rounding lerp,
    a + w (b - a) for w < 1/2 and b + (w - 1)(b - a) otherwise. (This is the
    form torch's CPU kernel produces bit for bit; tests pin it against
    torch.quantile.)

    Past 2^24 entries, where torch.quantile refuses the input and Liger PR
    #1558 ("Details", the large-input bullet) falls back to a sort, the same
    fp32 rank is kept (R9) and both order statistics are clamped to the last
    one: fp32(n - 1) can round up to n there.
    """
    xs = np.sort(np.asarray(x32, np.float32))
    n = xs.shape[0]
    if n == 0:
        return np.float32(np.nan)
    p32 = np.float32(prob)
    rank = np.float32(p32 * np.float32(n - 1))
    lo = min(int(np.floor(rank)), n - 1)
    hi = min(int(np.ceil(rank)), n - 1)
    w = np.float32(rank - np.float32(lo))
    a, b = xs[lo], xs[hi]
    d = np.float32(b - a)
    if w < np.float32(0.5):
        return _fma32(w, d, a)
    return _fma32(np.float32(w - np.float32(1.0)), d, b)


def entropy_quantile_mask(H32, active, q: float):
    """High-entropy token mask (PR #1558, Details bullet 2).

    thr = quantile of the active tokens' entropies at 1 - q, one threshold
    for the batch;
    mask = active & H >= thr. q = 1 keeps every active token (the feature off).
    Returns (mask bool [N], thr float32, NaN when undefined).
    """
    H32 = np.asarray(H32, np.float32)
    active = np.asarray(active).astype(bool)
    if not (0.0 <= q <= 1.0):
        raise ValueError("top_entropy_quantile must lie in [0, 1]")
    if q == 1.0:
        return active.copy(), np.float32(np.nan)
    vals = H32[active]
    if vals.size == 0:
        return np.zeros_like(active), np.float32(np.nan)
    thr = quantile_linear_f32(vals, 1.0 - q)
    return active & (H32 >= thr), thr


# ---------------------------------------------------------------------------
# Policy loss from per-token log-probs: GMPO, GSPO-token, K3 KL
# ---------------------------------------------------------------------------

def token_normaliser(cfg: LossConfig, completion_mask) -> int:
    """BNPO / DAPO divisor (R16): the caller's global token count for DAPO
    when given, else the number of completion tokens of the whole batch."""
    if cfg.loss_type == DAPO and cfg.global_tokens > 0:
        return int(cfg.global_tokens)
    return max(1, int((np.asarray(completion_mask) != 0).sum()))


def policy_loss(cfg: LossConfig, lp, old, ref, completion_mask, ratio_mask, advantages,
                entropy_mask=None, seq_offset: int = 0, B_total: Optional[int] = None,
                tokens_total: Optional[int] = None, token_advantages=None) -> dict:
    """Loss, metrics and g = dL/dlp for a run of whole sequences.

    lp: fp64 (or fp32) [b*T]; old, ref: fp32 [b*T] or None; masks u8/bool
    [b*T]; advantages fp32 [b]; entropy_mask bool [b*T] or None (= all ones).
    B_total is the batch size that divides the per-sample reduction (R5);
    tokens_total the BNPO / DAPO divisor (R16; default: from this run).
    token_advantages fp32 [b*T] replaces `advantages` with one value per
    token (R18; not for GMPO).

    GMPO (Liger PR #1320): c_t clipped per R1; r_i = exp(mean_{R_i} c);
    per-token policy term -A_i r_i.  GSPO-token (Tinker GSPO page): sequence
    log-ratio ls_i = mean_{R_i} lr; s_i = exp(ls_i); every token carries the
    value s_i with the gradient of its own log-prob; policy term
    -min(s A, clip(s, 1-eps_low, 1+eps_high) A).  Loss per token
    l_t = e_t policy_t + beta kl_t (R6, R7; kl_t = rho_t K3_t under R19),
    reduced per R5.
    """
    T = cfg.T
    lp = np.asarray(lp, np.float64)
    b = lp.shape[0] // T
    Bt = cfg.B if B_total is None else B_total
    lp = lp.reshape(b, T)
    lp32 = lp.astype(np.float32)
    old32 = lp32 if old is None else np.asarray(old, np.float32).reshape(b, T)
    lr32 = (lp32 - old32).astype(np.float32)               # fp32 predicate operand (R4)
    lr = lp - old32.astype(np.float64)                       # fp64 value
    M = np.asarray(completion_mask).reshape(b, T) != 0
    R = M if ratio_mask is None else (np.asarray(ratio_mask).reshape(b, T) != 0)
    e = np.ones((b, T), bool) if entropy_mask is None else (np.asarray(entropy_mask).reshape(b, T) != 0)
    if token_advantages is not None:
        if cfg.loss_type == GMPO:
            raise ValueError("GMPO takes per-sequence advantages (R18)")
        At = np.asarray(token_advantages, np.float32).astype(np.float64).reshape(b, T)
        A = None
    else:
        A = np.asarray(advantages, np.float32).astype(np.float64).reshape(b)
        At = np.broadcast_to(A[:, None], (b, T))
    n = np.maximum(1, M.sum(axis=1)).astype(np.float64)
    nt = np.maximum(1, R.sum(axis=1)).astype(np.float64)
    if cfg.loss_type == GRPO:
        w = 1.0 / (Bt * n)
    elif cfg.loss_type in (BNPO, DAPO):
        G = token_normaliser(cfg, M) if tokens_total is None else tokens_total
        w = np.full(b, 1.0 / G)
    elif cfg.reduction == "seq_mean":
        w = 1.0 / (Bt * n)
    elif cfg.reduction == "token_sum":
        w = np.ones(b)
    else:
        raise ValueError(cfg.reduction)

    seq_log_ratio = (np.where(R, lr, 0.0)).sum(axis=1) / nt
    if cfg.loss_type == GMPO:
        eh = np.float32(cfg.eps_high)
        el = np.float32(cfg.eps_low)
        clip_hi = R & (A > 0)[:, None] & (lr32 > eh)
        clip_lo = R & (A < 0)[:, None] & (lr32 < -el)
        clipped_tok = clip_hi | clip_lo
        c = np.where(clip_hi, float(eh), np.where(clip_lo, -float(el), lr))
        mean_c = np.where(R, c, 0.0).sum(axis=1) / nt
        with np.errstate(over="ignore"):
            r = np.where(A != 0, np.exp(np.where(A != 0, mean_c, 0.0)), 1.0)
        policy_seq = np.where(A != 0, -A * r, 0.0)
        K = (e & M).sum(axis=1).astype(np.float64)
        coef = np.where(A != 0, -A * r * K, 0.0) / nt
        g_pol = coef[:, None] * (R & ~clipped_tok)
        seq_ratio = r
        clipped_seq = np.zeros(b, bool)
        clipped_seq_any = np.zeros(b, bool)
    elif cfg.loss_type == GSPO_TOKEN and A is None:
        # per-token advantages (R18): each token's min(s A_t, clip(s) A_t)
        lo = np.float32(1.0 - cfg.eps_low)
        hi = np.float32(1.0 + cfg.eps_high)
        s = np.exp(seq_log_ratio)
        sc = s[:, None]
        held = ((At > 0) & (sc > float(hi))) | ((At < 0) & (sc < float(lo)))
        clipped_tok = M & held
        s_cl = np.clip(sc, float(lo), float(hi))
        live = (At != 0) & ~held                             # A_t = 0: no term, no gradient
        s_l = np.where(live, sc, 0.0)
        # min(s A_t, clip(s) A_t) is the clipped value exactly where `held`
        pol_tok_gspo = np.where(held, -s_cl * At, -s_l * At)
        g_pol = np.where(e & M & live, -At * s_l, 0.0)
        seq_ratio = s
        clipped_seq = clipped_tok.any(axis=1)
        clipped_seq_any = (s < lo) | (s > hi)
    elif cfg.loss_type == GSPO_TOKEN:
        lo = np.float32(1.0 - cfg.eps_low)
        hi = np.float32(1.0 + cfg.eps_high)
        s = np.exp(seq_log_ratio)
        clipped_seq = ((A > 0) & (s > hi)) | ((A < 0) & (s < lo))
        s_cl = np.clip(s, float(lo), float(hi))
        policy_seq = -np.minimum(s * A, s_cl * A)
        g_tok = np.where(clipped_seq, 0.0, -A * s)
        g_pol = g_tok[:, None] * (e & M)
        clipped_tok = np.broadcast_to(clipped_seq[:, None], (b, T)) & M
        seq_ratio = s
        clipped_seq_any = (s < lo) | (s > hi)
    elif cfg.loss_type in PPO_CLIP_LOSSES:
        lo = np.float32(1.0 - cfg.eps_low)
        hi = np.float32(1.0 + cfg.eps_high)
        Ac = At
        with np.errstate(over="ignore"):
            rho_pred = np.exp(lr32.astype(np.float64))      # R17
            rho = np.exp(lr)
        clip_hi = M & (Ac > 0) & (rho_pred > float(hi))
        clip_lo = M & (Ac < 0) & (rho_pred < float(lo))
        clipped_tok = clip_hi | clip_lo
        live = (Ac != 0) & ~clipped_tok                      # A = 0: no term, no gradient (R2)
        rho_l = np.where(live, rho, 0.0)
        # -min(rho A, clip(rho, lo, hi) A): the bound where the clip binds
        pol_ppo = np.where(clip_hi, -float(hi) * Ac, np.where(clip_lo, -float(lo) * Ac, -rho_l * Ac))
        g_pol = np.where(e & M & live, -rho_l * Ac, 0.0)
        with np.errstate(over="ignore"):
            seq_ratio = np.exp(seq_log_ratio)
        clipped_seq = np.zeros(b, bool)
        clipped_seq_any = np.zeros(b, bool)
    else:
        raise ValueError(cfg.loss_type)

    if cfg.loss_type in PPO_CLIP_LOSSES:
        policy_tok = pol_ppo
    elif cfg.loss_type == GSPO_TOKEN and A is None:
        policy_tok = pol_tok_gspo
    else:
        policy_tok = np.broadcast_to(policy_seq[:, None], (b, T))
    if ref is not None:
        x = np.asarray(ref, np.float32).astype(np.float64).reshape(b, T) - lp
        k3 = np.exp(x) - x - 1.0
        dk3 = 1.0 - np.exp(x)                                 # d K3 / d lp
        if cfg.kl_bias_correction:
            # R19: rho_t K3_t; d rho_t / d lp_t = rho_t (product rule), on
            # policy too (rho = exp(lp - const) = 1)
            with np.errstate(over="ignore"):
                rho_kl = np.ones((b, T)) if old is None else np.exp(lr)
            kl = rho_kl * k3
            dkl = rho_kl * k3 + rho_kl * dk3
        else:
            kl = k3
            dkl = dk3
    else:
        kl = np.zeros((b, T))
        dkl = np.zeros((b, T))
    beta = cfg.beta
    ell = np.where(e, policy_tok, 0.0) + beta * kl
    seq_sum = np.where(M, ell, 0.0).sum(axis=1)
    loss_sum = float((w * seq_sum).sum())
    g = w[:, None] * (g_pol + beta * np.where(M, dkl, 0.0))

    n_active = int(M.sum())
    n_clipped = int((clipped_tok & M).sum())
    n_kept = int((e & M).sum())
    mean_kl_sum = float((np.where(M, kl, 0.0).sum(axis=1) / n).sum())
    return {
        "loss_sum": loss_sum,                 # this run's contribution to L
        "g": g.reshape(-1),
        "lr32": lr32.reshape(-1),
        "clipped_tok": np.asarray(clipped_tok).reshape(-1),
        "seq_ratio": seq_ratio,
        "seq_log_ratio": seq_log_ratio,
        "clipped_seq": clipped_seq,
        "clipped_seq_any": clipped_seq_any,
        "counts": (n_active, n_clipped, n_kept),
        "mean_kl_sum": mean_kl_sum,
        "B_total": Bt,
    }


def finalize_metrics(parts, thr) -> tuple:
    """Combine per-chunk policy_loss results into (loss, metrics fp64 array)."""
    loss = sum(p["loss_sum"] for p in parts)
    Bt = parts[0]["B_total"]
    n_active = sum(p["counts"][0] for p in parts)
    n_clip = sum(p["counts"][1] for p in parts)
    n_kept = sum(p["counts"][2] for p in parts)
    slr = sum(float(p["seq_log_ratio"].sum()) for p in parts) / Bt
    cseq = sum(int(p["clipped_seq_any"].sum()) for p in parts) / Bt
    mkl = sum(p["mean_kl_sum"] for p in parts) / Bt
    den = np.float32(max(1, n_active))
    m = np.array([
        np.float32(n_clip) / den,
        slr,
        cseq,
        mkl,
        float(thr),
        np.float32(n_kept) / den if n_active else 0.0,
        n_active,
        n_clip,
    ], dtype=np.float64)
    return loss, m


# ---------------------------------------------------------------------------
# Backward of the fused linear layer
# ---------------------------------------------------------------------------

def _dz(z, lse, g, y, tau):
    """dL/dz = g_t (onehot(y_t) - softmax(z_t)) / tau, since
    d lp_t / d z[t,v] = [v = y_t] - p[t,v] and z carries the 1/tau."""
    dz = -np.exp(z - lse[:, None])
    dz[np.arange(z.shape[0]), y] += 1.0
    dz *= (g / tau)[:, None]
    return dz


def backward(h, W, b, tau: float, targets, lse, g, chunk: int = 256):
    """grad_h = dz W, grad_W = dz^T h, grad_b = sum_t dz with
    dz = g (onehot - softmax) / tau (PR #1320, The implementation: the
    fused layer returns gradients for h, W and b)."""
    W64 = np.asarray(W, np.float64)
    b64 = None if b is None else np.asarray(b, np.float64)
    h = np.asarray(h)
    N = h.shape[0]
    y = np.asarray(targets, np.int64)
    lse = np.asarray(lse, np.float64)
    g = np.asarray(g, np.float64)
    gh = np.zeros((N, W64.shape[1]))
    gW = np.zeros_like(W64)
    gb = np.zeros(W64.shape[0])
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        if not np.any(g[r0:r1]):
            continue
        h64 = np.asarray(h[r0:r1], np.float64)
        dz = _dz(logits(h64, W64, b64, tau), lse[r0:r1], g[r0:r1], y[r0:r1], tau)
        gh[r0:r1] = dz @ W64
        gW += dz.T @ h64
        gb += dz.sum(axis=0)
    return gh, gW, gb


def grad_h_rows(h_rows, W, b, tau, y_rows, lse_rows, g_rows):
    """grad_h for a subset of tokens, full vocabulary."""
    W64 = np.asarray(W, np.float64)
    dz = _dz(logits(h_rows, W64, b, tau), np.asarray(lse_rows, np.float64),
             np.asarray(g_rows, np.float64), np.asarray(y_rows, np.int64), tau)
    return dz @ W64


def grad_w_rows(h, W_rows, b_rows, tau, targets, lse, g, vrows, chunk: int = 65536):
    """grad_W[v] and grad_b[v] for a subset of vocabulary rows, summed over all
    tokens: sum_t g_t ([y_t = v] - exp(z[t,v] - lse_t)) h_t / tau."""
    vrows = np.asarray(vrows, np.int64)
    Wr = np.asarray(W_rows, np.float64)
    br = None if b_rows is None else np.asarray(b_rows, np.float64)
    y = np.asarray(targets, np.int64)
    lse = np.asarray(lse, np.float64)
    g = np.asarray(g, np.float64)
    N = y.shape[0]
    gW = np.zeros((len(vrows), Wr.shape[1]))
    gb = np.zeros(len(vrows))
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        h64 = np.asarray(h[r0:r1], np.float64)
        z = logits(h64, Wr, br, tau)
        dz = (y[r0:r1, None] == vrows[None, :]) - np.exp(z - lse[r0:r1, None])
        dz *= (g[r0:r1] / tau)[:, None]
        gW += dz.T @ h64
        gb += dz.sum(axis=0)
    return gW, gb


# ---------------------------------------------------------------------------
# The whole path
# ---------------------------------------------------------------------------

def run(cfg: LossConfig, h, W, b, targets, old, ref, completion_mask, ratio_mask, advantages,
        want_grads: bool = True, fwd: Optional[dict] = None, token_advantages=None) -> dict:
    """Forward statistics, batch-global entropy mask, loss and gradients.

    The outer loop walks chunks of whole sequences (PR #1320 tests outer chunk
    sizes 1, 2 and 5); the entropy threshold is taken over the whole batch
    before any chunk's loss (PR #1558: one-sequence chunks give the unchunked result).
    """
    B, T = cfg.B, cfg.T
    tau = cfg.temperature
    if fwd is None:
        fwd = forward_rows(h, W, b, tau, targets)
    lp, ent, lse = fwd["logp"], fwd["entropy"], fwd["lse"]
    H32 = ent.astype(np.float32)
    active = np.asarray(completion_mask) != 0
    q = cfg.top_entropy_quantile
    if q < 1.0:
        emask, thr = entropy_quantile_mask(H32, active, q)
    else:
        emask, thr = None, np.float32(np.nan)
    cs = cfg.chunk_sequences if cfg.chunk_sequences > 0 else B
    G = token_normaliser(cfg, completion_mask)   # batch-global, like B (R16)
    parts = []
    g = np.zeros(B * T)
    for s0 in range(0, B, cs):
        s1 = min(B, s0 + cs)
        sl = slice(s0 * T, s1 * T)
        p = policy_loss(cfg, lp[sl], None if old is None else old[sl], None if ref is None else ref[sl],
                        completion_mask[sl], None if ratio_mask is None else ratio_mask[sl],
                        None if advantages is None else advantages[s0:s1],
                        None if emask is None else emask[sl], B_total=B, tokens_total=G,
                        token_advantages=None if token_advantages is None else token_advantages[sl])
        g[sl] = p["g"]
        parts.append(p)
    loss, metrics = finalize_metrics(parts, thr)
    out = {"loss": loss, "metrics": metrics, "logp": lp, "entropy": ent, "lse": lse,
           "entropy_mask": emask, "threshold": thr, "g": g, "parts": parts}
    if want_grads:
        gh = np.zeros((B * T, np.asarray(W).shape[1]))
        gW = np.zeros((np.asarray(W).shape[0], np.asarray(W).shape[1]))
        gb = np.zeros(np.asarray(W).shape[0])
        for s0 in range(0, B, cs):
            s1 = min(B, s0 + cs)
            sl = slice(s0 * T, s1 * T)
            a, bW, bb = backward(h[sl], W, b, tau, targets[sl], lse[sl], g[sl])
            gh[sl] = a
            gW += bW
            gb += bb
        out.update(grad_h=gh, grad_W=gW, grad_b=gb)
    return out
