"""Pins of the oracle's bias-corrected KL term (reading R19).

Liger PR #1320 ("The implementation", "Testing") names a bias-corrected KL
option beside the K3 KL without printing it. The oracle reads it as K3
weighted by each token's importance ratio rho_t = exp(lp_t - old_t). The
pins below fix that reading by what the correction is for: averaged over
tokens drawn from the sampling policy, the corrected term must give the
exact KL divergence of the current policy from the reference (checked on an
enumerated three-outcome distribution against scipy's relative entropy),
its gradient, pushed through a softmax policy's score function, must be
the exact gradient of that divergence (on and off policy), it must match
finite differences of the oracle's own loss, and without old log-probs its
value must reduce to plain K3.
"""
import numpy as np
import pytest
from scipy.special import rel_entr

import oracle
from oracle.core import LossConfig, GMPO, GSPO_TOKEN, GRPO, BNPO, DAPO

LOSSES = (GMPO, GSPO_TOKEN, GRPO, BNPO, DAPO)


def _enumerated_batch():
    """One sequence whose 8 tokens are the outcomes y in {0, 1, 2} with
    multiplicities 1, 3, 4: an exact sample of pi_old = (1/8, 3/8, 4/8)."""
    pi = np.array([0.5, 0.3, 0.2])
    pi_old = np.array([1, 3, 4]) / 8.0
    pi_ref = np.array([0.2, 0.5, 0.3])
    ys = np.repeat(np.arange(3), [1, 3, 4])
    lp = np.log(pi[ys])
    old = np.log(pi_old[ys]).astype(np.float32)
    ref = np.log(pi_ref[ys]).astype(np.float32)
    return pi, pi_ref, lp, old, ref


@pytest.mark.parametrize("loss_type", LOSSES)
def test_corrected_kl_is_exact_divergence_under_sampler(loss_type):
    """mean over an exact pi_old sample of rho K3 = sum_y pi(y) K3(y) =
    KL(pi || pi_ref); the uncorrected mean is a different number. A = 0
    removes the policy term, beta = 1 and one sequence make the loss the
    token mean of the KL term; the mean_kl metric reports the same value."""
    pi, pi_ref, lp, old, ref = _enumerated_batch()
    T = lp.shape[0]
    comp = np.ones(T, np.uint8)
    A = np.zeros(1, np.float32)
    true_kl = float(rel_entr(pi, pi_ref).sum())
    cfg = LossConfig(B=1, T=T, loss_type=loss_type, beta=1.0, kl_bias_correction=True)
    part = oracle.policy_loss(cfg, lp, old, ref, comp, None, A)
    loss, m = oracle.finalize_metrics([part], np.float32(np.nan))
    # old and ref are fp32-rounded log-probs: the identity holds to ~1e-7
    assert abs(loss - true_kl) <= 2e-7 * max(1.0, true_kl), loss_type
    assert abs(m[3] - true_kl) <= 2e-7 * max(1.0, true_kl)
    plain = oracle.policy_loss(LossConfig(B=1, T=T, loss_type=loss_type, beta=1.0), lp, old, ref, comp, None, A)
    assert abs(plain["loss_sum"] - true_kl) > 1e-2


def _softmax(theta):
    e = np.exp(theta - theta.max())
    return e / e.sum()


@pytest.mark.parametrize("loss_type", LOSSES)
@pytest.mark.parametrize("on_policy", [False, True])
def test_corrected_kl_gradient_is_exact_divergence_gradient(loss_type, on_policy):
    """pi = softmax(theta) over three outcomes. For tokens sampled exactly
    from the sampler (pi_old, or pi itself on policy, as multiplicities 1, 3,
    4 of 8), sum_t g_t d lp_t / d theta, with d log pi(y) / d theta =
    onehot(y) - pi, must equal the gradient of KL(pi || pi_ref) in theta,
    taken here by central differences of scipy's relative entropy. Plain K3
    fails this (its expected gradient is that of the reverse divergence)."""
    pi_s = np.array([1, 3, 4]) / 8.0
    theta = np.log(pi_s) if on_policy else np.array([0.4, -0.1, -0.5])
    pi = _softmax(theta)
    pi_ref = np.array([0.2, 0.5, 0.3])
    ys = np.repeat(np.arange(3), [1, 3, 4])
    lp = np.log(pi[ys])
    old = None if on_policy else np.log(pi_s[ys]).astype(np.float32)
    ref = np.log(pi_ref[ys]).astype(np.float32)
    T = ys.shape[0]
    comp = np.ones(T, np.uint8)
    A = np.zeros(1, np.float32)
    score = np.eye(3)[ys] - pi[None, :]

    def kl_of(th):
        return float(rel_entr(_softmax(th), pi_ref).sum())

    eps = 1e-6
    want = np.array([(kl_of(theta + eps * np.eye(3)[k]) - kl_of(theta - eps * np.eye(3)[k])) / (2 * eps)
                     for k in range(3)])
    g = oracle.policy_loss(LossConfig(B=1, T=T, loss_type=loss_type, beta=1.0, kl_bias_correction=True),
                           lp, old, ref, comp, None, A)["g"]
    np.testing.assert_allclose(g @ score, want, rtol=1e-5, atol=1e-7)
    g_plain = oracle.policy_loss(LossConfig(B=1, T=T, loss_type=loss_type, beta=1.0), lp, old, ref, comp, None,
                                 A)["g"]
    assert np.abs(g_plain @ score - want).max() > 1e-2


def _random_problem(seed, B=3, T=9):
    rng = np.random.default_rng(seed)
    lp = -np.abs(rng.normal(1.0, 0.7, B * T))
    old = (lp + rng.normal(0.0, 0.3, B * T)).astype(np.float32)
    ref = (lp + rng.normal(0.0, 0.4, B * T)).astype(np.float32)
    comp = (rng.random(B * T) < 0.8).astype(np.uint8)
    comp[::T] = 1
    return lp, old, ref, comp


@pytest.mark.parametrize("loss_type", LOSSES)
def test_corrected_kl_gradient_matches_finite_differences(loss_type):
    """g = dL/dlp of the KL part (A = 0: no policy term) against central
    differences of the oracle's loss, per token, with the ratio
    differentiated through (its derivative in lp is itself)."""
    B, T = 3, 9
    lp, old, ref, comp = _random_problem(7, B, T)
    A = np.zeros(B, np.float32)
    cfg = LossConfig(B=B, T=T, loss_type=loss_type, beta=0.3, kl_bias_correction=True)
    g = oracle.policy_loss(cfg, lp, old, ref, comp, None, A)["g"]
    eps = 1e-5
    fd = np.empty_like(lp)
    for t in range(lp.shape[0]):
        up, dn = lp.copy(), lp.copy()
        up[t] += eps
        dn[t] -= eps
        fd[t] = (oracle.policy_loss(cfg, up, old, ref, comp, None, A)["loss_sum"]
                 - oracle.policy_loss(cfg, dn, old, ref, comp, None, A)["loss_sum"]) / (2 * eps)
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-9)
    # not the plain K3 gradient (the ratio factor and its derivative matter)
    g_plain = oracle.policy_loss(LossConfig(B=B, T=T, loss_type=loss_type, beta=0.3), lp, old, ref, comp, None,
                                 A)["g"]
    assert np.abs(g - g_plain).max() > 1e-3


def test_corrected_kl_adds_to_unclipped_policy_gradient():
    """GRPO with bounds too wide to bind: g is the policy gradient -A rho w
    plus beta times the KL gradient, and both together match finite
    differences of the full loss."""
    B, T = 2, 8
    lp, old, ref, comp = _random_problem(3, B, T)
    A = np.array([0.8, -1.3], np.float32)
    cfg = LossConfig(B=B, T=T, loss_type=GRPO, eps_low=0.99, eps_high=50.0, beta=0.5, kl_bias_correction=True)
    g = oracle.policy_loss(cfg, lp, old, ref, comp, None, A)["g"]
    eps = 1e-5
    for t in range(B * T):
        up, dn = lp.copy(), lp.copy()
        up[t] += eps
        dn[t] -= eps
        fd = (oracle.policy_loss(cfg, up, old, ref, comp, None, A)["loss_sum"]
              - oracle.policy_loss(cfg, dn, old, ref, comp, None, A)["loss_sum"]) / (2 * eps)
        assert abs(g[t] - fd) <= 1e-6 * max(1.0, abs(fd)), t


@pytest.mark.parametrize("loss_type", LOSSES)
def test_corrected_kl_on_policy_is_k3(loss_type):
    """Without old log-probs every ratio is 1: the corrected run's loss and
    KL metric equal the plain K3 run's exactly."""
    B, T = 3, 9
    lp, _, ref, comp = _random_problem(11, B, T)
    A = np.array([0.5, -0.7, 1.1], np.float32)
    a = oracle.policy_loss(LossConfig(B=B, T=T, loss_type=loss_type, beta=0.2, kl_bias_correction=True),
                           lp, None, ref, comp, None, A)
    b = oracle.policy_loss(LossConfig(B=B, T=T, loss_type=loss_type, beta=0.2), lp, None, ref, comp, None, A)
    assert a["loss_sum"] == b["loss_sum"]
    assert a["mean_kl_sum"] == b["mean_kl_sum"]
