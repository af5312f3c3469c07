"""Pins of the oracle's token-level clipped losses (GRPO, BNPO, DAPO).

Liger PR #1558 (Testing) and PR #1320 (Testing) name these loss types
without printing them; the oracle reads them as the Tinker GSPO page's
clipped objective with a per-token ratio, normalised per sample (GRPO), by
the batch's completion tokens (BNPO) or by a caller-given global token count
(DAPO). Each test checks the oracle against a closed form, an equivalent
one-sided formulation, an invariant between the normalisations, finite
differences or torch autograd of an independently written definition.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.core import LossConfig, GRPO, BNPO, DAPO

torch.set_default_dtype(torch.float64)

PPO = (GRPO, BNPO, DAPO)


def _rng(seed):
    return np.random.default_rng(seed)


def _comp(B, T, prompt):
    comp = np.zeros((B, T), np.uint8)
    for i in range(B):
        comp[i, prompt[i]:] = 1
    return comp.reshape(-1)


@pytest.mark.parametrize("loss_type", PPO)
def test_on_policy_closed_form(loss_type):
    """old = lp: every token ratio is 1, inside any clip range, so the policy
    term is -A_i per completion token. GRPO: L = -(1/B) sum A_i; BNPO and
    DAPO (no global count): L = -sum_i A_i n_i / sum_i n_i; g_t = -A_i w_i."""
    B, T = 5, 11
    prompt = [0, 3, 5, 10, 1]
    comp = _comp(B, T, prompt)
    r = _rng(1)
    lp = r.uniform(-7, -0.2, B * T)
    old = lp.astype(np.float32)
    A = np.array([1.3, -0.7, 0.0, 2.0, -1.1], np.float32)
    Ad = A.astype(np.float64)
    cfg = LossConfig(B=B, T=T, loss_type=loss_type, eps_low=0.2, eps_high=0.3)
    out = oracle.policy_loss(cfg, old.astype(np.float64), old, None, comp, None, A)
    n = comp.reshape(B, T).sum(1).astype(np.float64)
    if loss_type == GRPO:
        want = -Ad.sum() / B
        w = 1.0 / (B * n)
    else:
        want = -(Ad * n).sum() / n.sum()
        w = np.full(B, 1.0 / n.sum())
    assert out["loss_sum"] == pytest.approx(want, abs=1e-15)
    g_want = (-Ad * w)[:, None] * comp.reshape(B, T)
    np.testing.assert_allclose(out["g"], g_want.reshape(-1), rtol=1e-15, atol=0)
    assert not out["clipped_tok"].any()


def test_single_token_one_sided_form():
    """T = 1: the clipped surrogate equals its one-sided form, -A min(rho, hi)
    for A > 0 and -A max(rho, lo) for A < 0, and its derivative w.r.t. lp is
    -A rho where the ratio is not held at a bound, 0 where it is."""
    r = _rng(2)
    B, T = 600, 1
    el, eh = 0.2, 0.28
    lp = r.uniform(-5, -0.5, B)
    old = (lp + r.uniform(-0.7, 0.7, B)).astype(np.float32)
    A = r.standard_normal(B).astype(np.float32)
    A[::9] = 0
    comp = np.ones(B, np.uint8)
    cfg = LossConfig(B=B, T=T, loss_type=GRPO, eps_low=el, eps_high=eh)
    out = oracle.policy_loss(cfg, lp, old, None, comp, None, A)
    rho = np.exp(lp - old.astype(np.float64))
    lo, hi = float(np.float32(1 - el)), float(np.float32(1 + eh))
    Ad = A.astype(np.float64)
    want = np.where(Ad > 0, -Ad * np.minimum(rho, hi), np.where(Ad < 0, -Ad * np.maximum(rho, lo), 0.0))
    np.testing.assert_allclose(out["loss_sum"], want.mean(), rtol=1e-12, atol=1e-15)
    held = ((Ad > 0) & (rho > hi)) | ((Ad < 0) & (rho < lo))
    np.testing.assert_allclose(out["g"], np.where(held, 0.0, -rho * Ad) / B, rtol=1e-12, atol=1e-15)
    assert held.any() and (~held).any()


def test_grpo_equals_bnpo_with_equal_lengths():
    """Every sequence with the same number of completion tokens n: the
    per-sample mean (1/B) sum_i (1/n) S_i equals the token mean sum S / (B n)."""
    B, T = 6, 8
    comp = _comp(B, T, [2] * B)
    r = _rng(3)
    lp = r.uniform(-6, -0.3, B * T)
    old = (lp + r.normal(0, 0.3, B * T)).astype(np.float32)
    ref = (lp + r.normal(0, 0.2, B * T)).astype(np.float32)
    A = r.standard_normal(B).astype(np.float32)
    outs = [oracle.policy_loss(LossConfig(B=B, T=T, loss_type=lt, eps_low=0.2, eps_high=0.25, beta=0.05),
                               lp, old, ref, comp, None, A) for lt in (GRPO, BNPO)]
    assert outs[0]["loss_sum"] == pytest.approx(outs[1]["loss_sum"], rel=1e-13)
    np.testing.assert_allclose(outs[0]["g"], outs[1]["g"], rtol=1e-13, atol=1e-18)


def test_dapo_global_count_rescales_bnpo():
    """DAPO with a global count G equals BNPO times (batch tokens / G); with no
    count it equals BNPO."""
    B, T = 4, 9
    comp = _comp(B, T, [0, 4, 2, 7])
    r = _rng(4)
    lp = r.uniform(-6, -0.3, B * T)
    old = (lp + r.normal(0, 0.3, B * T)).astype(np.float32)
    A = r.standard_normal(B).astype(np.float32)
    kw = dict(B=B, T=T, eps_low=0.2, eps_high=0.2)
    bn = oracle.policy_loss(LossConfig(loss_type=BNPO, **kw), lp, old, None, comp, None, A)
    da0 = oracle.policy_loss(LossConfig(loss_type=DAPO, **kw), lp, old, None, comp, None, A)
    G = 97
    da = oracle.policy_loss(LossConfig(loss_type=DAPO, global_tokens=G, **kw), lp, old, None, comp, None, A)
    n = int(comp.sum())
    assert da0["loss_sum"] == bn["loss_sum"]
    assert da["loss_sum"] == pytest.approx(bn["loss_sum"] * n / G, rel=1e-14)
    np.testing.assert_allclose(da["g"], bn["g"] * n / G, rtol=1e-14, atol=1e-20)


def test_clip_predicate_at_the_bound():
    """The predicate compares exp(lr32) in fp64 with fp32(1 + eps_high): the
    two fp32 log-ratios around log(hi) fall on either side, and only the one
    above loses its gradient (A > 0)."""
    eh = 0.3
    hi = float(np.float32(1 + eh))
    x = np.float32(math.log(hi))
    below = x if math.exp(float(x)) < hi else np.nextafter(x, np.float32(-1))
    above = np.nextafter(below, np.float32(1))
    assert math.exp(float(below)) < hi < math.exp(float(above))
    B, T = 2, 1
    old = np.zeros(B, np.float32)
    lp = np.array([float(below), float(above)])
    A = np.ones(B, np.float32)
    out = oracle.policy_loss(LossConfig(B=B, T=T, loss_type=GRPO, eps_low=0.2, eps_high=eh),
                             lp, old, None, np.ones(B, np.uint8), None, A)
    assert list(out["clipped_tok"]) == [False, True]
    assert out["g"][0] == pytest.approx(-math.exp(float(below)) / B, rel=1e-15)
    assert out["g"][1] == 0.0


def test_zero_advantage_extreme_ratio_is_finite():
    """A = 0 with a log-ratio that overflows exp: no term, no gradient."""
    B, T = 2, 3
    lp = np.full(B * T, -0.1)
    old = np.full(B * T, -900.0, np.float32)
    A = np.array([0.0, 0.0], np.float32)
    out = oracle.policy_loss(LossConfig(B=B, T=T, loss_type=BNPO), lp, old, None, np.ones(B * T, np.uint8),
                             None, A)
    assert out["loss_sum"] == 0.0
    assert np.all(out["g"] == 0.0)


# ---------------------------------------------------------------------------
# Through the LM head: autograd of a plain torch definition, finite differences
# ---------------------------------------------------------------------------

def _problem(seed, loss_type, beta, bias, q, tau=1.0, B=3, T=7, H=5, V=23, global_tokens=0):
    r = _rng(seed)
    h = r.standard_normal((B * T, H))
    W = r.standard_normal((V, H)) * 0.5
    b = r.standard_normal(V) * 0.3 if bias else None
    y = r.integers(0, V, B * T)
    comp = _comp(B, T, [2, 0, 3][:B])
    fwd = oracle.forward_rows(h, W, b, tau, y)
    old = (fwd["logp"] + r.standard_normal(B * T) * 0.6).astype(np.float32)
    ref = (fwd["logp"] + r.standard_normal(B * T) * 0.2).astype(np.float32) if beta else None
    A = np.array([1.2, -0.8, 0.6], np.float32)[:B]
    cfg = LossConfig(B=B, T=T, loss_type=loss_type, eps_low=0.2, eps_high=0.3, beta=beta, temperature=tau,
                     top_entropy_quantile=q, global_tokens=global_tokens)
    return cfg, h, W, b, y, old, ref, comp, A


def _torch_loss(cfg, h, W, b, y, old, ref, comp, A, emask):
    """The clipped token surrogate written with torch.minimum / torch.clamp;
    autograd supplies the gradient."""
    B, T = cfg.B, cfg.T
    z = h @ W.T
    if b is not None:
        z = z + b
    z = z / cfg.temperature
    lp = torch.log_softmax(z, dim=1).gather(1, torch.as_tensor(y)[:, None])[:, 0].reshape(B, T)
    rho = torch.exp(lp - torch.as_tensor(old.astype(np.float64)).reshape(B, T))
    At = torch.as_tensor(A.astype(np.float64))[:, None]
    lo, hi = float(np.float32(1 - cfg.eps_low)), float(np.float32(1 + cfg.eps_high))
    pol = -torch.minimum(rho * At, torch.clamp(rho, lo, hi) * At)
    M = torch.as_tensor(comp.reshape(B, T) != 0)
    e = torch.ones(B, T, dtype=torch.bool) if emask is None else torch.as_tensor(emask.reshape(B, T))
    ell = torch.where(e, pol, torch.zeros_like(pol))
    if ref is not None:
        x = torch.as_tensor(ref.astype(np.float64)).reshape(B, T) - lp
        ell = ell + cfg.beta * (torch.exp(x) - x - 1)
    ell = torch.where(M, ell, torch.zeros_like(ell))
    if cfg.loss_type == GRPO:
        return (ell.sum(1) / M.sum(1).clamp(min=1)).sum() / B
    G = cfg.global_tokens if (cfg.loss_type == DAPO and cfg.global_tokens > 0) else max(1, int(M.sum()))
    return ell.sum() / G


CASES = [
    (GRPO, 0.0, False, 1.0, 1.0, 0),
    (GRPO, 0.04, True, 0.5, 0.8, 0),
    (BNPO, 0.0, True, 1.0, 1.0, 0),
    (BNPO, 0.04, False, 0.5, 1.2, 0),
    (DAPO, 0.04, True, 1.0, 1.0, 0),
    (DAPO, 0.0, False, 0.5, 1.0, 50),
]


@pytest.mark.parametrize("case", CASES)
def test_autograd_plain_definition(case):
    loss_type, beta, bias, q, tau, G = case
    cfg, h, W, b, y, old, ref, comp, A = _problem(21, loss_type, beta, bias, q, tau, global_tokens=G)
    out = oracle.run(cfg, h, W, b, y, old, ref, comp, None, A)
    assert any(p["clipped_tok"].any() for p in out["parts"])
    ht = torch.tensor(h, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    bt = None if b is None else torch.tensor(b, requires_grad=True)
    L = _torch_loss(cfg, ht, Wt, bt, y, old, ref, comp, A, out["entropy_mask"])
    L.backward()
    assert out["loss"] == pytest.approx(L.item(), rel=1e-12, abs=1e-14)
    np.testing.assert_allclose(out["grad_h"], ht.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(out["grad_W"], Wt.grad.numpy(), rtol=1e-10, atol=1e-13)
    if b is not None:
        np.testing.assert_allclose(out["grad_b"], bt.grad.numpy(), rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("case", CASES[:4])
def test_finite_differences(case):
    """Central differences of the oracle's loss (entropy mask held fixed)
    match its grad_h and grad_W; coordinates whose step flips a clip
    predicate are skipped."""
    loss_type, beta, bias, q, tau, G = case
    cfg, h, W, b, y, old, ref, comp, A = _problem(11, loss_type, beta, bias, q, tau, global_tokens=G)
    out = oracle.run(cfg, h, W, b, y, old, ref, comp, None, A)
    emask = out["entropy_mask"]
    base = out["parts"][0]["clipped_tok"]

    def loss_at():
        fwd = oracle.forward_rows(h, W, b, cfg.temperature, y)
        p = oracle.policy_loss(cfg, fwd["logp"], old, ref, comp, None, A, emask)
        return p["loss_sum"], p["clipped_tok"]

    r = _rng(12)
    delta = 1e-6
    checked = 0
    for arr, grad in ((h, out["grad_h"]), (W, out["grad_W"])):
        for fi in r.choice(arr.size, size=min(arr.size, 25), replace=False):
            idx = np.unravel_index(fi, arr.shape)
            save = arr[idx]
            arr[idx] = save + delta
            lpp, cp = loss_at()
            arr[idx] = save - delta
            lmm, cm = loss_at()
            arr[idx] = save
            if not (np.array_equal(cp, base) and np.array_equal(cm, base)):
                continue
            assert grad[idx] == pytest.approx((lpp - lmm) / (2 * delta), rel=2e-5, abs=1e-9)
            checked += 1
    assert checked >= 30


@pytest.mark.parametrize("loss_type", PPO)
def test_chunk_invariance(loss_type):
    """Outer chunks of 1, 2, 4 and B sequences agree: BNPO and DAPO divide by
    the batch's token count, not the chunk's."""
    r = _rng(41)
    B, T, H, V = 6, 9, 6, 31
    h = r.standard_normal((B * T, H))
    W = r.standard_normal((V, H)) * 0.4
    b = r.standard_normal(V) * 0.1
    y = r.integers(0, V, B * T)
    comp = _comp(B, T, [i % 4 for i in range(B)])
    fwd = oracle.forward_rows(h, W, b, 1.0, y)
    old = (fwd["logp"] + r.standard_normal(B * T) * 0.2).astype(np.float32)
    ref = (fwd["logp"] + r.standard_normal(B * T) * 0.1).astype(np.float32)
    A = r.standard_normal(B).astype(np.float32)
    outs = []
    for cs in (1, 2, 4, B):
        cfg = LossConfig(B=B, T=T, loss_type=loss_type, eps_low=0.2, eps_high=0.25, beta=0.04,
                         top_entropy_quantile=0.6, chunk_sequences=cs)
        outs.append(oracle.run(cfg, h, W, b, y, old, ref, comp, None, A))
    for o in outs[1:]:
        assert o["loss"] == pytest.approx(outs[0]["loss"], abs=1e-12)
        np.testing.assert_allclose(o["metrics"], outs[0]["metrics"], atol=1e-12)
        np.testing.assert_allclose(o["grad_h"], outs[0]["grad_h"], atol=1e-12)
        np.testing.assert_allclose(o["grad_W"], outs[0]["grad_W"], atol=1e-12)


def test_metrics_count_clipped_tokens():
    """The clip metric counts completion tokens whose ratio is held at a
    bound; prompt tokens never count."""
    B, T = 3, 4
    comp = np.array([[0, 1, 1, 1]] * B, np.uint8).reshape(-1)
    lp = np.full(B * T, -1.0)
    old = np.full(B * T, -1.0, np.float32)
    old[0] = -3.0    # prompt token of seq 0: ratio e^2, not counted
    old[1] = -3.0    # seq 0, A > 0, ratio e^2 > hi: clipped
    old[5] = 1.0     # seq 1, A < 0, ratio e^-2 < lo: clipped
    old[9] = 1.0     # seq 2, A > 0, ratio below lo: not held
    A = np.array([1.0, -1.0, 2.0], np.float32)
    out = oracle.policy_loss(LossConfig(B=B, T=T, loss_type=BNPO, eps_low=0.2, eps_high=0.2), lp, old, None,
                             comp, None, A)
    _, m = oracle.finalize_metrics([out], np.float32(np.nan))
    assert m[6] == 9 and m[7] == 2
    assert m[0] == np.float32(2) / np.float32(9)
