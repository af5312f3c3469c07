"""Pins of the CPU oracle to what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
closed form, a library routine (torch.quantile, torch.distributions,
scipy.special.logsumexp), a brute-force definition, finite differences, or
autograd of an independently written formulation.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle.core import LossConfig, GMPO, GSPO_TOKEN

torch.set_default_dtype(torch.float64)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# Forward: log-sum-exp, log-prob, entropy
# ---------------------------------------------------------------------------

def test_uniform_logits_closed_form():
    """W = 0, b = 0: every logit is 0, so lp = -ln V and H = ln V exactly."""
    N, H, V = 7, 16, 333
    h = _rng(0).standard_normal((N, H))
    out = oracle.forward_rows(h, np.zeros((V, H)), np.zeros(V), 1.0, np.arange(N) % V)
    np.testing.assert_allclose(out["logp"], -math.log(V), rtol=0, atol=1e-13)
    np.testing.assert_allclose(out["entropy"], math.log(V), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["lse"], math.log(V), rtol=0, atol=1e-12)


@pytest.mark.parametrize("tau", [1.0, 0.7])
@pytest.mark.parametrize("with_bias", [False, True])
def test_forward_matches_torch_and_scipy(tau, with_bias):
    """lp against torch.log_softmax, lse against scipy logsumexp, H against
    torch.distributions.Categorical(...).entropy() (the routine PR #1558 tests
    its streaming entropy against), all fp64."""
    r = _rng(1)
    N, H, V = 33, 24, 517
    h = r.standard_normal((N, H))
    W = r.standard_normal((V, H)) * 0.3
    b = r.standard_normal(V) * 0.5 if with_bias else None
    y = r.integers(0, V, N)
    out = oracle.forward_rows(h, W, b, tau, y, chunk=8)
    z = torch.from_numpy(h) @ torch.from_numpy(W).T
    if b is not None:
        z = z + torch.from_numpy(b)
    z = z / tau
    lp_t = torch.log_softmax(z, dim=1)[torch.arange(N), torch.from_numpy(y)]
    np.testing.assert_allclose(out["logp"], lp_t.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["lse"], scipy.special.logsumexp(z.numpy(), axis=1), rtol=0, atol=1e-12)
    ent_t = torch.distributions.Categorical(logits=z).entropy()
    np.testing.assert_allclose(out["entropy"], ent_t.numpy(), rtol=0, atol=1e-12)


def test_entropy_near_one_hot():
    """One logit far above the rest: H -> 0 and lp(target=argmax) -> 0."""
    V, H = 100, 4
    W = np.zeros((V, H))
    W[17, 0] = 60.0
    h = np.array([[1.0, 0, 0, 0]])
    out = oracle.forward_rows(h, W, None, 1.0, np.array([17]))
    assert out["entropy"][0] < 1e-20 + 1e-22 * V or out["entropy"][0] < 1e-23
    assert abs(out["logp"][0]) < 1e-24


# ---------------------------------------------------------------------------
# Quantile and the high-entropy mask
# ---------------------------------------------------------------------------

def test_quantile_bit_exact_vs_torch():
    """quantile_linear_f32 equals torch.quantile bit for bit (PR #1558 tests
    its quantile against torch.quantile)."""
    r = _rng(2)
    for it in range(1500):
        n = int(r.integers(1, 3000))
        x = (r.standard_normal(n) * r.uniform(1e-3, 5) + r.uniform(-3, 12)).astype(np.float32)
        if it % 5 == 0:  # heavy ties
            x = np.round(x * 4).astype(np.float32) / np.float32(4)
        q = [0.0, 0.2, 0.5, 0.8, 1.0][it % 5] if it % 2 else float(r.uniform())
        p = 1.0 - q
        want = np.float32(torch.quantile(torch.from_numpy(x), p).item())
        got = oracle.quantile_linear_f32(x, p)
        assert got.view(np.uint32) == want.view(np.uint32), (it, n, p, got, want)


def test_quantile_integral_rank_is_order_statistic():
    """When p (n-1) is an integer k, the quantile is the k-th smallest value:
    brute force by counting (#{x < v} <= k < #{x <= v})."""
    r = _rng(3)
    for n in [1, 2, 5, 11, 101, 1001]:
        x = np.round(r.standard_normal(n) * 3).astype(np.float32)
        for k in {0, n // 3, n // 2, n - 1}:
            p = k / (n - 1) if n > 1 else 0.5
            if np.float32(np.float32(p) * np.float32(n - 1)) != np.float32(k):
                continue
            v = oracle.quantile_linear_f32(x, p)
            assert (x < v).sum() <= k < (x <= v).sum()


def test_mask_invariants():
    """q = 1 keeps exactly the active set; q in {0.2, 0.5, 0.8} drops some but
    not all active tokens (PR #1558, Testing, checks this too, so that a mask
    that keeps everything cannot pass); no active token gives an empty mask;
    q = 0 keeps the top tie
    group; q outside [0, 1] raises."""
    r = _rng(4)
    N = 4000
    H = (11.7 + 0.01 * r.standard_normal(N)).astype(np.float32)
    active = r.uniform(size=N) < 0.8
    m, thr = oracle.entropy_quantile_mask(H, active, 1.0)
    assert np.array_equal(m, active) and np.isnan(thr)
    for q in (0.2, 0.5, 0.8):
        m, thr = oracle.entropy_quantile_mask(H, active, q)
        assert 0 < m.sum() < active.sum()
        assert not np.any(m & ~active)
        # fraction kept is q up to ties and the interpolation step
        assert abs(m.sum() / active.sum() - q) < 2.0 / active.sum() + 1e-3
    m, thr = oracle.entropy_quantile_mask(H, np.zeros(N, bool), 0.2)
    assert m.sum() == 0 and np.isnan(thr)
    m, thr = oracle.entropy_quantile_mask(H, active, 0.0)
    assert thr == H[active].max() and m.sum() == (H[active] == thr).sum()
    with pytest.raises(ValueError):
        oracle.entropy_quantile_mask(H, active, 1.5)


# ---------------------------------------------------------------------------
# Policy loss closed forms
# ---------------------------------------------------------------------------

def _seqs(B, T, prompt, seed=5):
    r = _rng(seed)
    comp = np.zeros((B, T), np.uint8)
    for i in range(B):
        comp[i, prompt[i] if hasattr(prompt, "__len__") else prompt:] = 1
    return comp.reshape(-1), r


def test_gmpo_on_policy_closed_form():
    """old = lp: every log-ratio is 0, r_i = 1, L = -(1/B) sum A_i and
    g_t = -A_i / (B |R_i|) on the ratio tokens (geometric mean of ones)."""
    B, T = 5, 13
    comp, r = _seqs(B, T, [0, 3, 5, 12, 1])
    lp = r.uniform(-8, -0.1, B * T)
    old = lp.astype(np.float32)
    A = np.array([1.3, -0.7, 0.0, 2.0, -1.1], np.float32)
    cfg = LossConfig(B=B, T=T, eps_low=0.2, eps_high=0.3)
    out = oracle.policy_loss(cfg, old.astype(np.float64), old, None, comp, None, A)
    np.testing.assert_allclose(out["seq_ratio"], 1.0, rtol=0, atol=0)
    assert out["loss_sum"] == pytest.approx(-A.astype(np.float64).sum() / B, abs=1e-15)
    n = comp.reshape(B, T).sum(1)
    want = (-A.astype(np.float64) / (B * n))[:, None] * comp.reshape(B, T)
    np.testing.assert_allclose(out["g"], want.reshape(-1), rtol=1e-15, atol=0)


def test_gmpo_geometric_mean_of_ratios():
    """No clip active: r_i equals the geometric mean of the token ratios
    p/q, computed as a direct product (PR #1320 Summary: sequence-level
    geometric mean)."""
    B, T = 3, 9
    comp, r = _seqs(B, T, [2, 0, 4])
    lp = r.uniform(-6, -1, B * T)
    old = (lp + r.uniform(-0.05, 0.05, B * T)).astype(np.float32)
    A = np.array([0.5, -1.0, 2.0], np.float32)
    cfg = LossConfig(B=B, T=T, eps_low=0.4, eps_high=0.4)
    out = oracle.policy_loss(cfg, lp, old, None, comp, None, A)
    assert not out["clipped_tok"].any()
    for i in range(B):
        sel = comp.reshape(B, T)[i] != 0
        ratios = np.exp(lp.reshape(B, T)[i][sel]) / np.exp(old.reshape(B, T)[i][sel].astype(np.float64))
        gm = np.prod(ratios) ** (1.0 / sel.sum())
        assert out["seq_ratio"][i] == pytest.approx(gm, rel=1e-13)


@pytest.mark.parametrize("loss_type", [GMPO, GSPO_TOKEN])
def test_single_token_sequences_are_ppo_clip(loss_type):
    """T = 1: both objectives reduce to the textbook PPO clipped surrogate
    -min(rho A, clip(rho, lo, hi) A) with ratio bounds [e^-eps_l, e^eps_h]
    for GMPO (log-space bounds) and [1-eps_l, 1+eps_h] for GSPO."""
    r = _rng(6)
    B, T = 400, 1
    el, eh = 0.2, 0.3
    lp = r.uniform(-5, -0.5, B)
    old = (lp + r.uniform(-0.8, 0.8, B)).astype(np.float32)
    A = r.standard_normal(B).astype(np.float32)
    A[::7] = 0
    comp = np.ones(B, np.uint8)
    cfg = LossConfig(B=B, T=T, loss_type=loss_type, eps_low=el, eps_high=eh)
    out = oracle.policy_loss(cfg, lp, old, None, comp, None, A)
    rho = np.exp(lp - old.astype(np.float64))
    if loss_type == GMPO:
        lo, hi = math.exp(-float(np.float32(el))), math.exp(float(np.float32(eh)))
    else:
        lo, hi = float(np.float32(1 - el)), float(np.float32(1 + eh))
    Ad = A.astype(np.float64)
    want = -np.minimum(rho * Ad, np.clip(rho, lo, hi) * Ad)
    np.testing.assert_allclose(out["loss_sum"], want.mean(), rtol=1e-12, atol=1e-15)
    # derivative of the surrogate w.r.t. lp: rho A where the unclipped branch is active
    unclipped = ~(((Ad > 0) & (rho > hi)) | ((Ad < 0) & (rho < lo)))
    np.testing.assert_allclose(out["g"], np.where(unclipped, -rho * Ad, 0.0) / B, rtol=1e-12, atol=1e-15)


def test_gmpo_all_clipped_positive_advantage():
    """A > 0 and every log-ratio above eps_high: r = e^eps_high, gradient 0."""
    B, T = 2, 6
    comp = np.ones(B * T, np.uint8)
    lp = np.full(B * T, -1.0)
    old = (lp - 5.0).astype(np.float32)
    A = np.array([1.0, 3.0], np.float32)
    cfg = LossConfig(B=B, T=T, eps_low=0.2, eps_high=0.3)
    out = oracle.policy_loss(cfg, lp, old, None, comp, None, A)
    np.testing.assert_allclose(out["seq_ratio"], math.exp(float(np.float32(0.3))), rtol=1e-15)
    assert np.all(out["g"] == 0.0)
    assert out["counts"][1] == B * T


def test_gmpo_exact_boundary_nextafter():
    """PR #1320, Testing (a log-ratio sitting exactly on a clip bound, and
    its fp32 neighbours): lr32 == fp32(eps) is not clipped (gradient flows);
    the next fp32 value outward is clipped (gradient zero); counts exact."""
    eh, el = 0.3, 0.2
    eh32, el32 = np.float32(eh), np.float32(el)
    old = np.float32(0.0)
    # old = 0 makes fp32(lp32 - old32) == lp32, so the boundary values are hit exactly
    lr_vals = [eh32, np.nextafter(eh32, np.float32(1)), np.nextafter(eh32, np.float32(0)),
               -el32, np.nextafter(-el32, np.float32(-1)), np.nextafter(-el32, np.float32(0))]
    B, T = len(lr_vals), 1
    def solve(v):
        # search the fp32 neighbourhood of v + old for an lp32 with fp32(lp32 - old) == v
        l = np.float32(v + old)
        for _ in range(64):
            d = np.float32(l - old)
            if d == v:
                return l
            l = np.nextafter(l, np.float32(np.inf) if d < v else np.float32(-np.inf))
        raise AssertionError("no exact boundary input")
    lp32 = np.array([solve(v) for v in lr_vals], np.float32)
    for v, l in zip(lr_vals, lp32):
        assert np.float32(l - old) == v
    A = np.array([1, 1, 1, -1, -1, -1], np.float32)
    cfg = LossConfig(B=B, T=T, eps_low=el, eps_high=eh)
    out = oracle.policy_loss(cfg, lp32.astype(np.float64), np.full(B, old, np.float32), None,
                             np.ones(B, np.uint8), None, A)
    assert out["clipped_tok"].tolist() == [False, True, False, False, True, False]
    assert (out["g"] != 0).tolist() == [True, False, True, True, False, True]
    # torch.nextafter agrees with numpy's on these values
    t = torch.nextafter(torch.tensor(eh32), torch.tensor(np.float32(1)))
    assert np.float32(t.item()) == lr_vals[1]


def test_gmpo_zero_advantage_extreme_ratio_finite():
    """A = 0 with extreme log-ratios: loss and gradient finite and zero
    (PR #1320, Testing: very large log-ratios must clip and keep the
    gradients finite)."""
    B, T = 2, 4
    comp = np.ones(B * T, np.uint8)
    lp = np.array([-1.0] * 8)
    old = np.array([-900.0, -1, -1, -1, 800.0, -1, -1, -1], np.float32)
    A = np.array([0.0, 0.0], np.float32)
    out = oracle.policy_loss(LossConfig(B=B, T=T), lp, old, None, comp, None, A)
    assert out["loss_sum"] == 0.0 and np.all(out["g"] == 0.0)
    A = np.array([1.0, -1.0], np.float32)
    out = oracle.policy_loss(LossConfig(B=B, T=T), lp, old, None, comp, None, A)
    assert np.isfinite(out["loss_sum"]) and np.all(np.isfinite(out["g"]))


def test_gspo_on_policy_ratio_is_one():
    B, T = 3, 7
    comp, r = _seqs(B, T, [1, 2, 3])
    lp32 = r.uniform(-5, -1, B * T).astype(np.float32)
    A = np.array([1.0, -2.0, 0.5], np.float32)
    cfg = LossConfig(B=B, T=T, loss_type=GSPO_TOKEN, eps_low=3e-4, eps_high=4e-4)
    out = oracle.policy_loss(cfg, lp32.astype(np.float64), lp32, None, comp, None, A)
    np.testing.assert_array_equal(out["seq_ratio"], 1.0)
    assert out["loss_sum"] == pytest.approx(-A.astype(np.float64).sum() / B, abs=1e-15)


def test_k3_kl_properties():
    """K3: kl >= 0, zero iff ref = lp, ~x^2/2 for small x, d kl/d lp = 1 - e^{ref-lp}."""
    B, T = 1, 200
    r = _rng(7)
    lp = r.uniform(-6, -1, B * T)
    x = np.concatenate([np.zeros(10), r.standard_normal(190) * np.logspace(-4, 0.5, 190)])
    ref = (lp + x).astype(np.float32)
    xd = ref.astype(np.float64) - lp
    comp = np.ones(B * T, np.uint8)
    cfg = LossConfig(B=B, T=T, beta=1.0)
    out = oracle.policy_loss(cfg, lp, lp.astype(np.float32), ref, comp, None, np.zeros(1, np.float32))
    kl_tok = np.exp(xd) - xd - 1
    assert np.all(kl_tok >= 0)
    assert out["mean_kl_sum"] == pytest.approx(kl_tok.mean(), rel=1e-13)
    small = (np.abs(xd) < 1e-3) & (np.abs(xd) > 1e-5)
    np.testing.assert_allclose(kl_tok[small], xd[small] ** 2 / 2, rtol=2e-3, atol=1e-15)
    np.testing.assert_allclose(out["g"], (1 - np.exp(xd)) / T, rtol=1e-12, atol=1e-18)


# ---------------------------------------------------------------------------
# Gradients: finite differences and autograd of the plain definition
# ---------------------------------------------------------------------------

def _tiny_problem(seed, loss_type, beta, bias, q, tau=1.0, B=3, T=7, H=5, V=23):
    r = _rng(seed)
    h = r.standard_normal((B * T, H))
    W = r.standard_normal((V, H)) * 0.5
    b = r.standard_normal(V) * 0.3 if bias else None
    y = r.integers(0, V, B * T)
    comp = np.zeros((B, T), np.uint8)
    for i, p in enumerate([2, 0, 3][:B]):
        comp[i, p:] = 1
    comp = comp.reshape(-1)
    fwd = oracle.forward_rows(h, W, b, tau, y)
    if loss_type == GMPO:
        old = (fwd["logp"] + r.standard_normal(B * T) * 0.3).astype(np.float32)
        eps = (0.2, 0.3)
    else:
        old = (fwd["logp"] + r.standard_normal(B * T) * 0.02).astype(np.float32)
        eps = (0.004, 0.003)
    ref = (fwd["logp"] + r.standard_normal(B * T) * 0.2).astype(np.float32) if beta else None
    A = np.array([1.2, -0.8, 0.6], np.float32)[:B]
    cfg = LossConfig(B=B, T=T, loss_type=loss_type, eps_low=eps[0], eps_high=eps[1], beta=beta,
                     temperature=tau, top_entropy_quantile=q)
    return cfg, h, W, b, y, old, ref, comp, A


def _loss_only(cfg, h, W, b, y, old, ref, comp, A, emask):
    fwd = oracle.forward_rows(h, W, b, cfg.temperature, y)
    p = oracle.policy_loss(cfg, fwd["logp"], old, ref, comp, None, A, emask)
    return p["loss_sum"], p["clipped_tok"], p["clipped_seq"]


CASES = [
    (GMPO, 0.0, False, 1.0, 1.0),
    (GMPO, 0.04, True, 1.0, 0.7),
    (GMPO, 0.0, True, 0.5, 1.0),
    (GSPO_TOKEN, 0.0, False, 1.0, 1.0),
    (GSPO_TOKEN, 0.04, True, 0.5, 1.3),
]


FD_CASES = [c for c in CASES if not (c[0] == GSPO_TOKEN and c[3] < 1.0)] + [
    (GSPO_TOKEN, 0.04, True, 1.0, 1.3)]


@pytest.mark.parametrize("case", FD_CASES)
def test_gradients_finite_differences(case):
    """Central differences of the oracle's loss (fp64, entropy mask held fixed
    as PR #1558's no-grad pre-pass does) match its analytic grad_h, grad_W,
    grad_b. Coordinates whose step flips a clip predicate are skipped.

    GSPO-token's gradient is, by the Tinker page's stop-gradient construction,
    the derivative of the loss only when every loss token carries the policy
    term (no entropy mask); masked GSPO-token is pinned by autograd below."""
    loss_type, beta, bias, q, tau = case
    cfg, h, W, b, y, old, ref, comp, A = _tiny_problem(11, loss_type, beta, bias, q, tau)
    out = oracle.run(cfg, h, W, b, y, old, ref, comp, None, A)
    emask = out["entropy_mask"]
    base_clip = (out["parts"][0]["clipped_tok"], out["parts"][0]["clipped_seq"])
    r = _rng(12)
    delta = 1e-6
    checked = 0

    def fd(arr, idx):
        save = arr[idx]
        arr[idx] = save + delta
        lpp, cp, sp = _loss_only(cfg, h, W, b, y, old, ref, comp, A, emask)
        arr[idx] = save - delta
        lmm, cm, sm = _loss_only(cfg, h, W, b, y, old, ref, comp, A, emask)
        arr[idx] = save
        flips = not (np.array_equal(cp, base_clip[0]) and np.array_equal(cm, base_clip[0])
                     and np.array_equal(sp, base_clip[1]) and np.array_equal(sm, base_clip[1]))
        return (lpp - lmm) / (2 * delta), flips

    for name, arr, grad in [("h", h, out["grad_h"]), ("W", W, out["grad_W"])] + (
            [("b", b, out["grad_b"])] if b is not None else []):
        flat_idx = r.choice(arr.size, size=min(arr.size, 25), replace=False)
        for fi in flat_idx:
            idx = np.unravel_index(fi, arr.shape)
            d, flips = fd(arr, idx)
            if flips:
                continue
            assert grad[idx] == pytest.approx(d, rel=2e-5, abs=1e-9), (name, idx)
            checked += 1
    assert checked >= 30


def _torch_plain_loss(cfg, h, W, b, y, old, ref, comp, A, emask, sequence_level_gspo=False):
    """An independent torch formulation written from the pages' definitions;
    autograd supplies the gradient."""
    B, T = cfg.B, cfg.T
    z = h @ W.T
    if b is not None:
        z = z + b
    z = z / cfg.temperature
    lp = torch.log_softmax(z, dim=1).gather(1, torch.as_tensor(y)[:, None])[:, 0].reshape(B, T)
    old_t = torch.as_tensor(old.astype(np.float64)).reshape(B, T)
    M = torch.as_tensor(comp.reshape(B, T) != 0)
    e = torch.ones(B, T, dtype=torch.bool) if emask is None else torch.as_tensor(emask.reshape(B, T))
    At = torch.as_tensor(A.astype(np.float64))[:, None]
    lr = lp - old_t
    n = M.sum(1).clamp(min=1).to(torch.float64)
    if cfg.loss_type == GMPO:
        lr32 = (lp.detach().float() - torch.as_tensor(old).reshape(B, T))
        eh, el = float(np.float32(cfg.eps_high)), float(np.float32(cfg.eps_low))
        hi_clip = (At > 0) & (lr32 > eh)
        lo_clip = (At < 0) & (lr32 < -el)
        c = torch.where(hi_clip, torch.full_like(lr, eh), torch.where(lo_clip, torch.full_like(lr, -el), lr))
        r = torch.exp((c * M).sum(1) / n)[:, None]
        pol = torch.where(At != 0, -At * r, torch.zeros_like(r)).expand(B, T)
    else:
        lo, hi = float(np.float32(1 - cfg.eps_low)), float(np.float32(1 + cfg.eps_high))
        ls = ((lr * M).sum(1) / n)[:, None]
        if sequence_level_gspo:
            s_t = torch.exp(ls).expand(B, T)
        else:
            s_t = torch.exp(ls.detach() + lp - lp.detach())
        pol = -torch.minimum(s_t * At, torch.clamp(s_t, lo, hi) * At)
    ell = torch.where(e, pol, torch.zeros_like(pol))
    if ref is not None:
        x = torch.as_tensor(ref.astype(np.float64)).reshape(B, T) - lp
        ell = ell + cfg.beta * (torch.exp(x) - x - 1)
    return ((ell * M).sum(1) / n).sum() / B


@pytest.mark.parametrize("case", CASES)
def test_gradients_autograd_plain_definition(case):
    loss_type, beta, bias, q, tau = case
    cfg, h, W, b, y, old, ref, comp, A = _tiny_problem(21, loss_type, beta, bias, q, tau)
    out = oracle.run(cfg, h, W, b, y, old, ref, comp, None, A)
    ht = torch.tensor(h, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    bt = None if b is None else torch.tensor(b, requires_grad=True)
    L = _torch_plain_loss(cfg, ht, Wt, bt, y, old, ref, comp, A, out["entropy_mask"])
    L.backward()
    assert out["loss"] == pytest.approx(L.item(), rel=1e-12, abs=1e-14)
    np.testing.assert_allclose(out["grad_h"], ht.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(out["grad_W"], Wt.grad.numpy(), rtol=1e-10, atol=1e-13)
    if b is not None:
        np.testing.assert_allclose(out["grad_b"], bt.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_gspo_token_gradient_equals_sequence_level_without_mask():
    """With no entropy mask and R = M, GSPO-token's gradient equals
    sequence-level GSPO's (d s / d lp_t = s / |M|): a derived invariant of the
    Tinker GSPO page's stop-gradient construction."""
    cfg, h, W, b, y, old, ref, comp, A = _tiny_problem(31, GSPO_TOKEN, 0.0, True, 1.0)
    out = oracle.run(cfg, h, W, b, y, old, ref, comp, None, A)
    ht = torch.tensor(h, requires_grad=True)
    L = _torch_plain_loss(cfg, ht, torch.tensor(W), torch.tensor(b), y, old, None, comp, A, None,
                          sequence_level_gspo=True)
    L.backward()
    np.testing.assert_allclose(out["grad_h"], ht.grad.numpy(), rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("loss_type,q", [(GMPO, 1.0), (GMPO, 0.5), (GSPO_TOKEN, 0.5)])
def test_chunk_invariance(loss_type, q):
    """Outer chunk sizes 1, 2, 5 and B agree (PR #1320 tests chunk sizes 1, 2,
    5; PR #1558: one quantile for the batch, so one-sequence chunks give the unchunked result)."""
    r = _rng(41)
    B, T, H, V = 6, 9, 6, 31
    h = r.standard_normal((B * T, H))
    W = r.standard_normal((V, H)) * 0.4
    b = r.standard_normal(V) * 0.1
    y = r.integers(0, V, B * T)
    comp = np.zeros((B, T), np.uint8)
    for i in range(B):
        comp[i, i % 4:] = 1
    comp = comp.reshape(-1)
    fwd = oracle.forward_rows(h, W, b, 1.0, y)
    old = (fwd["logp"] + r.standard_normal(B * T) * 0.2).astype(np.float32)
    ref = (fwd["logp"] + r.standard_normal(B * T) * 0.1).astype(np.float32)
    A = r.standard_normal(B).astype(np.float32)
    outs = []
    for cs in (1, 2, 5, B):
        cfg = LossConfig(B=B, T=T, loss_type=loss_type, eps_low=0.2, eps_high=0.25, beta=0.04,
                         top_entropy_quantile=q, chunk_sequences=cs)
        outs.append(oracle.run(cfg, h, W, b, y, old, ref, comp, None, A))
    for o in outs[1:]:
        assert o["loss"] == pytest.approx(outs[0]["loss"], abs=1e-12)
        np.testing.assert_allclose(o["metrics"], outs[0]["metrics"], atol=1e-12)
        np.testing.assert_allclose(o["grad_h"], outs[0]["grad_h"], atol=1e-12)
        np.testing.assert_allclose(o["grad_W"], outs[0]["grad_W"], atol=1e-12)
        np.testing.assert_allclose(o["grad_b"], outs[0]["grad_b"], atol=1e-12)


def test_metrics_counts():
    """Clip fraction is an integer count over the loss tokens divided once in
    fp32; GSPO's sequence clip fraction is two-sided over sequences."""
    B, T = 4, 5
    comp = np.array([[0, 1, 1, 1, 1]] * B, np.uint8).reshape(-1)
    lp = np.full(B * T, -1.0)
    old = np.full(B * T, -1.0, np.float32)
    old[1] = -2.0   # seq 0 token 1: lr = 1 > 0.3 with A>0 -> clipped
    old[0] = -2.0   # prompt token: never counted
    A = np.array([1.0, -1.0, 0.0, 2.0], np.float32)
    out = oracle.policy_loss(LossConfig(B=B, T=T, eps_low=0.2, eps_high=0.3), lp, old, None, comp, None, A)
    loss, m = oracle.finalize_metrics([out], np.float32(np.nan))
    assert m[6] == 16 and m[7] == 1
    assert m[0] == np.float32(1) / np.float32(16)
    cfg = LossConfig(B=B, T=T, loss_type=GSPO_TOKEN, eps_low=0.1, eps_high=0.1)
    old2 = np.full(B * T, -1.0, np.float32)
    old2[5:10] = -1.5   # seq 1: s = e^{0.5} > hi, A<0 -> not clipped but outside range
    old2[15:20] = -1.5  # seq 3: s > hi, A>0 -> clipped
    out = oracle.policy_loss(cfg, lp, old2, None, comp, None, A)
    loss, m = oracle.finalize_metrics([out], np.float32(np.nan))
    assert m[2] == 2 / 4
    assert m[7] == 4
    # mean over sequences of the sequence log-ratio: seqs 1 and 3 have 0.5, others 0
    assert m[1] == pytest.approx(0.25, abs=1e-15)


def test_quantile_past_torch_cap():
    """Past 2^24 entries (torch.quantile's cap; PR #1558 sorts instead):
    n = 2^24 + 4, so fp32(n - 1) rounds up to n. q = 0 must give the maximum
    exactly (the top tie group, not an index past the end); p = 1/2 gives the
    rank fp32(0.5 * fp32(n - 1)) = 2^23 + 2, an integer, so the quantile is
    that order statistic, checked by counting; and the kept fraction at
    q = 0.2 is 0.2 up to the rank's fp32 rounding."""
    n = (1 << 24) + 4
    assert np.float32(n - 1) == np.float32(n)
    r = _rng(31)
    x = (11.75 + 0.01 * r.standard_normal(n)).astype(np.float32)
    active = np.ones(n, bool)
    m, thr = oracle.entropy_quantile_mask(x, active, 0.0)
    assert thr == x.max() and m.sum() == (x == x.max()).sum()
    k = (1 << 23) + 2
    assert np.float32(np.float32(0.5) * np.float32(n - 1)) == np.float32(k)
    v = oracle.quantile_linear_f32(x, 0.5)
    assert (x < v).sum() <= k < (x <= v).sum()
    m, thr = oracle.entropy_quantile_mask(x, active, 0.2)
    assert abs(m.sum() - 0.2 * n) <= 8 + (x == thr).sum()
