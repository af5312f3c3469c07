"""Pins of the oracle's per-token advantages (the Tinker GSPO page's
"Input tensors": advantages of shape (N,), zero off the completion as its
"Building a datum" example sets them).

Checked against: the per-sequence path when every token repeats its
sequence's advantage, the page's GSPO snippet restated in torch (autograd
gives the gradient) through the LM head, and the token-level clipped
surrogate written with torch.minimum / torch.clamp.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.core import LossConfig, GMPO, GSPO_TOKEN, GRPO, BNPO, DAPO

torch.set_default_dtype(torch.float64)


def _rng(seed):
    return np.random.default_rng(seed)


def _comp(B, T, prompt):
    comp = np.zeros((B, T), np.uint8)
    for i in range(B):
        comp[i, prompt[i]:] = 1
    return comp.reshape(-1)


@pytest.mark.parametrize("loss_type,q", [(GSPO_TOKEN, 1.0), (GSPO_TOKEN, 0.5), (GRPO, 1.0), (BNPO, 0.5),
                                         (DAPO, 1.0)])
def test_repeated_sequence_advantage_matches_per_sequence_path(loss_type, q):
    """A_t = A_i on every token gives the per-sequence result."""
    r = _rng(1)
    B, T, H, V = 4, 9, 6, 29
    h = r.standard_normal((B * T, H))
    W = r.standard_normal((V, H)) * 0.5
    y = r.integers(0, V, B * T)
    comp = _comp(B, T, [0, 2, 5, 1])
    fwd = oracle.forward_rows(h, W, None, 1.0, y)
    noise = 0.02 if loss_type == GSPO_TOKEN else 0.4
    old = (fwd["logp"] + r.standard_normal(B * T) * noise).astype(np.float32)
    ref = (fwd["logp"] + r.standard_normal(B * T) * 0.1).astype(np.float32)
    A = np.array([1.1, -0.6, 0.0, 0.9], np.float32)
    eps = (0.001, 0.001) if loss_type == GSPO_TOKEN else (0.2, 0.25)
    cfg = LossConfig(B=B, T=T, loss_type=loss_type, eps_low=eps[0], eps_high=eps[1], beta=0.04,
                     top_entropy_quantile=q, chunk_sequences=2)
    a = oracle.run(cfg, h, W, None, y, old, ref, comp, None, A)
    b = oracle.run(cfg, h, W, None, y, old, ref, comp, None, None, token_advantages=np.repeat(A, T))
    assert any(p["clipped_tok"].any() for p in a["parts"])
    assert b["loss"] == pytest.approx(a["loss"], rel=1e-13, abs=1e-15)
    np.testing.assert_allclose(b["metrics"], a["metrics"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(b["g"], a["g"], rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(b["grad_W"], a["grad_W"], rtol=1e-11, atol=1e-15)


def test_gmpo_rejects_per_token_advantages():
    cfg = LossConfig(B=1, T=3)
    with pytest.raises(ValueError):
        oracle.policy_loss(cfg, np.zeros(3), np.zeros(3, np.float32), None, np.ones(3, np.uint8), None, None,
                           token_advantages=np.ones(3, np.float32))


def _datum_problem(seed, B=3, T=8, H=5, V=21, noise=0.01):
    r = _rng(seed)
    h = r.standard_normal((B * T, H))
    W = r.standard_normal((V, H)) * 0.5
    b = r.standard_normal(V) * 0.2
    y = r.integers(0, V, B * T)
    comp = _comp(B, T, [2, 0, 3])
    fwd = oracle.forward_rows(h, W, b, 1.0, y)
    old = (fwd["logp"] + r.standard_normal(B * T) * noise).astype(np.float32)
    # per-token advantages of both signs on the completion, zero on the prompt
    At = (r.standard_normal(B * T) * (comp != 0)).astype(np.float32)
    return h, W, b, y, comp, old, At


def test_gspo_snippet_with_per_token_advantages():
    """The Tinker page's GSPO code, restated in torch with advantages (N,) and
    the ratio mask = completion: loss = -sum(min(ratio A, clamp(ratio) A));
    the oracle (TOKEN_SUM reduction) matches it and its autograd gradient
    through the LM head."""
    B, T = 3, 8
    h, W, b, y, comp, old, At = _datum_problem(7, B, T)
    lo, hi = float(np.float32(1 - 0.001)), float(np.float32(1 + 0.001))
    cfg = LossConfig(B=B, T=T, loss_type=GSPO_TOKEN, eps_low=0.001, eps_high=0.001, reduction="token_sum")
    out = oracle.run(cfg, h, W, b, y, old, None, comp, None, None, token_advantages=At)
    assert any(p["clipped_tok"].any() for p in out["parts"])
    ht = torch.tensor(h, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    lp_all = torch.log_softmax(ht @ Wt.T + bt, dim=1).gather(1, torch.as_tensor(y)[:, None])[:, 0]
    total = 0.0
    for i in range(B):
        sl = slice(i * T, (i + 1) * T)
        target_logprobs = lp_all[sl]
        ref_logprobs = torch.as_tensor(old[sl].astype(np.float64))
        advantages = torch.as_tensor(At[sl].astype(np.float64))
        in_ratio = torch.as_tensor(comp[sl] != 0)
        log_ratio = (target_logprobs.detach() - ref_logprobs)[in_ratio].mean()
        ratio = torch.exp(log_ratio + target_logprobs - target_logprobs.detach())
        clipped_ratio = torch.clamp(ratio, lo, hi)
        objective = torch.minimum(ratio * advantages, clipped_ratio * advantages)
        total = total - objective.sum()
    total.backward()
    assert out["loss"] == pytest.approx(total.item(), rel=1e-12, abs=1e-14)
    np.testing.assert_allclose(out["grad_h"], ht.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(out["grad_W"], Wt.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(out["grad_b"], bt.grad.numpy(), rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("loss_type", [GRPO, BNPO])
def test_token_clip_with_per_token_advantages(loss_type):
    """GRPO / BNPO with advantages (N,): the clipped token surrogate with each
    token's own A_t, autograd of a torch.minimum / torch.clamp definition."""
    B, T = 3, 8
    h, W, b, y, comp, old, At = _datum_problem(9, B, T, noise=0.4)
    cfg = LossConfig(B=B, T=T, loss_type=loss_type, eps_low=0.2, eps_high=0.28)
    out = oracle.run(cfg, h, W, b, y, old, None, comp, None, None, token_advantages=At)
    assert any(p["clipped_tok"].any() for p in out["parts"])
    ht = torch.tensor(h, requires_grad=True)
    lp = torch.log_softmax(ht @ torch.tensor(W).T + torch.tensor(b), dim=1).gather(
        1, torch.as_tensor(y)[:, None])[:, 0].reshape(B, T)
    rho = torch.exp(lp - torch.as_tensor(old.astype(np.float64)).reshape(B, T))
    A = torch.as_tensor(At.astype(np.float64)).reshape(B, T)
    lo, hi = float(np.float32(0.8)), float(np.float32(1.28))
    M = torch.as_tensor(comp.reshape(B, T) != 0)
    ell = torch.where(M, -torch.minimum(rho * A, torch.clamp(rho, lo, hi) * A), torch.zeros_like(rho))
    if loss_type == GRPO:
        L = (ell.sum(1) / M.sum(1)).sum() / B
    else:
        L = ell.sum() / M.sum()
    L.backward()
    assert out["loss"] == pytest.approx(L.item(), rel=1e-12, abs=1e-14)
    np.testing.assert_allclose(out["grad_h"], ht.grad.numpy(), rtol=1e-10, atol=1e-13)
