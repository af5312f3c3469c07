"""GPU parity of the loss stage and the entropy quantile mask (no LM head):
the HIP path (through the C ABI) against the CPU oracle, bit-exact where the
result is an integer or a decision."""
import sys

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import dev_tensor, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import rl_policy_gradient_amd  # noqa: F401  (fails loudly when the library is missing)
    yield


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------------------
# entropy_quantile_mask: bit-exact against the oracle's quantile
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,q,kind", [
    (1, 0.2, "normal"), (2, 0.5, "normal"), (1000, 0.2, "normal"), (4099, 0.8, "ties"),
    (65536, 0.2, "narrow"), (300001, 0.5, "normal"), (5000, 0.0, "ties"), (5000, 1.0, "normal"),
    (777, 0.37, "empty"), (3000, 0.2, "negative"),
    # probabilities whose rank has a fraction that an fp32 multiply-add
    # (instead of a rounded product) would change
    (5003, 0.37, "normal"), (12345, 0.73, "negative"), (999, 0.91, "normal"),
    # past torch.quantile's 2^24-entry cap (PR #1558 falls back to a sort):
    # fp32(n - 1) rounds up to n, so the ranks are clamped
    ((1 << 24) + 4, 0.0, "narrow_all"), ((1 << 24) + 4, 0.2, "narrow_all"),
    ((1 << 24) + 20000, 0.2, "narrow_dense"),
])
def test_entropy_quantile_mask(N, q, kind):
    import rl_policy_gradient_amd as plp
    _say(f"quantile N={N} q={q} {kind}")
    r = np.random.default_rng(N + int(q * 100))
    if kind == "ties":
        H = (np.round(r.standard_normal(N) * 3) / 4 + 10).astype(np.float32)
    elif kind.startswith("narrow"):
        H = (11.75 + 0.01 * r.standard_normal(N)).astype(np.float32)
    elif kind == "negative":
        H = (r.standard_normal(N) * 1e-6).astype(np.float32)
    else:
        H = (r.standard_normal(N) * 2 + 8).astype(np.float32)
    if kind == "empty":
        active = np.zeros(N, bool)
    elif kind == "narrow_all":
        active = np.ones(N, bool)
    elif kind == "narrow_dense":
        active = r.uniform(size=N) < 0.9995
        assert active.sum() > (1 << 24)
    else:
        active = r.uniform(size=N) < 0.85
    want_mask, want_thr = oracle.entropy_quantile_mask(H, active, q)
    mask, thr = plp.entropy_quantile_mask(dev_tensor(H), dev_tensor(active.astype(np.uint8)), q)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(mask.cpu().numpy().astype(bool), want_mask)
    t = thr.cpu().numpy()[0]
    if np.isnan(want_thr):
        assert np.isnan(t)
    else:
        assert np.float32(t).view(np.uint32) == np.float32(want_thr).view(np.uint32), (t, want_thr)


# ---------------------------------------------------------------------------
# policy_loss_from_logprobs: the loss stage alone
# ---------------------------------------------------------------------------

def _loss_case(seed, B, T, loss_type, beta, q, ratio_mask, reduction, eps=(0.2, 0.3), noise=0.3):
    r = np.random.default_rng(seed)
    lp = r.uniform(-8, -0.05, B * T).astype(np.float32)
    old = (lp + r.standard_normal(B * T) * noise).astype(np.float32)
    ref = (lp + r.standard_normal(B * T) * 0.1).astype(np.float32) if beta else None
    comp = (r.uniform(size=B * T) < 0.8).astype(np.uint8)
    rm = (comp & (r.uniform(size=B * T) < 0.9)).astype(np.uint8) if ratio_mask else None
    A = r.standard_normal(B).astype(np.float32)
    A[::3] = 0
    ent = (r.standard_normal(B * T) + 5).astype(np.float32) if q < 1 else None
    cfg = oracle.LossConfig(B=B, T=T, loss_type=loss_type, eps_low=eps[0], eps_high=eps[1], beta=beta,
                            top_entropy_quantile=q, reduction=reduction)
    return cfg, lp, old, ref, comp, rm, A, ent


@pytest.mark.parametrize("loss_type,beta,q,ratio_mask,reduction,T", [
    ("gmpo", 0.0, 1.0, False, "seq_mean", 37),
    ("gmpo", 0.04, 0.4, True, "seq_mean", 5000),
    ("gmpo", 0.0, 1.0, False, "token_sum", 3000),
    ("gspo_token", 0.0, 1.0, False, "seq_mean", 64),
    ("gspo_token", 0.04, 0.5, True, "token_sum", 4500),
    ("grpo", 0.0, 1.0, False, "seq_mean", 41),
    ("grpo", 0.04, 0.4, True, "seq_mean", 5000),
    ("bnpo", 0.04, 1.0, False, "seq_mean", 3000),
    ("bnpo", 0.0, 0.5, False, "seq_mean", 77),
    ("dapo", 0.04, 0.5, False, "seq_mean", 4100),
    ("dapo_global", 0.0, 1.0, True, "seq_mean", 300),
])
def test_policy_loss_from_logprobs(loss_type, beta, q, ratio_mask, reduction, T):
    _loss_stage_case(loss_type, beta, q, ratio_mask, reduction, T)


@pytest.mark.parametrize("loss_type,q,on_policy,T", [
    ("gmpo", 1.0, False, 3000),
    ("gmpo", 0.4, True, 77),
    ("gspo_token", 0.5, False, 4500),
    ("grpo", 1.0, False, 41),
    ("grpo", 0.4, True, 5000),
    ("dapo", 0.5, False, 300),
])
def test_policy_loss_kl_bias_correction(loss_type, q, on_policy, T):
    """Bias-corrected KL (the K3 term weighted by the token importance
    ratio, differentiated through) against the oracle, off and on policy."""
    _loss_stage_case(loss_type, 0.1, q, False, "seq_mean", T, kl_bc=True, on_policy=on_policy)


def _loss_stage_case(loss_type, beta, q, ratio_mask, reduction, T, kl_bc=False, on_policy=False):
    import rl_policy_gradient_amd as plp
    B = 7
    G = 0
    if loss_type == "dapo_global":
        loss_type, G = "dapo", 12345
    eps = (0.2, 0.3) if loss_type in ("gmpo", "grpo", "bnpo", "dapo") else (3e-2, 4e-2)
    noise = 0.3 if loss_type in ("gmpo", "grpo", "bnpo", "dapo") else 0.1
    cfg, lp, old, ref, comp, rm, A, ent = _loss_case(T, B, T, loss_type, beta, q, ratio_mask, reduction, eps, noise)
    cfg = cfg.__class__(**{**cfg.__dict__, "global_tokens": G, "kl_bias_correction": kl_bc})
    if on_policy:
        old = None
    _say(f"loss stage {loss_type} beta={beta} q={q} ratio_mask={ratio_mask} {reduction} T={T} G={G} "
         f"kl_bc={kl_bc} on_policy={on_policy}")
    emask, thr = (oracle.entropy_quantile_mask(ent, comp != 0, q) if q < 1 else (None, np.float32(np.nan)))
    p = oracle.policy_loss(cfg, lp.astype(np.float64), old, ref, comp, rm, A, emask)
    loss, metrics = oracle.finalize_metrics([p], thr)
    out = plp.policy_loss_from_logprobs(dev_tensor(lp), dev_tensor(comp), dev_tensor(A), B, T,
                                        old_logp=dev_tensor(old), ref_logp=dev_tensor(ref),
                                        ratio_mask=dev_tensor(rm), entropy=dev_tensor(ent), loss_type=loss_type,
                                        reduction=reduction, epsilon_low=eps[0], epsilon_high=eps[1], beta=beta,
                                        top_entropy_quantile=q, global_tokens=G, kl_bias_correction=kl_bc)
    torch.cuda.synchronize()
    gl = out["loss"].cpu().numpy()[0]
    assert abs(gl - loss) <= 1e-5 * max(1.0, abs(loss)), (gl, loss)
    m = out["metrics"].cpu().numpy()
    assert m[6] == metrics[6] and m[7] == metrics[7]
    assert np.float32(m[0]).view(np.uint32) == np.float32(metrics[0]).view(np.uint32)
    np.testing.assert_allclose(m[[1, 2, 3, 5]], metrics[[1, 2, 3, 5]], rtol=1e-5, atol=1e-7)
    g = out["dlogp"].cpu().numpy()
    np.testing.assert_allclose(g, p["g"], rtol=1e-5, atol=1e-7 * np.abs(p["g"]).max())
    if emask is not None:
        np.testing.assert_array_equal(out["entropy_mask"].cpu().numpy().astype(bool), emask)


def test_policy_loss_exact_boundaries():
    """PR #1320: exact clip boundaries and their nextafter neighbours give the
    oracle's predicates bit for bit (clip count, clip fraction, which
    gradients are zero)."""
    import rl_policy_gradient_amd as plp
    _say("nextafter boundaries")
    eh32, el32 = np.float32(0.3), np.float32(0.2)
    vals = [eh32, np.nextafter(eh32, np.float32(1)), np.nextafter(eh32, np.float32(0)),
            -el32, np.nextafter(-el32, np.float32(-1)), np.nextafter(-el32, np.float32(0))]
    B, T = 6, 3
    lp = np.zeros(B * T, np.float32)
    old = np.zeros(B * T, np.float32)
    for i, v in enumerate(vals):
        lp[i * T:(i + 1) * T] = v          # old = 0 makes fp32(lp - old) exactly v
    A = np.array([1, 1, 1, -1, -1, -1], np.float32)
    comp = np.ones(B * T, np.uint8)
    cfg = oracle.LossConfig(B=B, T=T, eps_low=0.2, eps_high=0.3)
    p = oracle.policy_loss(cfg, lp.astype(np.float64), old, None, comp, None, A)
    loss, metrics = oracle.finalize_metrics([p], np.float32(np.nan))
    out = plp.policy_loss_from_logprobs(dev_tensor(lp), dev_tensor(comp), dev_tensor(A), B, T,
                                        old_logp=dev_tensor(old), epsilon_low=0.2, epsilon_high=0.3)
    torch.cuda.synchronize()
    m = out["metrics"].cpu().numpy()
    assert m[7] == metrics[7] == 6
    assert np.float32(m[0]).view(np.uint32) == np.float32(metrics[0]).view(np.uint32)
    g = out["dlogp"].cpu().numpy()
    np.testing.assert_array_equal(g != 0, p["g"] != 0)
    assert abs(out["loss"].cpu().numpy()[0] - loss) <= 1e-6


def test_token_clip_exact_boundaries():
    """GRPO: fp32 log-ratios on either side of log(fp32(1 + eps_high)) and
    log(fp32(1 - eps_low)) give the oracle's predicates bit for bit."""
    import math
    import rl_policy_gradient_amd as plp
    _say("token-clip boundaries")
    hi, lo = float(np.float32(1.3)), float(np.float32(0.8))

    def around(bound):
        x = np.float32(math.log(bound))
        below = x if math.exp(float(x)) < bound else np.nextafter(x, np.float32(-10))
        return [below, np.nextafter(below, np.float32(10))]

    vals = around(hi) + around(lo)
    B, T = 4, 3
    lp = np.zeros(B * T, np.float32)
    for i, v in enumerate(vals):
        lp[i * T:(i + 1) * T] = v
    old = np.zeros(B * T, np.float32)
    A = np.array([1, 1, -1, -1], np.float32)
    comp = np.ones(B * T, np.uint8)
    cfg = oracle.LossConfig(B=B, T=T, loss_type="grpo", eps_low=0.2, eps_high=0.3)
    p = oracle.policy_loss(cfg, lp.astype(np.float64), old, None, comp, None, A)
    loss, metrics = oracle.finalize_metrics([p], np.float32(np.nan))
    assert metrics[7] == 6  # above hi with A > 0 (3 tokens), below lo with A < 0 (3 tokens)
    out = plp.policy_loss_from_logprobs(dev_tensor(lp), dev_tensor(comp), dev_tensor(A), B, T,
                                        old_logp=dev_tensor(old), loss_type="grpo", epsilon_low=0.2,
                                        epsilon_high=0.3)
    torch.cuda.synchronize()
    m = out["metrics"].cpu().numpy()
    assert m[7] == metrics[7]
    g = out["dlogp"].cpu().numpy()
    np.testing.assert_array_equal(g != 0, p["g"] != 0)
    assert abs(out["loss"].cpu().numpy()[0] - loss) <= 1e-6


@pytest.mark.parametrize("loss_type,reduction,q,T", [
    ("gspo_token", "token_sum", 1.0, 50),
    ("gspo_token", "seq_mean", 0.5, 4500),
    ("grpo", "seq_mean", 1.0, 3000),
    ("dapo", "seq_mean", 0.5, 90),
])
def test_policy_loss_token_advantages(loss_type, reduction, q, T):
    """Per-token advantages (N,), both signs on the completion, zero
    elsewhere: loss, metrics and dL/dlogp against the oracle."""
    import rl_policy_gradient_amd as plp
    B = 6
    gspo = loss_type == "gspo_token"
    eps = (2e-4, 2e-4) if gspo else (0.2, 0.3)
    cfg, lp, old, ref, comp, rm, A, ent = _loss_case(T + 7, B, T, loss_type, 0.04, q, False, reduction, eps,
                                                     0.01 if gspo else 0.3)
    r = np.random.default_rng(T)
    At = (r.standard_normal(B * T) * (comp != 0)).astype(np.float32)
    _say(f"token advantages {loss_type} {reduction} q={q} T={T}")
    emask, thr = (oracle.entropy_quantile_mask(ent, comp != 0, q) if q < 1 else (None, np.float32(np.nan)))
    p = oracle.policy_loss(cfg, lp.astype(np.float64), old, ref, comp, None, None, emask, token_advantages=At)
    assert p["clipped_tok"].any()
    loss, metrics = oracle.finalize_metrics([p], thr)
    out = plp.policy_loss_from_logprobs(dev_tensor(lp), dev_tensor(comp), None, B, T, old_logp=dev_tensor(old),
                                        ref_logp=dev_tensor(ref), entropy=dev_tensor(ent), loss_type=loss_type,
                                        reduction=reduction, epsilon_low=eps[0], epsilon_high=eps[1], beta=0.04,
                                        top_entropy_quantile=q, token_advantages=dev_tensor(At))
    torch.cuda.synchronize()
    gl = out["loss"].cpu().numpy()[0]
    assert abs(gl - loss) <= 1e-5 * max(1.0, abs(loss)), (gl, loss)
    m = out["metrics"].cpu().numpy()
    assert m[6] == metrics[6] and m[7] == metrics[7], (m, metrics)
    assert np.float32(m[0]).view(np.uint32) == np.float32(metrics[0]).view(np.uint32)
    np.testing.assert_allclose(m[[1, 2, 3, 5]], metrics[[1, 2, 3, 5]], rtol=1e-5, atol=1e-7)
    g = out["dlogp"].cpu().numpy()
    np.testing.assert_allclose(g, p["g"], rtol=1e-5, atol=1e-7 * np.abs(p["g"]).max())
