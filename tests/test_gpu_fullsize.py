"""GPU parity at the workloads' full sizes (H=896, V=151936), through the C ABI.

cfg 2 (B=1, T=512): against the whole live oracle run.
cfg 3 (B=8, T=2048, GMPO + K3 KL + bias) and cfg 4 (B=2, T=32768,
GSPO-token + batch-global entropy mask q=0.2): every token's log-prob,
entropy and dL/dlogp, the loss and metrics against the oracle fed with the
oracle's stored forward statistics (tests/golden/fwd_cfg{3,4}.npz, written by
tests/golden/make_golden.py from oracle/ only); grad_h on 256 sampled tokens
and grad_W / grad_b on 64 sampled vocabulary rows computed by the oracle
one row at a time over all tokens.

Where the fp32 entropies of the GPU and the oracle straddle the batch-global
threshold (tokens within the entropy tolerance of it), both masks are valid
readings of the same definition: those tokens are excluded from the
per-token comparisons and their largest possible effect widens the loss
tolerance; every other token's mask bit must agree exactly.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import cosine, make_case, rel_l2, require_gpu, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
LP_TOL = 2e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import rl_policy_gradient_amd  # noqa: F401
    yield


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _golden_fwd(cfg):
    path = os.path.join(GOLDEN, f"fwd_cfg{cfg}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (python tests/golden/make_golden.py {cfg})")
    g = np.load(path)
    return {"logp": g["logp"].astype(np.float64), "lse": g["lse"].astype(np.float64),
            "entropy": g["entropy"].astype(np.float64)}


def _grad_ok(a, b, what):
    r, c = rel_l2(a, b), cosine(a, b)
    assert r <= 1e-2 and c >= 0.9999, (what, r, c)
    return r, c


def test_cfg2_full_against_live_oracle():
    spec = synth.CONFIGS[2]
    _say("cfg2 full")
    d = make_case(spec)
    ref = run_oracle(spec, d)
    gpu = run_gpu(spec, d)
    np.testing.assert_allclose(gpu["logp"], ref["logp"], rtol=0, atol=LP_TOL)
    np.testing.assert_allclose(gpu["entropy"], ref["entropy"], rtol=0, atol=LP_TOL)
    assert abs(gpu["loss"][0] - ref["loss"]) <= 1e-4
    m, mo = gpu["metrics"], ref["metrics"]
    assert m[6] == mo[6] and m[7] == mo[7]
    assert np.float32(m[0]).view(np.uint32) == np.float32(mo[0]).view(np.uint32)
    np.testing.assert_allclose(gpu["dlogp"], ref["g"], rtol=0, atol=1e-4 * np.abs(ref["g"]).max())
    _grad_ok(gpu["grad_hidden"], ref["grad_h"], "grad_h")
    _grad_ok(gpu["grad_weight"], ref["grad_W"], "grad_W")


# The other loss types at the B=1 T=512 size (same inputs as cfg 2 but for
# the loss settings), against the whole live oracle run.
FULL2_VARIANTS = {
    "grpo_token_adv": dict(loss_type=synth.GRPO, eps_low=0.2, eps_high=0.28, token_adv=True),
    "bnpo_kl": dict(loss_type=synth.BNPO, eps_low=0.2, eps_high=0.28, beta=0.04, ref_noise_std=0.05),
    "dapo_global": dict(loss_type=synth.DAPO, eps_low=0.2, eps_high=0.28, global_tokens=4096),
    "gspo_token_adv": dict(loss_type=synth.GSPO_TOKEN, eps_low=3e-4, eps_high=4e-4, old_noise_std=1e-4,
                           token_adv=True),
    "gmpo_kl_bias_corrected": dict(beta=0.04, ref_noise_std=0.05, kl_bias_correction=True),
}


@pytest.mark.parametrize("variant", list(FULL2_VARIANTS))
def test_cfg2_size_loss_types(variant):
    from tests.test_gpu_parity import _check_fused
    spec = synth.CONFIGS[2].replace(name=f"{variant}_bf16_b1_t512", **FULL2_VARIANTS[variant])
    _say(f"cfg2-size {variant}")
    d = make_case(spec)
    ref = run_oracle(spec, d)
    gpu = run_gpu(spec, d)
    _check_fused(spec, d, gpu, ref, lp_tol=LP_TOL)


@pytest.mark.parametrize("cfg", [3, 4])
def test_full_size_sampled(cfg):
    spec = synth.CONFIGS[cfg]
    _say(f"cfg{cfg} full size")
    fwd = _golden_fwd(cfg)
    d = make_case(spec, fwd=fwd)
    ref = run_oracle(spec, d, want_grads=False)
    gpu = run_gpu(spec, d)
    N = spec.N
    comp = d["completion_mask"] != 0

    # forward statistics of every token
    np.testing.assert_allclose(gpu["logp"], fwd["logp"], rtol=0, atol=LP_TOL)
    np.testing.assert_allclose(gpu["entropy"], fwd["entropy"], rtol=0, atol=LP_TOL)

    # entropy mask: exact outside the tolerance band around the threshold
    band = np.zeros(N, bool)
    if spec.top_entropy_quantile < 1.0:
        thr, thr_gpu = float(ref["threshold"]), float(gpu["metrics"][4])
        assert abs(thr_gpu - thr) <= LP_TOL
        band = comp & (np.abs(fwd["entropy"].astype(np.float32) - thr) <= LP_TOL)
        em_gpu = gpu["entropy_mask"].astype(bool)
        # the GPU mask follows its own entropies and threshold exactly
        np.testing.assert_array_equal(em_gpu, comp & (gpu["entropy"] >= thr_gpu))
        diff = em_gpu != ref["entropy_mask"]
        assert not np.any(diff & ~band), np.nonzero(diff & ~band)[0][:10]
        print(f"[info] cfg{cfg}: {band.sum()} tokens in the threshold band, {diff.sum()} mask bits differ there",
              flush=True)
        kept = ref["entropy_mask"].sum()
        assert 0 < kept < comp.sum()

    # clip predicates: every active log-ratio sits further from a bound than
    # the GPU's log-prob differs from the oracle's, so no decision can differ
    if spec.loss_type == synth.GMPO:
        lr = fwd["logp"] - d["old"].astype(np.float64)
        m_hi = np.abs(lr - np.float32(spec.eps_high))[comp].min()
        m_lo = np.abs(lr + np.float32(spec.eps_low))[comp].min()
        dlp = float(np.abs(gpu["logp"].astype(np.float64) - fwd["logp"])[comp].max())
        print(f"[info] cfg{cfg}: clip margin {min(m_hi, m_lo):.2e}, max |dlogp| {dlp:.2e}", flush=True)
        assert min(m_hi, m_lo) > 2 * dlp

    # loss and metrics
    w = 1.0 / (spec.B * np.maximum(1, comp.reshape(spec.B, spec.T).sum(1)))
    pol = np.array([abs(p["seq_ratio"] * d["advantages"].astype(np.float64)).max() for p in ref["parts"]])
    band_bound = float((band.reshape(spec.B, spec.T).sum(1) * w).sum() * max(1.0, pol.max()) * 1.01)
    assert abs(gpu["loss"][0] - ref["loss"]) <= 1e-4 + band_bound, (gpu["loss"][0], ref["loss"], band_bound)
    m, mo = gpu["metrics"], ref["metrics"]
    assert m[6] == mo[6] and m[7] == mo[7], (m, mo)
    assert np.float32(m[0]).view(np.uint32) == np.float32(mo[0]).view(np.uint32)
    np.testing.assert_allclose(m[[1, 2, 3]], mo[[1, 2, 3]], rtol=1e-4, atol=1e-6)
    if spec.top_entropy_quantile < 1.0:
        assert abs(m[5] - mo[5]) * mo[6] <= band.sum() + 0.5

    # dL/dlogp of every token outside the band
    ok = ~band
    g_ref = ref["g"]
    np.testing.assert_allclose(gpu["dlogp"][ok], g_ref[ok], rtol=0, atol=1e-4 * np.abs(g_ref).max())

    # grad_h on sampled tokens with a gradient (outside the band)
    rng = np.random.default_rng(1000 + cfg)
    cand = np.nonzero((g_ref != 0) & ok)[0]
    rows = np.sort(rng.choice(cand, size=min(256, len(cand)), replace=False))
    gh_ref = oracle.grad_h_rows(d["h"][rows], d["W"], d["b"], spec.temperature, d["targets"][rows],
                                fwd["lse"][rows], g_ref[rows])
    _grad_ok(gpu["grad_hidden"][rows], gh_ref, "grad_h rows")
    assert np.all(gpu["grad_hidden"][ok & (g_ref == 0)] == 0)

    # grad_W / grad_b on sampled vocabulary rows (half of them targets)
    tg = np.unique(d["targets"][g_ref != 0])
    vrows = np.unique(np.concatenate([rng.choice(tg, 32, replace=False), rng.choice(spec.V, 32, replace=False)]))
    gW_ref, gb_ref = oracle.grad_w_rows(d["h"], d["W"][vrows], None if d["b"] is None else d["b"][vrows],
                                        spec.temperature, d["targets"], fwd["lse"], g_ref, vrows)
    _grad_ok(gpu["grad_weight"][vrows], gW_ref, "grad_W rows")
    if spec.bias:
        _grad_ok(gpu["grad_bias"][vrows], gb_ref, "grad_b rows")
    for k in ("grad_hidden", "grad_weight", "loss", "metrics", "logp", "entropy", "dlogp"):
        if k in gpu and k != "metrics":
            assert np.all(np.isfinite(gpu[k])), k


def test_cfg5_largest_single_gpu_shape():
    """B=128, T=32768 (4.19M tokens), bias, outer chunks of 8 sequences.

    old_logp = fp32(current + noise) with the current log-probs from the GPU's
    own forward (an fp64 oracle pass over 4.19M tokens takes hours), so the
    oracle checks only what does not depend on old_logp: log-prob and entropy
    of 8 sequences x 256 completion tokens, and the direction of their grad_h
    rows, W_y - sum_v p_v W_v. The rest are properties that hold at any size:
    every output finite; grad_W and grad_b sum to zero over the vocabulary
    (sum_v (onehot - p) = 0); dL/dlogp is one constant per sequence on its
    unclipped ratio tokens and zero elsewhere (GMPO, q = 1, beta = 0); outer
    chunks of 8 sequences agree with the whole batch in one chunk."""
    import concurrent.futures as cf

    import rl_policy_gradient_amd as plp
    from tests.gpu_helpers import dev_tensor

    spec = synth.CONFIGS[5]
    B, T, H, V, N = spec.B, spec.T, spec.H, spec.V, spec.N
    _say("cfg5: generating inputs")
    dev = torch.device("cuda:0")
    h = torch.empty(N, H, dtype=torch.bfloat16, device=dev)
    nblk = (N + 4095) // 4096

    def blk(bi):
        return bi, synth.hidden_block(spec, bi)[1]

    with cf.ThreadPoolExecutor(max_workers=16) as ex:
        for bi, raw in ex.map(blk, range(nblk)):
            h[bi * 4096: bi * 4096 + raw.shape[0]] = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(dev)
    W32, Wraw = synth.weight(spec)
    b32, braw = synth.bias(spec)
    y = synth.targets(spec)
    comp = synth.completion_mask(spec)
    adv = synth.advantages(spec)
    Wt, bt_, yt = dev_tensor(Wraw, "bf16"), dev_tensor(braw, "bf16"), dev_tensor(y)
    _say("cfg5: current log-probs on the GPU")
    _, lp_cur = plp.selective_entropy(h, Wt, bt_, yt)
    old = (lp_cur.double() + torch.from_numpy(synth.old_noise(spec)).to(dev)).float()
    kw = dict(B=B, T=T, bias=bt_, old_logp=old, epsilon_low=spec.eps_low, epsilon_high=spec.eps_high,
              diagnostics=True)
    _say("cfg5: fused, chunks of 8 sequences")
    out = plp.fused_lmhead_policy_loss_fwd_bwd(h, Wt, yt, dev_tensor(comp), dev_tensor(adv),
                                               chunk_sequences=spec.chunk_sequences, **kw)
    torch.cuda.synchronize()
    for k, v in out.items():
        if k == "metrics":   # the entropy threshold is NaN by definition when q = 1
            assert bool(torch.isnan(v[4])) and bool(torch.isfinite(v[torch.arange(8, device=dev) != 4]).all())
            continue
        assert bool(torch.isfinite(v.float()).all()), k

    # sums over the vocabulary vanish: sum_v dz[t,v] = g_t (1 - sum_v p[t,v]) / tau = 0
    gW = out["grad_weight"].float()
    colsum = gW.sum(0).abs()
    colabs = gW.abs().sum(0)
    assert float((colsum / colabs.clamp(min=1e-30)).max()) < 2e-2
    gb = out["grad_bias"].float()
    assert float(gb.sum().abs()) < 2e-2 * float(gb.abs().sum())

    # dL/dlogp structure per sequence
    g = out["dlogp"].cpu().numpy().reshape(B, T)
    cm = comp.reshape(B, T) != 0
    assert np.all(g[~cm] == 0)
    for i in range(B):
        nz = g[i][g[i] != 0]
        if adv[i] == 0:
            assert nz.size == 0
        elif nz.size:
            assert np.all(nz == nz[0]) and np.sign(nz[0]) == -np.sign(adv[i])

    # oracle on sampled tokens
    rng = np.random.default_rng(5005)
    seqs = np.sort(rng.choice(B, 8, replace=False))
    rows = np.concatenate([i * T + np.sort(rng.choice(np.nonzero(cm[i])[0], 256, replace=False)) for i in seqs])
    hs, _ = synth.hidden(spec, rows)
    _say("cfg5: oracle on 2048 sampled tokens")
    f = oracle.forward_rows(hs, W32, b32, spec.temperature, y[rows])
    np.testing.assert_allclose(out["logp"][torch.from_numpy(rows).to(dev)].cpu().numpy(), f["logp"], rtol=0,
                               atol=LP_TOL)
    np.testing.assert_allclose(out["entropy"][torch.from_numpy(rows).to(dev)].cpu().numpy(), f["entropy"],
                               rtol=0, atol=LP_TOL)
    vdir = oracle.grad_h_rows(hs, W32, b32, spec.temperature, y[rows], f["lse"], np.ones(len(rows)))
    ghs = out["grad_hidden"][torch.from_numpy(rows).to(dev)].float().cpu().numpy()
    gs = g.reshape(-1)[rows]
    for k in np.nonzero(gs)[0]:
        assert cosine(ghs[k], np.sign(gs[k]) * vdir[k]) >= 0.9999

    # the whole batch in one chunk gives the same result
    _say("cfg5: fused, one chunk")
    del gW
    out1 = plp.fused_lmhead_policy_loss_fwd_bwd(h, Wt, yt, dev_tensor(comp), dev_tensor(adv), chunk_sequences=0,
                                                **kw)
    torch.cuda.synchronize()
    assert abs(float(out1["loss"][0]) - float(out["loss"][0])) <= 1e-5
    assert torch.equal(out1["dlogp"], out["dlogp"]) or float((out1["dlogp"] - out["dlogp"]).abs().max()) < 1e-9
    r = float((out1["grad_weight"].float() - out["grad_weight"].float()).norm() / out["grad_weight"].float().norm())
    assert r < 1e-2, r
