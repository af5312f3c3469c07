"""GPU parity at the workloads' full sizes (H=896, V=151936), through the C ABI.

B=1 T=512 GMPO: against the whole live oracle run; the no-grad
selective_entropy entry point against the oracle's full-vocabulary forward.
B=8 T=2048 (GMPO + K3 KL + bias) and B=2 T=32768 (GSPO-token +
batch-global entropy mask q=0.2): every token's log-prob, entropy and
dL/dlogp, the loss and metrics against the oracle fed with the oracle's
stored forward statistics (tests/golden/fwd_<workload>.npz, written by
tests/golden/make_golden.py from oracle/ only); grad_h on 256 sampled tokens
and grad_W / grad_b on 64 sampled vocabulary rows computed by the oracle
one row at a time over all tokens.

The entropy mask is a decision taken on fp32 entropies about two tokens per
fp32 ulp apart near the threshold at B=2 T=32768, so it is checked in two steps:
the GPU's mask and threshold equal, bit for bit, the oracle's quantile
selection applied to the GPU's own entropy vector (whose values are checked
against the oracle's within the entropy tolerance), and the loss, metrics and
dL/dlogp are then compared with the oracle's loss stage fed that mask. The
number of tokens where the oracle's selection on its own entropies differs
is printed for information.

B=128 T=32768 (4.19M tokens, bias, outer chunks of 8 sequences): the
oracle recomputes the whole loss stage (loss, metrics, every token's
dL/dlogp) from the GPU's exported log-probs, the log-prob, entropy and grad_h
rows of 8 sequences x 256 sampled tokens with the full vocabulary, and 64
grad_W / grad_b rows summed over all 4.19M tokens.
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


def _golden_fwd(name):
    path = os.path.join(GOLDEN, f"fwd_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (python tests/golden/make_golden.py {name})")
    g = np.load(path)
    return {"logp": g["logp"].astype(np.float64), "lse": g["lse"].astype(np.float64),
            "entropy": g["entropy"].astype(np.float64)}


def _grad_ok(a, b, what):
    r, c = rel_l2(a, b), cosine(a, b)
    assert r <= 1e-2 and c >= 0.9999, (what, r, c)
    return r, c


def test_b1_t512_full_against_live_oracle():
    spec = synth.WORKLOADS["gmpo_bf16_b1_t512"]
    _say("B=1 T=512 full")
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

    # the no-grad streaming entropy entry point at the full vocabulary
    import rl_policy_gradient_amd as plp
    from tests.gpu_helpers import dev_tensor
    ent, lp = plp.selective_entropy(dev_tensor(d["h_raw"], "bf16"), dev_tensor(d["W_raw"], "bf16"), None,
                                    dev_tensor(d["targets"]))
    torch.cuda.synchronize()
    np.testing.assert_allclose(ent.cpu().numpy(), d["fwd"]["entropy"], rtol=0, atol=LP_TOL)
    np.testing.assert_allclose(lp.cpu().numpy(), d["fwd"]["logp"], rtol=0, atol=LP_TOL)
    ent2, lp2 = plp.selective_entropy(dev_tensor(d["h_raw"], "bf16"), dev_tensor(d["W_raw"], "bf16"))
    torch.cuda.synchronize()
    assert lp2 is None and torch.equal(ent2, ent)


# The other loss types at the B=1 T=512 size (same inputs as that workload but for
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
def test_b1_t512_loss_types(variant):
    from tests.test_gpu_parity import _check_fused
    spec = synth.WORKLOADS["gmpo_bf16_b1_t512"].replace(name=f"{variant}_bf16_b1_t512", **FULL2_VARIANTS[variant])
    _say(f"B=1 T=512 {variant}")
    d = make_case(spec)
    ref = run_oracle(spec, d)
    gpu = run_gpu(spec, d)
    _check_fused(spec, d, gpu, ref, lp_tol=LP_TOL)


@pytest.mark.parametrize("name", ["gmpo_kl_bf16_b8_t2048", "gspo_token_entropy_bf16_b2_t32768"])
def test_full_size_sampled(name):
    spec = synth.WORKLOADS[name]
    _say(f"{name} full size")
    fwd = _golden_fwd(name)
    d = make_case(spec, fwd=fwd)
    ref = run_oracle(spec, d, want_grads=False)
    gpu = run_gpu(spec, d)
    N = spec.N
    comp = d["completion_mask"] != 0

    # forward statistics of every token
    np.testing.assert_allclose(gpu["logp"], fwd["logp"], rtol=0, atol=LP_TOL)
    np.testing.assert_allclose(gpu["entropy"], fwd["entropy"], rtol=0, atol=LP_TOL)

    # entropy mask: the oracle's selection on the GPU's entropy vector, bit
    # for bit; the loss stage is then the oracle's with that mask
    if spec.top_entropy_quantile < 1.0:
        em_gpu = gpu["entropy_mask"].astype(bool)
        sel_mask, sel_thr = oracle.entropy_quantile_mask(gpu["entropy"], comp, spec.top_entropy_quantile)
        np.testing.assert_array_equal(em_gpu, sel_mask)
        thr_gpu = np.float32(gpu["metrics"][4])
        assert thr_gpu.view(np.uint32) == np.float32(sel_thr).view(np.uint32), (thr_gpu, sel_thr)
        diff = int((em_gpu != ref["entropy_mask"]).sum())
        print(f"[info] {name}: mask bits where the oracle's selection on its own entropies differs: {diff}; "
              f"thresholds gpu {float(thr_gpu)!r} oracle {float(ref['threshold'])!r}", flush=True)
        kept = em_gpu.sum()
        assert 0 < kept < comp.sum()
        cfg_l = oracle.LossConfig.from_spec(spec)
        part = oracle.policy_loss(cfg_l, fwd["logp"], d["old"], d["ref"], d["completion_mask"], None,
                                  d["advantages"], entropy_mask=em_gpu, B_total=spec.B)
        loss_ref, m_ref = oracle.finalize_metrics([part], sel_thr)
        ref = dict(ref, loss=loss_ref, metrics=m_ref, g=part["g"], entropy_mask=em_gpu, parts=[part])

    # clip predicates: every active log-ratio sits further from a bound than
    # the GPU's log-prob differs from the oracle's, so no decision can differ
    if spec.loss_type == synth.GMPO:
        lr = fwd["logp"] - d["old"].astype(np.float64)
        m_hi = np.abs(lr - np.float32(spec.eps_high))[comp].min()
        m_lo = np.abs(lr + np.float32(spec.eps_low))[comp].min()
        dlp = float(np.abs(gpu["logp"].astype(np.float64) - fwd["logp"])[comp].max())
        print(f"[info] {name}: clip margin {min(m_hi, m_lo):.2e}, max |dlogp| {dlp:.2e}", flush=True)
        assert min(m_hi, m_lo) > 2 * dlp

    # loss and metrics
    assert abs(gpu["loss"][0] - ref["loss"]) <= 1e-4, (gpu["loss"][0], ref["loss"])
    m, mo = gpu["metrics"], ref["metrics"]
    assert m[6] == mo[6] and m[7] == mo[7], (m, mo)
    assert np.float32(m[0]).view(np.uint32) == np.float32(mo[0]).view(np.uint32)
    np.testing.assert_allclose(m[[1, 2, 3]], mo[[1, 2, 3]], rtol=1e-4, atol=1e-6)
    if spec.top_entropy_quantile < 1.0:
        assert np.float32(m[5]).view(np.uint32) == np.float32(mo[5]).view(np.uint32), (m[5], mo[5])

    # dL/dlogp of every token
    ok = np.ones(N, bool)
    g_ref = ref["g"]
    np.testing.assert_allclose(gpu["dlogp"], g_ref, rtol=0, atol=1e-4 * np.abs(g_ref).max())

    # grad_h on sampled tokens with a gradient
    rng = np.random.default_rng(1000 + spec.cfg_id)
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


def test_b128_t32768_chunked_largest_single_gpu_shape():
    """B=128, T=32768 (4.19M tokens), bias, outer chunks of 8 sequences.

    old_logp = fp32(current + noise) with the current log-probs from the GPU's
    own forward (an fp64 oracle pass over 4.19M tokens takes hours). Against
    the oracle: the whole loss stage (loss, metrics, dL/dlogp of every token)
    recomputed in fp64 from the GPU's exported log-probs; log-prob, entropy
    and grad_h of 8 sequences x 256 completion tokens with the full
    vocabulary; 64 grad_W / grad_b rows summed over all 4.19M tokens with
    lse_t = z[t, y_t] (oracle) - logp_t (GPU). Every output finite; the
    whole batch in one outer chunk gives the same loss and gradients."""
    import concurrent.futures as cf
    import time

    import rl_policy_gradient_amd as plp
    from tests.gpu_helpers import dev_tensor

    spec = synth.WORKLOADS["gmpo_bf16_b128_t32768_chunked"]
    B, T, H, V, N = spec.B, spec.T, spec.H, spec.V, spec.N
    tau = spec.temperature
    t_start = time.time()
    _say("B=128 T=32768: generating inputs")
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
    _say(f"B=128 T=32768: current log-probs on the GPU ({time.time() - t_start:.0f} s)")
    _, lp_cur = plp.selective_entropy(h, Wt, bt_, yt)
    old = (lp_cur.double() + torch.from_numpy(synth.old_noise(spec)).to(dev)).float()
    del lp_cur
    kw = dict(B=B, T=T, bias=bt_, old_logp=old, epsilon_low=spec.eps_low, epsilon_high=spec.eps_high,
              diagnostics=True)
    _say(f"B=128 T=32768: fused, chunks of 8 sequences ({time.time() - t_start:.0f} s)")
    out = plp.fused_lmhead_policy_loss_fwd_bwd(h, Wt, yt, dev_tensor(comp), dev_tensor(adv),
                                               chunk_sequences=spec.chunk_sequences, **kw)
    torch.cuda.synchronize()
    for k, v in out.items():
        if k == "metrics":   # the entropy threshold is NaN by definition when q = 1
            assert bool(torch.isnan(v[4])) and bool(torch.isfinite(v[torch.arange(8, device=dev) != 4]).all())
            continue
        assert bool(torch.isfinite(v.float()).all()), k

    # ---- the loss stage by the oracle from the GPU's log-probs ------------
    _say(f"B=128 T=32768: oracle loss stage over 4.19M tokens ({time.time() - t_start:.0f} s)")
    lp_gpu = out["logp"].cpu().numpy().astype(np.float64)
    old_np = old.cpu().numpy()
    cfg_l = oracle.LossConfig.from_spec(spec)
    cs = spec.chunk_sequences
    parts, g_ref = [], np.zeros(N)
    for s0 in range(0, B, cs):
        sl = slice(s0 * T, (s0 + cs) * T)
        p = oracle.policy_loss(cfg_l, lp_gpu[sl], old_np[sl], None, comp[sl], None, adv[s0:s0 + cs], B_total=B)
        g_ref[sl] = p["g"]
        parts.append(p)
    loss_ref, m_ref = oracle.finalize_metrics(parts, np.float32(np.nan))
    m = out["metrics"].cpu().numpy()
    assert abs(float(out["loss"][0]) - loss_ref) <= 1e-4, (float(out["loss"][0]), loss_ref)
    assert m[6] == m_ref[6] and m[7] == m_ref[7], (m, m_ref)
    assert np.float32(m[0]).view(np.uint32) == np.float32(m_ref[0]).view(np.uint32)
    np.testing.assert_allclose(m[[1, 2, 3]], m_ref[[1, 2, 3]], rtol=1e-4, atol=1e-6)
    g = out["dlogp"].cpu().numpy()
    np.testing.assert_allclose(g, g_ref, rtol=0, atol=1e-4 * np.abs(g_ref).max())
    assert np.array_equal(g != 0, g_ref != 0)

    # ---- sampled tokens: log-prob, entropy and grad_h by value ------------
    rng = np.random.default_rng(5005)
    cm = comp.reshape(B, T) != 0
    seqs = np.sort(rng.choice(B, 8, replace=False))
    rows = np.concatenate([i * T + np.sort(rng.choice(np.nonzero(cm[i])[0], 256, replace=False)) for i in seqs])
    hs, _ = synth.hidden(spec, rows)
    _say(f"B=128 T=32768: oracle on 2048 sampled tokens ({time.time() - t_start:.0f} s)")
    f = oracle.forward_rows(hs, W32, b32, tau, y[rows])
    rows_t = torch.from_numpy(rows).to(dev)
    np.testing.assert_allclose(out["logp"][rows_t].cpu().numpy(), f["logp"], rtol=0, atol=LP_TOL)
    np.testing.assert_allclose(out["entropy"][rows_t].cpu().numpy(), f["entropy"], rtol=0, atol=LP_TOL)
    gh_ref = oracle.grad_h_rows(hs, W32, b32, tau, y[rows], f["lse"], g_ref[rows])
    _grad_ok(out["grad_hidden"][rows_t].float().cpu().numpy(), gh_ref, "grad_h rows")

    # ---- 64 grad_W / grad_b rows summed over every token ------------------
    _say(f"B=128 T=32768: oracle grad_W rows over 4.19M tokens ({time.time() - t_start:.0f} s)")
    tg = np.unique(y[g_ref != 0])
    vrows = np.unique(np.concatenate([rng.choice(tg, 32, replace=False), rng.choice(V, 32, replace=False)]))
    gW_ref = np.zeros((len(vrows), H))
    gb_ref = np.zeros(len(vrows))
    step = 65536
    for r0 in range(0, N, step):
        r1 = min(N, r0 + step)
        if not np.any(g_ref[r0:r1]):
            continue
        hc = h[r0:r1].float().cpu().numpy().astype(np.float64)
        yc = y[r0:r1]
        zy = (np.einsum("ij,ij->i", hc, W32[yc].astype(np.float64)) + b32[yc].astype(np.float64)) / tau
        lse = zy - lp_gpu[r0:r1]
        a_, b_ = oracle.grad_w_rows(hc, W32[vrows], b32[vrows], tau, yc, lse, g_ref[r0:r1], vrows)
        gW_ref += a_
        gb_ref += b_
        if (r0 // step) % 16 == 15:
            _say(f"B=128 T=32768: grad_W rows, {r1} tokens done ({time.time() - t_start:.0f} s)")
    _grad_ok(out["grad_weight"][torch.from_numpy(vrows).to(dev)].float().cpu().numpy(), gW_ref, "grad_W rows")
    _grad_ok(out["grad_bias"][torch.from_numpy(vrows).to(dev)].float().cpu().numpy(), gb_ref, "grad_b rows")

    # ---- the whole batch in one outer chunk gives the same result ---------
    _say(f"B=128 T=32768: fused, one chunk ({time.time() - t_start:.0f} s)")
    out1 = plp.fused_lmhead_policy_loss_fwd_bwd(h, Wt, yt, dev_tensor(comp), dev_tensor(adv), chunk_sequences=0,
                                                **kw)
    torch.cuda.synchronize()
    assert abs(float(out1["loss"][0]) - float(out["loss"][0])) <= 1e-5
    assert float((out1["dlogp"] - out["dlogp"]).abs().max()) < 1e-9
    r = float((out1["grad_weight"].float() - out["grad_weight"].float()).norm() / out["grad_weight"].float().norm())
    assert r < 1e-2, r
    _say(f"B=128 T=32768: done ({time.time() - t_start:.0f} s)")
