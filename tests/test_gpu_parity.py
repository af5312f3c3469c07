"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, element by element.

Bars (fp32 | bf16): loss rel 1e-5 | abs 1e-4; gradients rel-L2 1e-4 | 1e-2
with cosine >= 0.9999 for bf16; log-prob and entropy abs 1e-5 | 2e-5; clip
metric, counts and entropy mask bit-exact.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import (clip_margin, cosine, dev_tensor, grad_tol, make_case, rel_l2, require_gpu,
                               run_gpu, run_oracle)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import rl_policy_gradient_amd  # noqa: F401  (fails loudly when the library is missing)
    yield


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _check_fused(spec, d, gpu, ref, lp_tol=None):
    lp_tol = lp_tol or (1e-5 if spec.dtype == "f32" else 2e-5)
    np.testing.assert_allclose(gpu["logp"], ref["logp"], rtol=0, atol=lp_tol)
    np.testing.assert_allclose(gpu["entropy"], ref["entropy"], rtol=0, atol=lp_tol)
    # a clip predicate can only differ where a log-ratio sits closer to its
    # bound than the two paths' log-probs differ
    margin = clip_margin(spec, d, ref["logp"])
    dlp = float(np.abs(gpu["logp"].astype(np.float64) - ref["logp"]).max())
    assert margin > 2 * dlp + 1e-6, f"a clip predicate sits {margin:.2e} from its bound (|dlp| {dlp:.1e})"
    if spec.dtype == "f32":
        assert abs(gpu["loss"][0] - ref["loss"]) <= 1e-5 * max(1.0, abs(ref["loss"])), (gpu["loss"][0], ref["loss"])
    else:
        assert abs(gpu["loss"][0] - ref["loss"]) <= 1e-4, (gpu["loss"][0], ref["loss"])
    m, mo = gpu["metrics"], ref["metrics"]
    assert m[6] == mo[6] and m[7] == mo[7], (m, mo)                      # counts exact
    assert np.float32(m[0]).view(np.uint32) == np.float32(mo[0]).view(np.uint32)  # clip fraction bit-exact
    np.testing.assert_allclose(m[[1, 2, 3, 5]], mo[[1, 2, 3, 5]], rtol=1e-4, atol=1e-6)
    if np.isnan(mo[4]):
        assert np.isnan(m[4])
    else:
        assert abs(m[4] - mo[4]) <= lp_tol
    if ref["entropy_mask"] is not None:
        np.testing.assert_array_equal(gpu["entropy_mask"].astype(bool), ref["entropy_mask"])
    g_scale = max(1e-30, np.abs(ref["g"]).max())
    np.testing.assert_allclose(gpu["dlogp"], ref["g"], rtol=0, atol=1e-4 * g_scale + 1e-12)
    tol_l2, tol_cos = grad_tol(spec)
    for k_gpu, k_ref in (("grad_hidden", "grad_h"), ("grad_weight", "grad_W"), ("grad_bias", "grad_b")):
        if k_gpu not in gpu:
            continue
        a, b = gpu[k_gpu], ref[k_ref]
        if not np.any(b):
            # an exactly zero gradient (V = 1: p = onehot): the GPU's may only
            # differ by rounding of the recomputed logits
            assert np.abs(a).max() <= 1e-5, (k_gpu, float(np.abs(a).max()))
            continue
        r, c = rel_l2(a, b), cosine(a, b)
        assert r <= tol_l2 and c >= tol_cos, (k_gpu, r, c)


# ---------------------------------------------------------------------------
# The fused path on small shapes that span several tiles with ragged tails
# ---------------------------------------------------------------------------

SMALL = {
    # bf16 MFMA path: N = 200 (64-row tiles + 8), V = 1000 (32-wide tiles + 8)
    "mfma_gmpo": synth.small("mfma_gmpo", B=2, T=100, H=256, V=1000, eps_low=0.2, eps_high=0.3),
    "mfma_gmpo_kl_bias_tau": synth.small("mfma_gmpo_kl", cfg_id=101, B=3, T=70, H=128, V=777, bias=True,
                                         beta=0.04, ref_noise_std=0.05, temperature=0.8, eps_low=0.2,
                                         eps_high=0.3),
    "mfma_gspo_q": synth.small("mfma_gspo_q", cfg_id=102, B=2, T=96, H=256, V=1500, loss_type=synth.GSPO_TOKEN,
                               eps_low=3e-3, eps_high=4e-3, old_noise_std=1e-2, top_entropy_quantile=0.5),
    "mfma_gmpo_q_chunked": synth.small("mfma_gmpo_q_ch", cfg_id=103, B=5, T=40, H=384, V=900, bias=True,
                                       top_entropy_quantile=0.5, chunk_sequences=2, beta=0.04,
                                       ref_noise_std=0.05),
    "mfma_gmpo_h896": synth.small("mfma_h896", cfg_id=104, B=1, T=130, H=896, V=2053, w_std=0.02),
    "mfma_zero_adv_token_sum": synth.small("mfma_tsum", cfg_id=105, B=4, T=33, H=128, V=600,
                                           zero_adv_fraction=0.5, reduction="token_sum"),
    # token-level clipped losses (GRPO / BNPO / DAPO)
    "mfma_grpo_kl_bias": synth.small("mfma_grpo", cfg_id=111, B=3, T=70, H=256, V=1100, bias=True,
                                     loss_type=synth.GRPO, eps_low=0.1, eps_high=0.12, beta=0.04,
                                     ref_noise_std=0.05),
    "mfma_bnpo_q_chunked": synth.small("mfma_bnpo", cfg_id=112, B=5, T=48, H=384, V=900,
                                       loss_type=synth.BNPO, eps_low=0.1, eps_high=0.1,
                                       top_entropy_quantile=0.5, chunk_sequences=2),
    "mfma_dapo_global_h896": synth.small("mfma_dapo", cfg_id=113, B=2, T=80, H=896, V=1500, w_std=0.02,
                                         loss_type=synth.DAPO, eps_low=0.1, eps_high=0.1, global_tokens=1000),
    "generic_f32_dapo": synth.small("generic_dapo", cfg_id=114, dtype="f32", B=3, T=30, H=48, V=300,
                                    loss_type=synth.DAPO, eps_low=0.1, eps_high=0.12, chunk_sequences=2,
                                    top_entropy_quantile=0.3, beta=0.04, ref_noise_std=0.05),
    # bias-corrected KL: K3 weighted by the token importance ratio
    "mfma_gmpo_kl_bias_corrected": synth.small("mfma_gmpo_klbc", cfg_id=117, B=3, T=70, H=256, V=1000, bias=True,
                                               beta=0.1, ref_noise_std=0.2, old_noise_std=0.3, eps_low=0.2,
                                               eps_high=0.3, kl_bias_correction=True),
    "mfma_grpo_kl_bias_corrected_q": synth.small("mfma_grpo_klbc", cfg_id=118, B=4, T=48, H=384, V=900,
                                                 loss_type=synth.GRPO, eps_low=0.2, eps_high=0.28, beta=0.1,
                                                 ref_noise_std=0.2, old_noise_std=0.3, top_entropy_quantile=0.5,
                                                 chunk_sequences=3, kl_bias_correction=True),
    "generic_f32_gspo_kl_bias_corrected": synth.small("generic_gspo_klbc", cfg_id=119, dtype="f32", B=3, T=30,
                                                      H=48, V=300, loss_type=synth.GSPO_TOKEN, eps_low=0.01,
                                                      eps_high=0.01, old_noise_std=0.01, beta=0.1,
                                                      ref_noise_std=0.2, kl_bias_correction=True),
    # per-token advantages (N,), zero off the completion
    "mfma_gspo_token_adv_sum": synth.small("mfma_gspo_tadv", cfg_id=115, B=3, T=64, H=256, V=1200,
                                           loss_type=synth.GSPO_TOKEN, eps_low=2e-3, eps_high=2e-3,
                                           old_noise_std=1e-2, token_adv=True, reduction="token_sum",
                                           top_entropy_quantile=0.5),
    "generic_f32_grpo_token_adv": synth.small("generic_grpo_tadv", cfg_id=116, dtype="f32", B=3, T=30, H=48,
                                              V=300, loss_type=synth.GRPO, eps_low=0.1, eps_high=0.1,
                                              token_adv=True, chunk_sequences=2, beta=0.04, ref_noise_std=0.05),
    # more compacted tokens than one weight-gradient launch takes (74880 at
    # H=896): several launches accumulate grad_W in fp32, with and without
    # outer chunks
    "mfma_gmpo_wgrad_launches": synth.small("mfma_wg_split", cfg_id=120, B=3, T=32768, H=896, V=1000, w_std=0.02,
                                            bias=True, prompt_lo=100, prompt_hi=4000),
    "mfma_gmpo_wgrad_launches_chunked": synth.small("mfma_wg_split_ch", cfg_id=121, B=3, T=32768, H=896, V=1000,
                                                    w_std=0.02, prompt_lo=100, prompt_hi=4000,
                                                    chunk_sequences=2),
    # every hidden size the matrix-core sweeps are built for (128 ... 896 in
    # steps of 128), and tiny vocabularies: one ragged tile, and V = 1 (every
    # log-prob 0, every entropy 0, all entropies tied at the threshold)
    "mfma_h512_v40_bias": synth.small("mfma_h512", cfg_id=122, B=2, T=50, H=512, V=40, bias=True, eps_low=0.2,
                                      eps_high=0.3),
    "mfma_h640_gspo_q": synth.small("mfma_h640", cfg_id=123, B=3, T=70, H=640, V=1300, w_std=0.03,
                                    loss_type=synth.GSPO_TOKEN, eps_low=3e-3, eps_high=4e-3, old_noise_std=1e-2,
                                    top_entropy_quantile=0.5),
    "mfma_h768_kl_chunked": synth.small("mfma_h768", cfg_id=124, B=4, T=33, H=768, V=700, w_std=0.03,
                                        chunk_sequences=2, beta=0.04, ref_noise_std=0.05, eps_low=0.2,
                                        eps_high=0.3),
    "mfma_v1_degenerate_q": synth.small("mfma_v1", cfg_id=125, B=2, T=30, H=128, V=1, top_entropy_quantile=0.5),
    "generic_bf16_v1": synth.small("generic_v1", cfg_id=126, B=2, T=20, H=96, V=1, bias=True),
    # generic (vector ALU) path: fp32, and bf16 with H not a multiple of 128
    "generic_f32_tiny_b2_t16": synth.WORKLOADS["tiny_gmpo_f32"],
    "generic_bf16_h96": synth.small("generic_h96", cfg_id=106, B=2, T=50, H=96, V=700, bias=True),
    "generic_f32_gspo_chunked": synth.small("generic_gspo", cfg_id=107, dtype="f32", B=3, T=30, H=48, V=300,
                                            loss_type=synth.GSPO_TOKEN, eps_low=0.01, eps_high=0.01,
                                            old_noise_std=0.01, chunk_sequences=2, top_entropy_quantile=0.3),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_small(name):
    spec = SMALL[name]
    _say(f"fused {name} B={spec.B} T={spec.T} H={spec.H} V={spec.V} {spec.dtype}")
    d = make_case(spec)
    ref = run_oracle(spec, d)
    gpu = run_gpu(spec, d)
    _check_fused(spec, d, gpu, ref)


@pytest.mark.parametrize("name", ["mfma_gmpo_kl_bias_tau", "mfma_gspo_q", "mfma_gmpo_q_chunked", "mfma_gmpo_h896",
                                  "mfma_gmpo_wgrad_launches_chunked"])
def test_fused_prepared_weight(name):
    """With the weight's matrix-core copy made beforehand (plp_prepare_weight)
    the call reads the same tiles: every output bitwise equal to the call
    that makes the copy itself, and the oracle's bar met."""
    spec = SMALL[name]
    _say(f"prepared weight {name} B={spec.B} T={spec.T} H={spec.H} V={spec.V}")
    d = make_case(spec)
    a = run_gpu(spec, d)
    b = run_gpu(spec, d, prepare_weight=True)
    assert set(a) == set(b)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    if spec.T <= 4096:
        _check_fused(spec, d, b, run_oracle(spec, d))


def test_fused_deterministic():
    spec = SMALL["mfma_gmpo_q_chunked"]
    _say("determinism")
    d = make_case(spec)
    a = run_gpu(spec, d)
    b = run_gpu(spec, d)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_fused_chunk_invariance():
    """Outer chunk sizes 1, 2 and B agree (batch-global threshold and mean)."""
    base = SMALL["mfma_gmpo_q_chunked"]
    d = make_case(base)
    outs = []
    for cs in (1, 2, 0):
        _say(f"chunk {cs}")
        outs.append(run_gpu(base.replace(chunk_sequences=cs), d))
    for o in outs[1:]:
        assert abs(o["loss"][0] - outs[0]["loss"][0]) < 1e-6
        np.testing.assert_array_equal(o["entropy_mask"], outs[0]["entropy_mask"])
        assert rel_l2(o["grad_weight"], outs[0]["grad_weight"]) < 1e-2
        assert rel_l2(o["grad_hidden"], outs[0]["grad_hidden"]) < 1e-2


def test_fused_bnpo_chunk_invariance():
    """BNPO divides by the batch's completion tokens, not a chunk's: outer
    chunk sizes 1, 2 and B agree."""
    base = SMALL["mfma_bnpo_q_chunked"]
    d = make_case(base)
    outs = []
    for cs in (1, 2, 0):
        _say(f"bnpo chunk {cs}")
        outs.append(run_gpu(base.replace(chunk_sequences=cs), d))
    for o in outs[1:]:
        assert abs(o["loss"][0] - outs[0]["loss"][0]) < 1e-6
        np.testing.assert_array_equal(o["metrics"][[6, 7]], outs[0]["metrics"][[6, 7]])
        assert rel_l2(o["grad_weight"], outs[0]["grad_weight"]) < 1e-2
        assert rel_l2(o["grad_hidden"], outs[0]["grad_hidden"]) < 1e-2


@pytest.mark.parametrize("q,B,T", [(1.0, 2, 40), (0.5, 2, 40), (1.0, 1, 33000)])
def test_fused_flagged_rows_recomputed(q, B, T):
    """Logits far above the first vocabulary tile's max (bias -100 on the first
    tile, +60 further on) make the MFMA sweep flag the rows; a second sweep
    takes them again against their largest logit. With q < 1 the grad_h
    accumulator runs as its own pass over the rows with a gradient, against
    their log-sum-exp. With 33000 flagged rows, the 232 past the second
    sweep's 32768 are recomputed by the merge on the vector ALU."""
    spec = synth.small("flagged", cfg_id=108, B=B, T=T, H=128, V=1000, bias=True, top_entropy_quantile=q)
    _say(f"flagged rows q={q} B={B} T={T}")
    d = synth.make(spec)
    b = d["b"].copy()
    b[:32] = -100.0
    b[700:710] = 60.0
    d["b_raw"] = synth.round_bf16_bits(b)
    d["b"] = synth.bf16_bits_to_f32(d["b_raw"])
    d["fwd"] = oracle.forward_rows(d["h"], d["W"], d["b"], spec.temperature, d["targets"])
    d["old"] = synth.compose_logp(d["fwd"]["logp"], d["old_noise"])
    d["ref"] = None
    ref = run_oracle(spec, d)
    gpu = run_gpu(spec, d)
    _check_fused(spec, d, gpu, ref, lp_tol=1e-4)


def test_fused_outputs_optional():
    """Skipping gradients leaves loss, metrics and diagnostics unchanged."""
    spec = SMALL["mfma_gmpo"]
    d = make_case(spec)
    _say("optional outputs")
    full = run_gpu(spec, d)
    part = run_gpu(spec, d, grad_hidden=False, grad_weight=False)
    for k in ("loss", "metrics", "logp", "entropy", "dlogp"):
        np.testing.assert_array_equal(full[k], part[k], err_msg=k)
    assert "grad_hidden" not in part and "grad_weight" not in part


# ---------------------------------------------------------------------------
# selective_entropy
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", [
    dict(N=200, H=256, V=1000, dtype="bf16", bias=False, tau=1.0),
    dict(N=131, H=896, V=4099, dtype="bf16", bias=True, tau=1.3),
    dict(N=37, H=64, V=517, dtype="f32", bias=True, tau=0.7),
    dict(N=70, H=96, V=300, dtype="bf16", bias=False, tau=1.0),
    dict(N=90, H=640, V=40, dtype="bf16", bias=True, tau=1.0),
    dict(N=300, H=768, V=1, dtype="bf16", bias=False, tau=0.9),
    dict(N=1, H=512, V=2053, dtype="bf16", bias=False, tau=1.0),
])
def test_selective_entropy(case):
    import rl_policy_gradient_amd as plp
    spec = synth.small("se", cfg_id=110, B=1, T=case["N"], H=case["H"], V=case["V"], dtype=case["dtype"],
                       bias=case["bias"], w_std=0.05, prompt_fixed=0)  # prompts play no part here
    _say(f"selective_entropy {case}")
    d = synth.make(spec)
    ref = oracle.forward_rows(d["h"], d["W"], d["b"], case["tau"], d["targets"])
    dt = "bf16" if spec.dtype == "bf16" else None
    ent, lp = plp.selective_entropy(dev_tensor(d["h_raw"], dt), dev_tensor(d["W_raw"], dt),
                                    dev_tensor(d["b_raw"], dt) if d["b_raw"] is not None else None,
                                    dev_tensor(d["targets"]), temperature=case["tau"])
    ent2, none = plp.selective_entropy(dev_tensor(d["h_raw"], dt), dev_tensor(d["W_raw"], dt),
                                       dev_tensor(d["b_raw"], dt) if d["b_raw"] is not None else None, None,
                                       temperature=case["tau"])
    torch.cuda.synchronize()
    tol = 1e-5 if spec.dtype == "f32" else 2e-5
    np.testing.assert_allclose(ent.cpu().numpy(), ref["entropy"], rtol=0, atol=tol)
    np.testing.assert_allclose(lp.cpu().numpy(), ref["logp"], rtol=0, atol=tol)
    assert none is None
    np.testing.assert_array_equal(ent.cpu().numpy(), ent2.cpu().numpy())


@pytest.mark.parametrize("case", [
    dict(N=200, H=256, V=1000, bias=False, tau=1.0, flag=False),
    dict(N=131, H=896, V=4099, bias=True, tau=1.3, flag=False),
    dict(N=90, H=640, V=40, bias=True, tau=1.0, flag=False),
    dict(N=300, H=256, V=1500, bias=True, tau=1.0, flag=True),
])
def test_selective_entropy_prepared_weight(case):
    """plp_selective_entropy_prepared on the weight's matrix-core copy made
    beforehand (plp_prepare_weight): entropy and log-prob bitwise equal to the
    plain call's (which makes the same copy itself), twice in a row on the same
    copy, and the oracle's bar met; with flag, logits far above the first
    tile's (as in the flagged-row test) send every row through the second
    sweep, which reads the prepared copy too."""
    import rl_policy_gradient_amd as plp
    spec = synth.small("se_prep", cfg_id=111, B=1, T=case["N"], H=case["H"], V=case["V"], bias=case["bias"],
                       w_std=0.05, prompt_fixed=0)
    _say(f"selective_entropy prepared weight {case}")
    d = synth.make(spec)
    b_raw = d["b_raw"]
    if case["flag"]:
        b = d["b"].copy()
        b[:32] = -100.0
        b[900:905] = 60.0
        b_raw = synth.round_bf16_bits(b)
    b_f = synth.bf16_bits_to_f32(b_raw) if b_raw is not None else None
    ref = oracle.forward_rows(d["h"], d["W"], b_f, case["tau"], d["targets"])
    h = dev_tensor(d["h_raw"], "bf16")
    W = dev_tensor(d["W_raw"], "bf16")
    bt = dev_tensor(b_raw, "bf16") if b_raw is not None else None
    y = dev_tensor(d["targets"])
    wp = plp.prepare_weight(W)
    ent, lp = plp.selective_entropy(h, W, bt, y, temperature=case["tau"])
    outs = [plp.selective_entropy(h, W, bt, y, temperature=case["tau"], weight_prepared=wp) for _ in range(2)]
    torch.cuda.synchronize()
    for ent_p, lp_p in outs:
        np.testing.assert_array_equal(ent_p.cpu().numpy(), ent.cpu().numpy())
        np.testing.assert_array_equal(lp_p.cpu().numpy(), lp.cpu().numpy())
    tol = 1e-4 if case["flag"] else 2e-5
    np.testing.assert_allclose(outs[0][0].cpu().numpy(), ref["entropy"], rtol=0, atol=tol)
    np.testing.assert_allclose(outs[0][1].cpu().numpy(), ref["logp"], rtol=0, atol=tol)


def test_selective_entropy_flagged_rows():
    """The no-grad entropy entry point with logits far above the first
    tile's (bias -100 on it, +60 further on): every row flagged and taken
    again by the second sweep."""
    import rl_policy_gradient_amd as plp
    spec = synth.small("se_flag", cfg_id=109, B=1, T=300, H=256, V=1500, bias=True, w_std=0.05)
    _say("selective_entropy flagged rows")
    d = synth.make(spec)
    b = d["b"].copy()
    b[:32] = -100.0
    b[900:905] = 60.0
    b_raw = synth.round_bf16_bits(b)
    ref = oracle.forward_rows(d["h"], d["W"], synth.bf16_bits_to_f32(b_raw), 1.0, d["targets"])
    ent, lp = plp.selective_entropy(dev_tensor(d["h_raw"], "bf16"), dev_tensor(d["W_raw"], "bf16"),
                                    dev_tensor(b_raw, "bf16"), dev_tensor(d["targets"]))
    torch.cuda.synchronize()
    np.testing.assert_allclose(ent.cpu().numpy(), ref["entropy"], rtol=0, atol=1e-4)
    np.testing.assert_allclose(lp.cpu().numpy(), ref["logp"], rtol=0, atol=1e-4)




# ---------------------------------------------------------------------------
# Degenerate batches: no token carries a gradient, or a single token
# ---------------------------------------------------------------------------

DEGENERATE = {
    # every advantage zero: the policy term and g vanish (no KL), so the
    # weight-gradient sweep sees no token and every gradient is exactly zero
    "all_zero_advantages": (synth.small("deg_zero_adv", cfg_id=121, B=3, T=40, H=256, V=1000, bias=True),
                            lambda d: d["advantages"].fill(0.0)),
    # no completion token at all
    "empty_completion": (synth.small("deg_empty", cfg_id=122, B=2, T=48, H=128, V=700, bias=True,
                                     loss_type=synth.GRPO, eps_low=0.2, eps_high=0.2),
                         lambda d: d["completion_mask"].fill(0)),
}


@pytest.mark.parametrize("name", list(DEGENERATE))
def test_fused_no_gradient_tokens(name):
    spec, mutate = DEGENERATE[name]
    _say(f"degenerate {name} B={spec.B} T={spec.T} H={spec.H} V={spec.V}")
    d = make_case(spec)
    mutate(d)
    ref = run_oracle(spec, d)
    gpu = run_gpu(spec, d)
    assert ref["loss"] == 0.0 and gpu["loss"][0] == 0.0
    assert not np.any(ref["g"]) and not np.any(gpu["dlogp"])
    for k in ("grad_hidden", "grad_weight", "grad_bias"):
        assert not np.any(gpu[k]), k                      # exactly zero, not merely small
    m, mo = gpu["metrics"], ref["metrics"]
    assert m[6] == mo[6] and m[7] == mo[7], (m, mo)
    np.testing.assert_allclose(gpu["logp"], ref["logp"], rtol=0, atol=2e-5)


def test_fused_single_token():
    """B = T = 1: one completion token against the oracle (the smallest
    problem: one partial row block, one token tile)."""
    spec = synth.small("deg_one", cfg_id=123, B=1, T=1, H=256, V=1000, bias=True, prompt_lo=0, prompt_hi=0,
                       eps_low=0.2, eps_high=0.3)
    _say("degenerate single token")
    d = make_case(spec)
    d["completion_mask"][:] = 1
    d["advantages"][:] = 0.75
    ref = run_oracle(spec, d)
    gpu = run_gpu(spec, d)
    _check_fused(spec, d, gpu, ref)
