"""Helpers shared by the GPU parity tests: seeded inputs -> device tensors,
the oracle on the same inputs, and the comparison metrics."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; run them with -m gpu on a GPU box")


def dev_tensor(x, dtype=None):
    if x is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def make_case(spec: synth.Spec, fwd=None):
    """Inputs of a workload plus the oracle's forward pass on them; old/ref
    are composed from the oracle's log-probs (never from the GPU)."""
    d = synth.make(spec)
    if fwd is None:
        fwd = oracle.forward_rows(d["h"], d["W"], d["b"], spec.temperature, d["targets"])
    d["fwd"] = fwd
    d["old"] = synth.compose_logp(fwd["logp"], d["old_noise"])
    d["ref"] = synth.compose_logp(fwd["logp"], d["ref_noise"])
    return d


def gpu_inputs(spec: synth.Spec, d: dict) -> dict:
    dt = "bf16" if spec.dtype == "bf16" else None
    return dict(
        hidden=dev_tensor(d["h_raw"], dt),
        weight=dev_tensor(d["W_raw"], dt),
        bias=dev_tensor(d["b_raw"], dt) if d["b_raw"] is not None else None,
        targets=dev_tensor(d["targets"]),
        completion_mask=dev_tensor(d["completion_mask"]),
        advantages=dev_tensor(d["advantages"]) if d.get("token_advantages") is None else None,
        token_advantages=dev_tensor(d.get("token_advantages")),
        old_logp=dev_tensor(d["old"]),
        ref_logp=dev_tensor(d["ref"]),
    )


def run_gpu(spec: synth.Spec, d: dict, prepare_weight: bool = False, **kw) -> dict:
    """The fused call on the seeded inputs; prepare_weight: pass the
    weight's matrix-core copy made beforehand by plp.prepare_weight."""
    import rl_policy_gradient_amd as plp
    g = gpu_inputs(spec, d)
    if prepare_weight:
        kw["weight_prepared"] = plp.prepare_weight(g["weight"])
    args = dict(B=spec.B, T=spec.T, loss_type=spec.loss_type, epsilon_low=spec.eps_low,
                epsilon_high=spec.eps_high, beta=spec.beta, temperature=spec.temperature,
                top_entropy_quantile=spec.top_entropy_quantile, chunk_sequences=spec.chunk_sequences,
                reduction=spec.reduction, global_tokens=spec.global_tokens,
                token_advantages=g["token_advantages"], kl_bias_correction=spec.kl_bias_correction,
                diagnostics=True)
    args.update(kw)
    out = plp.fused_lmhead_policy_loss_fwd_bwd(g["hidden"], g["weight"], g["targets"], g["completion_mask"],
                                               g["advantages"], bias=g["bias"], old_logp=g["old_logp"],
                                               ref_logp=g["ref_logp"], **args)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() if v.dtype != torch.uint8 else v.cpu().numpy() for k, v in out.items()}


def run_oracle(spec: synth.Spec, d: dict, want_grads=True) -> dict:
    cfg = oracle.LossConfig.from_spec(spec)
    tadv = d.get("token_advantages")
    return oracle.run(cfg, d["h"], d["W"], d["b"], d["targets"], d["old"], d["ref"], d["completion_mask"], None,
                      None if tadv is not None else d["advantages"], want_grads=want_grads, fwd=d["fwd"],
                      token_advantages=tadv)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def clip_margin(spec: synth.Spec, d: dict, lp) -> float:
    """Smallest distance of an active fp32 log-ratio to a token clip bound in
    log space (GMPO: eps_high, -eps_low; GRPO / BNPO / DAPO: log of the fp32
    ratio bounds). A predicate closer than the log-prob tolerance could
    legitimately flip."""
    if d["old"] is None:
        return np.inf
    if spec.loss_type == synth.GMPO:
        hi, lo = float(np.float32(spec.eps_high)), -float(np.float32(spec.eps_low))
    elif spec.loss_type in (synth.GRPO, synth.BNPO, synth.DAPO):
        hi = np.log(float(np.float32(1 + spec.eps_high)))
        lo = np.log(float(np.float32(1 - spec.eps_low)))
    else:
        return np.inf
    lr = np.asarray(lp, np.float64) - d["old"].astype(np.float64)
    act = d["completion_mask"] != 0
    return float(min(np.abs(lr - hi)[act].min(), np.abs(lr - lo)[act].min()))


def grad_tol(spec: synth.Spec):
    """(rel-L2 bound, cosine bound) for gradients at the workload's dtype."""
    return (1e-4, 0.99999999) if spec.dtype == "f32" else (1e-2, 0.9999)
