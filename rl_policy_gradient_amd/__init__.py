"""Fused LM-head + GRPO-family policy loss on AMD MI355X (gfx950).

Thin torch binding over the C ABI in include/plp.h (libplp.so, built in-tree
by ``python -m rl_policy_gradient_amd.build``). The functions here only turn
torch tensors into device pointers and the current HIP stream, allocate
outputs and workspace with torch, and call the library; every step of the
path runs in the library's HIP kernels. There is no CPU fallback: inputs
must be GPU tensors and the library must be built.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _abi
from ._abi import METRIC_NAMES, PlpError  # noqa: F401

__all__ = [
    "fused_lmhead_policy_loss_fwd_bwd",
    "selective_entropy",
    "entropy_quantile_mask",
    "entropy_quantile_mask_noalloc",
    "policy_loss_from_logprobs",
    "prepare_weight",
    "prepared_weight_size",
    "workspace_size",
    "METRIC_NAMES",
    "PlpError",
]

_LOSS = {"gmpo": _abi.LOSS_GMPO, "gspo_token": _abi.LOSS_GSPO_TOKEN, "grpo": _abi.LOSS_GRPO,
         "bnpo": _abi.LOSS_BNPO, "dapo": _abi.LOSS_DAPO}
_RED = {"seq_mean": _abi.REDUCE_SEQ_MEAN, "token_sum": _abi.REDUCE_TOKEN_SUM}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("plp runs on the GPU only: got a CPU tensor")
    if not t.is_contiguous():
        raise ValueError("plp needs contiguous tensors")
    return t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return _abi.DTYPE_F32
    if t.dtype == torch.bfloat16:
        return _abi.DTYPE_BF16
    raise ValueError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _check_vec(t, n, dtype, name):
    if t is None:
        return None
    if t.numel() != n or t.dtype != dtype:
        raise ValueError(f"{name}: expected {n} elements of {dtype}, got {tuple(t.shape)} {t.dtype}")
    return t


def _mask_u8(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if t.dtype == torch.uint8:
        return t.contiguous()
    return (t != 0).to(torch.uint8).contiguous()


def _fill_args(hidden, weight, bias, targets, old_logp, ref_logp, completion_mask, ratio_mask, advantages, B, T,
               loss_type, importance_sampling_level, reduction, epsilon_low, epsilon_high, beta, temperature,
               top_entropy_quantile, chunk_sequences, global_tokens=0, token_advantages=None,
               kl_bias_correction=False, weight_prepared=None) -> _abi.PlpArgs:
    a = _abi.new_args()
    a.B, a.T = int(B), int(T)
    if hidden is not None:
        a.dtype = _dtype_code(hidden)
        a.H = int(hidden.shape[-1])
        a.V = int(weight.shape[0])
        a.hidden, a.weight, a.bias = _ptr(hidden), _ptr(weight), _ptr(bias)
        a.targets = _ptr(targets)
    a.old_logp, a.ref_logp = _ptr(old_logp), _ptr(ref_logp)
    a.completion_mask, a.ratio_mask = _ptr(completion_mask), _ptr(ratio_mask)
    a.advantages = _ptr(advantages)
    a.loss_type = _LOSS[loss_type]
    if importance_sampling_level is None:
        importance_sampling_level = "sequence" if loss_type == "gspo_token" else "token"
    a.is_level = {"token": _abi.IS_TOKEN, "sequence": _abi.IS_SEQUENCE}[importance_sampling_level]
    a.reduction = _RED[reduction]
    a.epsilon_low, a.epsilon_high = float(epsilon_low), float(epsilon_high)
    a.beta, a.temperature = float(beta), float(temperature)
    a.top_entropy_quantile = float(top_entropy_quantile)
    a.chunk_sequences = int(chunk_sequences)
    a.global_tokens = int(global_tokens)
    a.token_advantages = _ptr(token_advantages)
    a.kl_bias_correction = 1 if kl_bias_correction else 0
    a.weight_prepared = _ptr(weight_prepared)
    return a


def workspace_size(B, T, H, V, dtype=torch.bfloat16, bias=False, top_entropy_quantile=1.0, chunk_sequences=0,
                   loss_type="gmpo", weight_prepared=False) -> int:
    """Bytes of workspace the fused call needs (host arithmetic, no GPU)."""
    a = _abi.new_args()
    a.B, a.T, a.H, a.V = B, T, H, V
    a.dtype = _abi.DTYPE_F32 if dtype == torch.float32 else _abi.DTYPE_BF16
    a.bias = 1 if bias else None
    a.weight_prepared = 256 if weight_prepared else None
    a.loss_type = _LOSS[loss_type]
    a.is_level = _abi.IS_SEQUENCE if loss_type == "gspo_token" else _abi.IS_TOKEN
    a.top_entropy_quantile = top_entropy_quantile
    a.chunk_sequences = chunk_sequences
    n = ctypes.c_size_t()
    _abi.check(_abi.lib().plp_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    return n.value


def fused_lmhead_policy_loss_fwd_bwd(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                                     completion_mask: torch.Tensor, advantages: torch.Tensor, *,
                                     B: Optional[int] = None, T: Optional[int] = None,
                                     bias: Optional[torch.Tensor] = None, old_logp: Optional[torch.Tensor] = None,
                                     ref_logp: Optional[torch.Tensor] = None,
                                     ratio_mask: Optional[torch.Tensor] = None, loss_type: str = "gmpo",
                                     importance_sampling_level: Optional[str] = None, reduction: str = "seq_mean",
                                     epsilon_low: float = 0.2, epsilon_high: float = 0.2, beta: float = 0.0,
                                     temperature: float = 1.0, top_entropy_quantile: float = 1.0,
                                     chunk_sequences: int = 0, global_tokens: int = 0,
                                     token_advantages: Optional[torch.Tensor] = None,
                                     kl_bias_correction: bool = False,
                                     weight_prepared: Optional[torch.Tensor] = None,
                                     grad_hidden: bool = True, grad_weight: bool = True,
                                     grad_bias: Optional[bool] = None, diagnostics: bool = False,
                                     workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None) -> dict:
    """Loss, metrics and gradients of the fused LM head + GMPO / GSPO-token /
    GRPO / BNPO / DAPO objective (plp_fused_lmhead_policy_loss_fwd_bwd);
    global_tokens is DAPO's divisor (0 = the batch's completion tokens);
    token_advantages fp32 [B*T] replaces advantages [B] (pass None for it);
    kl_bias_correction weights each token's K3 term by its importance ratio;
    weight_prepared is prepare_weight(weight) made from the weight's current
    values (the call then skips that copy).
    hidden: [B, T, H] or
    [B*T, H] (then pass B and T); weight [V, H]; targets int64 [B*T];
    masks bool/u8 [B*T]; advantages fp32 [B]. Returns a dict of tensors."""
    if hidden.dim() == 3:
        B, T = hidden.shape[0], hidden.shape[1]
    if B is None or T is None:
        raise ValueError("pass B and T when hidden is 2-D")
    N, H = B * T, hidden.shape[-1]
    V = weight.shape[0]
    dev = hidden.device
    completion_mask = _mask_u8(completion_mask)
    ratio_mask = _mask_u8(ratio_mask)
    _check_vec(targets, N, torch.int64, "targets")
    _check_vec(advantages, B, torch.float32, "advantages")
    _check_vec(token_advantages, N, torch.float32, "token_advantages")
    _check_vec(old_logp, N, torch.float32, "old_logp")
    _check_vec(ref_logp, N, torch.float32, "ref_logp")
    if weight.dtype != hidden.dtype or (bias is not None and bias.dtype != hidden.dtype):
        raise ValueError("hidden, weight and bias must share one dtype")
    if grad_bias is None:
        grad_bias = bias is not None
    a = _fill_args(hidden, weight, bias, targets, old_logp, ref_logp, completion_mask, ratio_mask, advantages, B, T,
                   loss_type, importance_sampling_level, reduction, epsilon_low, epsilon_high, beta, temperature,
                   top_entropy_quantile, chunk_sequences, global_tokens, token_advantages, kl_bias_correction,
                   weight_prepared)
    L = _abi.lib()
    n = ctypes.c_size_t()
    _abi.check(L.plp_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    ws = _workspace(n.value, dev, workspace)
    res = out if out is not None else {}
    if out is None:
        res["loss"] = torch.empty(1, dtype=torch.float32, device=dev)
        res["metrics"] = torch.empty(_abi.NUM_METRICS, dtype=torch.float32, device=dev)
        if grad_hidden:
            res["grad_hidden"] = torch.empty(N, H, dtype=hidden.dtype, device=dev)
        if grad_weight:
            res["grad_weight"] = torch.empty(V, H, dtype=hidden.dtype, device=dev)
        if grad_bias:
            res["grad_bias"] = torch.empty(V, dtype=hidden.dtype, device=dev)
        if diagnostics:
            res["logp"] = torch.empty(N, dtype=torch.float32, device=dev)
            res["entropy"] = torch.empty(N, dtype=torch.float32, device=dev)
            res["entropy_mask"] = torch.empty(N, dtype=torch.uint8, device=dev)
            res["dlogp"] = torch.empty(N, dtype=torch.float32, device=dev)
    o = _abi.new_outputs()
    o.loss, o.metrics = _ptr(res["loss"]), _ptr(res["metrics"])
    o.grad_hidden = _ptr(res.get("grad_hidden"))
    o.grad_weight = _ptr(res.get("grad_weight"))
    o.grad_bias = _ptr(res.get("grad_bias"))
    o.logp_out = _ptr(res.get("logp"))
    o.entropy_out = _ptr(res.get("entropy"))
    o.entropy_mask_out = _ptr(res.get("entropy_mask"))
    o.dlogp_out = _ptr(res.get("dlogp"))
    _abi.check(L.plp_fused_lmhead_policy_loss_fwd_bwd(ctypes.byref(a), ctypes.byref(o), ws.data_ptr(),
                                                      ws.numel() * ws.element_size(), _stream(dev)))
    return res


def prepared_weight_size(H: int, V: int, dtype=torch.bfloat16) -> int:
    """Bytes of the weight's matrix-core copy (plp_prepared_weight_size)."""
    n = ctypes.c_size_t()
    code = _abi.DTYPE_F32 if dtype == torch.float32 else _abi.DTYPE_BF16
    _abi.check(_abi.lib().plp_prepared_weight_size(int(H), int(V), code, ctypes.byref(n)))
    return n.value


def prepare_weight(weight: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The matrix-core copy of weight [V, H] (plp_prepare_weight), for the
    fused call's weight_prepared while the weight keeps these values."""
    V, H = int(weight.shape[0]), int(weight.shape[1])
    n = prepared_weight_size(H, V, weight.dtype)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=weight.device)
    if out.numel() * out.element_size() < n:
        raise ValueError(f"out holds {out.numel() * out.element_size()} bytes, {n} needed")
    _abi.check(_abi.lib().plp_prepare_weight(_ptr(weight), H, V, _dtype_code(weight), _ptr(out),
                                             out.numel() * out.element_size(), _stream(weight.device)))
    return out


def selective_entropy(hidden: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                      targets: Optional[torch.Tensor] = None, temperature: float = 1.0,
                      workspace: Optional[torch.Tensor] = None, weight_prepared: Optional[torch.Tensor] = None):
    """Per-row entropy (and target log-prob when targets are given) by a
    streaming online log-sum-exp over vocabulary tiles
    (plp_selective_entropy; with weight_prepared, made by prepare_weight from
    the weight's current values, plp_selective_entropy_prepared, which skips
    that copy). Returns (entropy, logp or None), fp32 [N]."""
    h2 = hidden.reshape(-1, hidden.shape[-1])
    N, H = h2.shape
    V = weight.shape[0]
    dev = hidden.device
    if targets is not None:
        _check_vec(targets, N, torch.int64, "targets")
    L = _abi.lib()
    n = ctypes.c_size_t()
    dt = _dtype_code(h2)
    if weight_prepared is None:
        _abi.check(L.plp_selective_entropy_workspace_size(N, H, V, dt, ctypes.byref(n)))
    else:
        _abi.check(L.plp_selective_entropy_prepared_workspace_size(N, H, V, dt, ctypes.byref(n)))
    ws = _workspace(n.value, dev, workspace)
    ent = torch.empty(N, dtype=torch.float32, device=dev)
    lp = torch.empty(N, dtype=torch.float32, device=dev) if targets is not None else None
    if weight_prepared is None:
        _abi.check(L.plp_selective_entropy(_ptr(h2), _ptr(weight), _ptr(bias), N, H, V, dt,
                                           ctypes.c_float(temperature), _ptr(targets), _ptr(ent), _ptr(lp),
                                           ws.data_ptr(), ws.numel(), _stream(dev)))
    else:
        _abi.check(L.plp_selective_entropy_prepared(_ptr(h2), _ptr(weight), _ptr(weight_prepared), _ptr(bias), N,
                                                    H, V, dt, ctypes.c_float(temperature), _ptr(targets),
                                                    _ptr(ent), _ptr(lp), ws.data_ptr(), ws.numel(), _stream(dev)))
    return ent, lp


def entropy_quantile_mask(entropy: torch.Tensor, active: torch.Tensor, q: float,
                          workspace: Optional[torch.Tensor] = None):
    """Batch-global high-entropy mask (plp_entropy_quantile_mask).
    Returns (mask u8 [N], threshold fp32 [1])."""
    N = entropy.numel()
    dev = entropy.device
    active = _mask_u8(active)
    _check_vec(entropy, N, torch.float32, "entropy")
    L = _abi.lib()
    n = ctypes.c_size_t()
    _abi.check(L.plp_entropy_quantile_mask_workspace_size(N, ctypes.byref(n)))
    ws = _workspace(n.value, dev, workspace)
    mask = torch.empty(N, dtype=torch.uint8, device=dev)
    thr = torch.empty(1, dtype=torch.float32, device=dev)
    _abi.check(L.plp_entropy_quantile_mask(_ptr(entropy), _ptr(active), N, float(q), _ptr(mask), _ptr(thr),
                                           ws.data_ptr(), ws.numel(), _stream(dev)))
    return mask, thr


def entropy_quantile_mask_noalloc(entropy: torch.Tensor, active: torch.Tensor, q: float, out=None):
    """The batch-global high-entropy mask without a workspace
    (plp_entropy_quantile_mask_noalloc: the select state lives in a static
    device array of the library). Pass out=(mask u8 [N], threshold fp32 [1])
    and a u8 `active` to call without any allocation. Returns (mask,
    threshold)."""
    N = entropy.numel()
    dev = entropy.device
    active = _mask_u8(active)
    _check_vec(entropy, N, torch.float32, "entropy")
    if out is None:
        out = (torch.empty(N, dtype=torch.uint8, device=dev), torch.empty(1, dtype=torch.float32, device=dev))
    mask, thr = out
    _check_vec(mask, N, torch.uint8, "mask")
    _abi.check(_abi.lib().plp_entropy_quantile_mask_noalloc(_ptr(entropy), _ptr(active), N, float(q), _ptr(mask),
                                                            _ptr(thr), _stream(dev)))
    return mask, thr


def policy_loss_from_logprobs(logp: torch.Tensor, completion_mask: torch.Tensor, advantages: torch.Tensor, B: int,
                              T: int, *, old_logp=None, ref_logp=None, ratio_mask=None, entropy=None,
                              loss_type: str = "gmpo", importance_sampling_level: Optional[str] = None,
                              reduction: str = "seq_mean", epsilon_low: float = 0.2, epsilon_high: float = 0.2,
                              beta: float = 0.0, top_entropy_quantile: float = 1.0, global_tokens: int = 0,
                              token_advantages: Optional[torch.Tensor] = None,
                              kl_bias_correction: bool = False,
                              workspace: Optional[torch.Tensor] = None) -> dict:
    """The loss stage alone from per-token log-probs
    (plp_policy_loss_from_logprobs). Returns loss, metrics, dlogp and
    entropy_mask."""
    N = B * T
    dev = logp.device
    completion_mask = _mask_u8(completion_mask)
    ratio_mask = _mask_u8(ratio_mask)
    _check_vec(logp, N, torch.float32, "logp")
    _check_vec(advantages, B, torch.float32, "advantages")
    _check_vec(token_advantages, N, torch.float32, "token_advantages")
    a = _fill_args(None, None, None, None, old_logp, ref_logp, completion_mask, ratio_mask, advantages, B, T,
                   loss_type, importance_sampling_level, reduction, epsilon_low, epsilon_high, beta, 1.0,
                   top_entropy_quantile, 0, global_tokens, token_advantages, kl_bias_correction)
    L = _abi.lib()
    n = ctypes.c_size_t()
    _abi.check(L.plp_policy_loss_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    ws = _workspace(n.value, dev, workspace)
    res = {
        "loss": torch.empty(1, dtype=torch.float32, device=dev),
        "metrics": torch.empty(_abi.NUM_METRICS, dtype=torch.float32, device=dev),
        "dlogp": torch.empty(N, dtype=torch.float32, device=dev),
        "entropy_mask": torch.empty(N, dtype=torch.uint8, device=dev),
    }
    o = _abi.new_outputs()
    o.loss, o.metrics = _ptr(res["loss"]), _ptr(res["metrics"])
    o.dlogp_out, o.entropy_mask_out = _ptr(res["dlogp"]), _ptr(res["entropy_mask"])
    _abi.check(L.plp_policy_loss_from_logprobs(ctypes.byref(a), _ptr(logp), _ptr(entropy), ctypes.byref(o),
                                               ws.data_ptr(), ws.numel(), _stream(dev)))
    return res
