"""Seeded synthetic inputs for the fused LM-head policy-loss path.

This module draws random numbers and rounds them to the storage dtype. It
holds none of the method's arithmetic: no logits, no log-probabilities, no
loss. Quantities that the workloads define relative to the current policy
("old = current log-prob + noise") are returned as the noise alone; the
caller adds it to a log-prob that it obtained by its own means.

Both the CPU oracle (under ``oracle/``) and the GPU path consume these
arrays; neither side imports the other.

Workloads (shapes and value distributions follow the pages' Qwen-0.5B LM-head
setting, hidden 896 and vocabulary 151936, Liger PR #1320 "Forward and
backward numerical comparison"; GSPO defaults from the Tinker GSPO page,
"Choosing clipping thresholds"; entropy masking from Liger PR #1558):

  cfg 1  tiny GMPO, fp32   B=2  T=16    H=64  V=512
  cfg 2  GMPO, bf16        B=1  T=512   H=896 V=151936
  cfg 3  GMPO + K3 KL      B=8  T=2048  H=896 V=151936, bias
  cfg 4  GSPO-token + q    B=2  T=32768 H=896 V=151936
  cfg 5  GMPO, chunked     B=128 T=32768 H=896 V=151936, bias
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

GMPO = "gmpo"
GSPO_TOKEN = "gspo_token"
GRPO = "grpo"
BNPO = "bnpo"
DAPO = "dapo"

# Stream ids inside SeedSequence([seed, cfg_id, stream]).
_S_H, _S_W, _S_B, _S_Y, _S_P, _S_A, _S_OLD, _S_REF, _S_ZERO = range(9)
_S_TADV = 20


@dataclass(frozen=True)
class Spec:
    """One synthetic workload: shapes, dtype, loss settings, generator recipe."""

    name: str
    cfg_id: int
    B: int
    T: int
    H: int
    V: int
    dtype: str = "bf16"            # "f32" or "bf16": storage dtype of h, W, b
    bias: bool = False
    h_std: float = 1.0
    w_std: float = 0.02
    b_std: float = 0.01
    loss_type: str = GMPO
    eps_low: float = 0.4
    eps_high: float = 0.4
    beta: float = 0.0
    temperature: float = 1.0
    top_entropy_quantile: float = 1.0
    old_noise_std: float = 0.1
    ref_noise_std: Optional[float] = None   # None: no reference log-probs
    prompt_fixed: Optional[int] = None      # fixed prompt length, else uniform
    prompt_lo: int = 32
    prompt_hi: int = 128
    adv_kind: str = "normal"                # "normal" or "pm1z" ({+1,-1,0})
    zero_adv_fraction: float = 0.0          # exact share of sequences with A=0
    chunk_sequences: int = 0                # 0: whole batch in one chunk
    reduction: str = "seq_mean"             # "seq_mean" or "token_sum"
    global_tokens: int = 0                  # DAPO divisor; 0 = the batch's completion tokens
    token_adv: bool = False                 # one advantage per token (N,) instead of per sequence
    kl_bias_correction: bool = False        # KL term weighted by the token importance ratio
    seed: int = 0

    @property
    def N(self) -> int:
        return self.B * self.T

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


_SPECS = (
    Spec("tiny_gmpo_f32", 1, B=2, T=16, H=64, V=512, dtype="f32", w_std=0.05,
         old_noise_std=0.2, prompt_fixed=4, adv_kind="pm1z"),
    Spec("gmpo_bf16_b1_t512", 2, B=1, T=512, H=896, V=151936,
         prompt_lo=32, prompt_hi=128),
    Spec("gmpo_kl_bf16_b8_t2048", 3, B=8, T=2048, H=896, V=151936, bias=True,
         eps_low=0.2, eps_high=0.3, beta=0.04, ref_noise_std=0.05,
         prompt_lo=64, prompt_hi=512, zero_adv_fraction=0.25),
    Spec("gspo_token_entropy_bf16_b2_t32768", 4, B=2, T=32768, H=896, V=151936,
         loss_type=GSPO_TOKEN, eps_low=3e-4, eps_high=4e-4, old_noise_std=1e-4,
         top_entropy_quantile=0.2, prompt_lo=256, prompt_hi=2048),
    Spec("gmpo_bf16_b128_t32768_chunked", 5, B=128, T=32768, H=896, V=151936,
         bias=True, chunk_sequences=8, prompt_lo=32, prompt_hi=128),
)
# the workloads by name, and by the workload id that also seeds them
WORKLOADS = {s.name: s for s in _SPECS}
BY_ID = {s.cfg_id: s for s in _SPECS}


def _rng(spec: Spec, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([spec.seed, spec.cfg_id, stream]))


def round_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Adds 0x7FFF plus the lowest kept bit and truncates; in uint32 this cannot
    wrap for any non-NaN input (NaNs are set to the canonical quiet NaN)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    out = np.empty(x32.shape, dtype=np.uint16)
    flat_in = x32.reshape(-1).view(np.uint32)
    flat_out = out.reshape(-1)
    step = 1 << 22
    for a in range(0, flat_in.size, step):
        u = flat_in[a:a + step]
        r = (u >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        r += u
        r >>= np.uint32(16)
        flat_out[a:a + step] = r
        nan = np.isnan(x32.reshape(-1)[a:a + step])
        if nan.any():
            flat_out[a:a + step][nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _store(spec: Spec, x32: np.ndarray):
    """Round to the storage dtype. Returns (values widened to fp32, raw storage)."""
    if spec.dtype == "bf16":
        bits = round_bf16_bits(x32)
        return bf16_bits_to_f32(bits), bits
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    return x32, x32


def _normal_f32(rng, shape, std, chunk_rows=65536):
    """Standard-normal draws scaled by std, generated in row chunks to bound memory."""
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32) * np.float32(std)
    return out


def prompt_lengths(spec: Spec) -> np.ndarray:
    if spec.prompt_fixed is not None:
        return np.full(spec.B, spec.prompt_fixed, dtype=np.int64)
    lo, hi = spec.prompt_lo, min(spec.prompt_hi, spec.T)
    return _rng(spec, _S_P).integers(lo, hi + 1, size=spec.B, dtype=np.int64)


def completion_mask(spec: Spec) -> np.ndarray:
    """u8 [B*T]: token t of sequence i is a completion token iff t >= prompt_i."""
    P = prompt_lengths(spec)
    t = np.arange(spec.T, dtype=np.int64)
    return (t[None, :] >= P[:, None]).astype(np.uint8).reshape(-1)


def advantages(spec: Spec) -> np.ndarray:
    rng = _rng(spec, _S_A)
    if spec.adv_kind == "pm1z":
        a = rng.choice(np.array([1.0, -1.0, 0.0], dtype=np.float32), size=spec.B)
    else:
        a = rng.standard_normal(spec.B).astype(np.float32)
    if spec.zero_adv_fraction > 0:
        k = int(round(spec.zero_adv_fraction * spec.B))
        zero = _rng(spec, _S_ZERO).choice(spec.B, size=k, replace=False)
        a[zero] = 0.0
    return a.astype(np.float32)


def token_advantages(spec: Spec, completion: np.ndarray) -> np.ndarray:
    """Per-token advantages [N]: N(0,1) on completion tokens, 0 elsewhere (the
    layout of a datum whose advantages are zeroed off the completion)."""
    a = _rng(spec, _S_TADV).standard_normal(spec.N).astype(np.float32)
    return np.where(np.asarray(completion) != 0, a, np.float32(0.0)).astype(np.float32)


def targets(spec: Spec) -> np.ndarray:
    return _rng(spec, _S_Y).integers(0, spec.V, size=spec.N, dtype=np.int64)


def hidden(spec: Spec, rows: Optional[np.ndarray] = None):
    """Hidden states [N,H]. Rows are generated in fixed blocks of 4096 so that a
    row subset can be regenerated without drawing the whole matrix."""
    blk = 4096
    if rows is None:
        out = np.empty((spec.N, spec.H), dtype=np.float32)
        for b0 in range(0, spec.N, blk):
            b1 = min(spec.N, b0 + blk)
            out[b0:b1] = _hidden_block(spec, b0 // blk)[: b1 - b0]
        return _store(spec, out)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), spec.H), dtype=np.float32)
    for bi in np.unique(rows // blk):
        blkv = _hidden_block(spec, int(bi))
        sel = np.nonzero(rows // blk == bi)[0]
        out[sel] = blkv[rows[sel] - bi * blk]
    return _store(spec, out)


def hidden_block(spec: Spec, bi: int):
    """Rows [4096 bi, 4096 bi + 4096) of the hidden states, as (fp32 values,
    raw storage); blocks are independent, so they can be drawn in parallel."""
    return _store(spec, _hidden_block(spec, bi))


def _hidden_block(spec: Spec, bi: int) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([spec.seed, spec.cfg_id, _S_H, bi]))
    rows = min(4096, spec.N - bi * 4096)
    return rng.standard_normal((rows, spec.H), dtype=np.float32) * np.float32(spec.h_std)


def weight(spec: Spec):
    return _store(spec, _normal_f32(_rng(spec, _S_W), (spec.V, spec.H), spec.w_std))


def bias(spec: Spec):
    if not spec.bias:
        return None, None
    return _store(spec, _rng(spec, _S_B).standard_normal(spec.V, dtype=np.float32) * np.float32(spec.b_std))


def old_noise(spec: Spec) -> np.ndarray:
    """fp64 noise added to the current-policy log-prob to form old_logp."""
    return _rng(spec, _S_OLD).standard_normal(spec.N) * spec.old_noise_std


def ref_noise(spec: Spec) -> Optional[np.ndarray]:
    if spec.ref_noise_std is None:
        return None
    return _rng(spec, _S_REF).standard_normal(spec.N) * spec.ref_noise_std


def compose_logp(current_logp: np.ndarray, noise: Optional[np.ndarray]) -> Optional[np.ndarray]:
    """fp32(fp32(current) + noise): the recipe for old/ref log-probs (the
    current-policy log-prob is taken at fp32, as a sampler would report it)."""
    if noise is None:
        return None
    cur = np.asarray(current_logp, dtype=np.float32).astype(np.float64)
    return (cur + noise).astype(np.float32)


def small(name="small", **kw) -> Spec:
    """A small ad-hoc workload for parity tests (cfg_id 100 keeps it apart)."""
    base = dict(cfg_id=100, B=2, T=40, H=128, V=1000, dtype="bf16", w_std=0.05,
                prompt_lo=3, prompt_hi=10)
    base.update(kw)
    return Spec(name, **base)


def make(spec: Spec, with_hidden: bool = True) -> dict:
    """All inputs except the log-prob-relative ones, as numpy arrays.

    Keys: h (fp32 values), h_raw (storage: uint16 bf16 bits or fp32), W, W_raw,
    b, b_raw (None without bias), targets, completion_mask, advantages,
    old_noise, ref_noise.
    """
    d = {}
    if with_hidden:
        d["h"], d["h_raw"] = hidden(spec)
    d["W"], d["W_raw"] = weight(spec)
    d["b"], d["b_raw"] = bias(spec)
    d["targets"] = targets(spec)
    d["completion_mask"] = completion_mask(spec)
    d["advantages"] = advantages(spec)
    d["token_advantages"] = token_advantages(spec, d["completion_mask"]) if spec.token_adv else None
    d["old_noise"] = old_noise(spec)
    d["ref_noise"] = ref_noise(spec)
    return d
