#!/usr/bin/env python3
"""Throughput of the fused LM-head + GMPO / GSPO-token forward+backward on one
MI355X, with the roofline of the dominant kernel and the CPU oracle beside it.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2|3|4|5]
                  [--loss gmpo|gspo_token|grpo|bnpo|dapo] [--token-advantages]

The default workload is the largest one-GPU shape: GMPO at B=128, T=32768
(4.19M tokens), H=896, V=151936, with a bias, in outer chunks of 8 sequences.
--config 2 is B=1 T=512, 3 is B=8 T=2048 GMPO + K3 KL, 4 is B=2 T=32768
GSPO-token with the entropy mask.

--prepared-weight makes the weight's matrix-core copy once before the timed
steps (the case of several calls per weight update); the line's workload
name carries "+prepared_weight".

--loss runs the workload's inputs under another loss type (same clip
parameters); --token-advantages gives every completion token its own
advantage (N(0,1), zero off the completion) instead of one per sequence.

One step = one call of plp_fused_lmhead_policy_loss_fwd_bwd on one batch of
synthetic inputs already resident in HBM: forward statistics, loss, metrics,
grad_hidden, grad_weight (and grad_bias). Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "tokens/s fused LM-head+GMPO fwd+bwd, H=896 V=151936; % bf16 MFMA peak"


def _workload(cfg: int, device):
    """Inputs of workload `cfg` on the GPU. cfg 2 uses the seeded generators
    shared with the parity tests; the larger ones draw the same distributions
    with a seeded torch generator on the device (host generation of 7.5 GB of
    hidden states would dominate the run)."""
    import numpy as np
    import torch

    import synth
    from rl_policy_gradient_amd import selective_entropy

    spec = synth.BY_ID[cfg]
    B, T, H, V, N = spec.B, spec.T, spec.H, spec.V, spec.N
    if cfg in (1, 2):
        d = synth.make(spec)
        dt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32

        def up(x, bf):
            if x is None:
                return None
            if bf:
                return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
            return torch.from_numpy(np.ascontiguousarray(x)).to(device)

        bf = spec.dtype == "bf16"
        h, W = up(d["h_raw"], bf), up(d["W_raw"], bf)
        b = up(d["b_raw"], bf)
        y = up(d["targets"], False)
        comp = up(d["completion_mask"], False)
        adv = up(d["advantages"], False)
        old_noise = torch.from_numpy(d["old_noise"]).to(device)
        ref_noise = None if d["ref_noise"] is None else torch.from_numpy(d["ref_noise"]).to(device)
    else:
        g = torch.Generator(device=device)
        g.manual_seed(1000 + cfg)
        h = torch.randn(N, H, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
        W = (torch.randn(V, H, generator=g, device=device) * spec.w_std).to(torch.bfloat16)
        b = (torch.randn(V, generator=g, device=device) * spec.b_std).to(torch.bfloat16) if spec.bias else None
        y = torch.randint(0, V, (N,), generator=g, device=device, dtype=torch.int64)
        P = torch.randint(spec.prompt_lo, spec.prompt_hi + 1, (B,), generator=g, device=device)
        comp = (torch.arange(T, device=device)[None, :] >= P[:, None]).to(torch.uint8).reshape(-1).contiguous()
        adv = torch.randn(B, generator=g, device=device)
        if spec.zero_adv_fraction > 0:
            k = int(round(spec.zero_adv_fraction * B))
            adv[torch.randperm(B, generator=g, device=device)[:k]] = 0
        old_noise = torch.randn(N, generator=g, device=device, dtype=torch.float64) * spec.old_noise_std
        ref_noise = (torch.randn(N, generator=g, device=device, dtype=torch.float64) * spec.ref_noise_std
                     if spec.ref_noise_std is not None else None)
    # old / ref = current log-prob + noise; the current log-prob comes from the
    # GPU's own forward (outside the timed region)
    _, lp = selective_entropy(h, W, b, y, temperature=spec.temperature)
    old = (lp.double() + old_noise).float().contiguous()
    ref = (lp.double() + ref_noise).float().contiguous() if ref_noise is not None else None
    torch.cuda.synchronize()
    return spec, dict(hidden=h, weight=W, bias=b, targets=y, completion_mask=comp, advantages=adv,
                      old_logp=old, ref_logp=ref)


def _traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain-copy calibration), read from the committed
    summary; None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    from rl_policy_gradient_amd.profsum import kernel_src_hash

    if d.get("kernel_src_hash") != kernel_src_hash():
        return None
    return d.get("bytes_per_launch")


def _cpu_baseline(spec) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the workload: one
    sequence of up to 512 tokens at the workload's H and V (the whole workload
    for config 2), forward + loss + backward, on all host cores."""
    import numpy as np

    import oracle
    import synth

    sample = spec.replace(B=1, T=min(spec.T, 512), chunk_sequences=0)
    d = synth.make(sample)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    fwd = oracle.forward_rows(d["h"], d["W"], d["b"], sample.temperature, d["targets"])
    old = synth.compose_logp(fwd["logp"], d["old_noise"])
    ref = synth.compose_logp(fwd["logp"], d["ref_noise"])
    out = oracle.run(oracle.LossConfig.from_spec(sample), d["h"], d["W"], d["b"], d["targets"], old, ref,
                     d["completion_mask"], None, d["advantages"], fwd=fwd)
    dt = time.perf_counter() - t0
    assert np.isfinite(out["loss"])
    return {"value": round(sample.N / dt, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"B=1 T={sample.T} H={sample.H} V={sample.V} ({sample.N} tokens of {spec.name}); "
                      f"fp64 forward+loss+backward in {dt:.2f} s"}


def _memory_sweep(dev) -> int:
    """Peak device memory of one fused call (GMPO, bf16, H=896, grads of h
    and W) beyond its inputs, over vocabulary sizes and token counts: the
    caching allocator's peak during the call minus what was allocated before
    it (workspace + outputs), beside the bytes a materialised [N, V] bf16
    logit tensor would take. One JSON line per shape."""
    import torch

    import rl_policy_gradient_amd as plp

    H = 896
    for V in (32000, 65536, 151936):
        for N in (512, 4096, 32768):
            B, T = max(1, N // 4096), min(N, 4096)
            g = torch.Generator(device=dev)
            g.manual_seed(N + V)
            h = torch.randn(N, H, generator=g, device=dev).to(torch.bfloat16)
            W = (torch.randn(V, H, generator=g, device=dev) * 0.02).to(torch.bfloat16)
            y = torch.randint(0, V, (N,), generator=g, device=dev)
            comp = torch.ones(N, dtype=torch.uint8, device=dev)
            adv = torch.randn(B, generator=g, device=dev)
            torch.cuda.synchronize()
            before = torch.cuda.memory_allocated(dev)
            torch.cuda.reset_peak_memory_stats(dev)
            out = plp.fused_lmhead_policy_loss_fwd_bwd(h, W, y, comp, adv, B=B, T=T, epsilon_low=0.4,
                                                       epsilon_high=0.4)
            torch.cuda.synchronize()
            peak = torch.cuda.max_memory_allocated(dev) - before
            ws = plp.workspace_size(B, T, H, V)
            print(json.dumps({"V": V, "N": N, "H": H, "peak_bytes_beyond_inputs": int(peak), "workspace_bytes": int(ws),
                              "outputs_bytes": int(N * H * 2 + V * H * 2 + 8 + 32),
                              "materialised_bf16_logits_bytes": int(N * V * 2)}), flush=True)
            del out, h, W, y, comp, adv
            torch.cuda.empty_cache()
    return 0


def _flagged_rows(h, W, b, spec) -> int:
    """Rows the forward sweep flags for the exact recompute: in some
    vocabulary split a logit exceeds the max of the split's first 32-row tile
    by more than 64 (the sweep's exponent reference slack). Computed here
    from the logits with torch, split by split as the sweep walks them."""
    import torch

    z = (h.float() @ W.float().T + b.float()[None, :]) / spec.temperature
    n_tiles = -(-spec.V // 32)
    nrb = -(-spec.N // 64)
    sv = 1
    while sv * nrb < 256 and sv < 64 and sv * 2 <= n_tiles:
        sv *= 2
    tps = -(-n_tiles // sv)
    flag = torch.zeros(spec.N, dtype=torch.bool, device=z.device)
    for s0 in range(0, n_tiles, tps):
        v0, v1 = 32 * s0, min(spec.V, 32 * (s0 + tps))
        ref = z[:, v0:min(v1, v0 + 32)].max(dim=1).values
        flag |= z[:, v0:v1].max(dim=1).values > ref + 64.0
    return int(flag.sum().item())


def _cpu_baseline_full(cfg: int) -> dict:
    """The fp64 oracle, as it stands, on a whole workload (forward, loss and
    backward over every token, all host cores); the long-run companion of
    the bounded sample timed beside each GPU measurement."""
    import numpy as np

    import oracle
    import synth

    spec = synth.BY_ID[cfg]
    d = synth.make(spec)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    fwd = oracle.forward_rows(d["h"], d["W"], d["b"], spec.temperature, d["targets"])
    t1 = time.perf_counter()
    old = synth.compose_logp(fwd["logp"], d["old_noise"])
    ref = synth.compose_logp(fwd["logp"], d["ref_noise"])
    out = oracle.run(oracle.LossConfig.from_spec(spec), d["h"], d["W"], d["b"], d["targets"], old, ref,
                     d["completion_mask"], None, d["advantages"], fwd=fwd)
    t2 = time.perf_counter()
    assert np.isfinite(out["loss"])
    return {"workload": spec.name, "tokens": spec.N, "cores": int(cores), "kind": "oracle",
            "forward_s": round(t1 - t0, 2), "loss_and_backward_s": round(t2 - t1, 2),
            "total_s": round(t2 - t0, 2), "tokens_per_s": round(spec.N / (t2 - t0), 3)}


def _gemm_ceiling(dev) -> int:
    """Plain library GEMMs (torch.mm, bf16 operands, fp32 accumulation) at the
    contraction shapes of the sweeps, H=896 V=151936: the logits [N,H]x[H,V],
    the grad_W product [V,N]x[N,H] and the grad_h product [N,V]x[V,H], each
    timed with events over a few repetitions. They give the rate a vendor
    GEMM reaches on this chip at these shapes, beside the sweeps' executed
    rate; they are not part of the path. One JSON line per product."""
    import torch

    H, V = 896, 151936
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    for N in (16384, 65536):
        h = torch.randn(N, H, generator=g, device=dev).to(torch.bfloat16)
        wt = (torch.randn(H, V, generator=g, device=dev) * 0.02).to(torch.bfloat16)   # [H, V], contiguous
        p = (torch.rand(N, V, generator=g, device=dev) * 1e-5).to(torch.bfloat16)      # [N, V]
        pt = p.t().contiguous()                                                        # [V, N]
        w = wt.t().contiguous()                                                        # [V, H]
        cases = (("logits", lambda: torch.mm(h, wt), (N, H, V)),
                 ("grad_w", lambda: torch.mm(pt, h), (V, N, H)),
                 ("grad_h", lambda: torch.mm(p, w), (N, V, H)))
        for name, fn, (m, k, n) in cases:
            for _ in range(2):
                out = fn()
            torch.cuda.synchronize()
            reps = 5
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                out = fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            tf = 2.0 * m * k * n / (ms * 1e-3) / 1e12
            print(json.dumps({"gemm": name, "M": m, "K": k, "N": n, "ms": round(ms, 4), "tflops": round(tf, 1),
                              "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}), flush=True)
            del out
        del h, wt, p, pt, w
        torch.cuda.empty_cache()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=5, choices=[2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--loss", choices=["gmpo", "gspo_token", "grpo", "bnpo", "dapo"], default=None)
    ap.add_argument("--token-advantages", action="store_true")
    ap.add_argument("--kl-bias-correction", action="store_true",
                    help="K3 KL weighted by the token importance ratio (workloads with a KL term)")
    ap.add_argument("--prepared-weight", action="store_true",
                    help="make the weight's matrix-core copy once, before the timed steps (plp_prepare_weight), "
                         "as for the calls between two weight updates, e.g. the micro-batches of a gradient "
                         "accumulation; the steps then skip that copy")
    ap.add_argument("--memory-sweep", action="store_true",
                    help="peak device memory of one fused call over vocabulary sizes and token counts (one line each)")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="time plain library bf16 GEMMs at the sweeps' contraction shapes (one line each)")
    ap.add_argument("--bias-std", type=float, default=None,
                    help="--config 2 with a bias ~ N(0, S^2): logits far above a vocabulary split's first tile "
                         "make the sweep flag rows for the exact recompute; reports how many")
    ap.add_argument("--cpu-baseline-full", action="store_true",
                    help="only time the CPU oracle on the whole workload (--config 2, 3 or 4; no GPU)")
    args = ap.parse_args()
    if args.cpu_baseline_full:
        if args.config == 5:
            print("the whole 4.19M-token workload takes the oracle hours: its time is the sample rate "
                  "extrapolated (cpu_baseline.extrapolated_full_workload_s)", file=sys.stderr)
            return 2
        print(json.dumps(_cpu_baseline_full(args.config)), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU: there is no multi-GPU path (asked for --gpus {args.gpus}); "
              "the path shards by whole sequences, each GPU running this call on its own share",
              file=sys.stderr)
        return 2

    import torch

    import rl_policy_gradient_amd as plp
    from rl_policy_gradient_amd import _abi

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.memory_sweep:
        return _memory_sweep(dev)
    if args.gemm_ceiling:
        return _gemm_ceiling(dev)
    spec, inp = _workload(args.config, dev)
    flagged = None
    if args.bias_std is not None:
        if args.config != 2:
            print("--bias-std is for --config 2", file=sys.stderr)
            return 2
        g = torch.Generator(device=dev)
        g.manual_seed(77)
        b = (torch.randn(spec.V, generator=g, device=dev) * args.bias_std).to(torch.bfloat16)
        inp["bias"] = b
        spec = spec.replace(bias=True, name=f"{spec.name}_bias_std{args.bias_std:g}")
        flagged = _flagged_rows(inp["hidden"], inp["weight"], b, spec)
        _, lp = plp.selective_entropy(inp["hidden"], inp["weight"], b, inp["targets"])
        inp["old_logp"] = (lp.double() + torch.randn(spec.N, generator=g, device=dev, dtype=torch.float64)
                           * spec.old_noise_std).float().contiguous()
    N, H, V = spec.N, spec.H, spec.V
    variant = ""
    if args.loss and args.loss != spec.loss_type:
        spec = spec.replace(loss_type=args.loss)
        variant += "+" + args.loss
    tadv = None
    if args.token_advantages:
        if spec.loss_type == "gmpo":
            print("--token-advantages needs a loss other than gmpo (GMPO's advantages are per sequence)",
                  file=sys.stderr)
            return 2
        g = torch.Generator(device=dev)
        g.manual_seed(4242 + args.config)
        tadv = (torch.randn(N, generator=g, device=dev) * (inp["completion_mask"] != 0)).float().contiguous()
        variant += "+token_adv"
    if args.kl_bias_correction:
        if spec.beta == 0.0 or inp["ref_logp"] is None:
            print("--kl-bias-correction needs a workload with a KL term (--config 3)", file=sys.stderr)
            return 2
        spec = spec.replace(kl_bias_correction=True)
        variant += "+kl_bias_corrected"
    kw = dict(B=spec.B, T=spec.T, loss_type=spec.loss_type, epsilon_low=spec.eps_low, epsilon_high=spec.eps_high,
              beta=spec.beta, temperature=spec.temperature, top_entropy_quantile=spec.top_entropy_quantile,
              chunk_sequences=spec.chunk_sequences, kl_bias_correction=spec.kl_bias_correction,
              diagnostics=False)
    torch.cuda.synchronize()
    mem_inputs = torch.cuda.memory_allocated(dev)  # inputs resident before the call's own memory
    torch.cuda.reset_peak_memory_stats(dev)
    ws = torch.empty(plp.workspace_size(spec.B, spec.T, H, V, bias=spec.bias,
                                        top_entropy_quantile=spec.top_entropy_quantile,
                                        chunk_sequences=spec.chunk_sequences, loss_type=spec.loss_type,
                                        weight_prepared=args.prepared_weight),
                     dtype=torch.uint8, device=dev)
    wprep = plp.prepare_weight(inp["weight"]) if args.prepared_weight else None
    if wprep is not None:
        variant += "+prepared_weight"
    call_args = (inp["hidden"], inp["weight"], inp["targets"], inp["completion_mask"], inp["advantages"])
    call_kw = dict(bias=inp["bias"], old_logp=inp["old_logp"], ref_logp=inp["ref_logp"], workspace=ws,
                   token_advantages=tadv, weight_prepared=wprep, **kw)
    out = plp.fused_lmhead_policy_loss_fwd_bwd(*call_args, **call_kw)
    out["dlogp"] = torch.empty(N, dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        plp.fused_lmhead_policy_loss_fwd_bwd(*call_args, out=out, **call_kw)
    torch.cuda.synchronize()

    L = _abi.lib()
    n_chunks = 1 if spec.chunk_sequences == 0 else -(-spec.B // spec.chunk_sequences)
    # event pairs: a forward and up to a few weight-gradient launches per chunk
    _abi.check(L.plp_profile_start(16 * args.steps * n_chunks + 64))
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        plp.fused_lmhead_policy_loss_fwd_bwd(*call_args, out=out, **call_kw)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (ctypes.c_double * 3)()
    cnt = (ctypes.c_int32 * 3)()
    _abi.check(L.plp_profile_stop_n(ms, cnt, 3))
    elapsed = t1 - t0
    ms_step = 1e3 * elapsed / args.steps
    tokens_s = N * args.steps / elapsed
    flops_tok = 6.0 * H * V
    tflops = tokens_s * flops_tok / 1e12
    peak_delta = torch.cuda.max_memory_allocated(dev) - mem_inputs

    # roofline of the dominant sweep
    n_active = int((out["dlogp"] != 0).sum().item())
    # per launch: algorithmic FLOP and HBM bytes of each sweep, the step's
    # amount over its launches (the library times every launch of each kind
    # with HIP events on the call's stream):
    # - fwd_sweep, the forward sweep over every row of a chunk: the logits
    #   (2HV per row) and, without the entropy mask, the grad_h accumulator
    #   (another 2HV); it reads W once per launch and each row once;
    # - fwd_compact_sweep (entropy mask on): the logits and the accumulator
    #   again for the rows with a gradient only, 4HV each; W once per
    #   launch, those rows once;
    # - wgrad_sweep: 4HV per row with a gradient, the sweep's own step: it
    #   forms the logits again, since the [N, V] probabilities are never
    #   stored, and then the grad_W product (that product alone, 2HV, is
    #   reported beside it); W read and grad_W written once per step, those
    #   rows once, bias and grad_b when present.
    q_lt_1 = spec.top_entropy_quantile < 1.0
    bias_b = 2.0 * V if spec.bias else 0.0
    steps_f = float(args.steps)
    kinds = {
        "fwd_sweep": (0, (2.0 if q_lt_1 else 4.0) * H * V * N, 2.0 * H * N, 2.0 * H * V + bias_b),
        "wgrad_sweep": (1, 4.0 * H * V * n_active, 2.0 * H * n_active + 4.0 * H * V + 2.0 * bias_b, 0.0),
        "fwd_compact_sweep": (2, 4.0 * H * V * n_active, 2.0 * H * n_active, 2.0 * H * V + bias_b),
    }
    per_launch = {}
    for name, (k, fl_step, bytes_step, bytes_per_launch) in kinds.items():
        if cnt[k] == 0:
            continue
        launches_step = cnt[k] / steps_f
        per_launch[name] = (fl_step / launches_step, bytes_step / launches_step + bytes_per_launch,
                            ms[k] / cnt[k], ms[k] / steps_f, int(cnt[k]))
    fwd_flops = sum(kinds[n][1] for n in ("fwd_sweep", "fwd_compact_sweep") if n in per_launch)
    wg_flops = kinds["wgrad_sweep"][1]
    dom = max(per_launch, key=lambda n: per_launch[n][3])
    flops, alg_bytes, avg_ms, _, n_launch = per_launch[dom]
    workload = spec.name + variant
    # the roof that binds is the one the algorithmic intensity falls under
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / alg_bytes >= ridge:
        achieved = flops / (avg_ms * 1e-3) / 1e12
        bound, peak, unit = "mfma", PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved = alg_bytes / (avg_ms * 1e-3) / 1e9
        bound, peak, unit = "hbm", PEAK_HBM_GBS, "GB/s"
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4),
                "traffic": _traffic_from_profiles(dom, workload),
                "alg_flop_per_launch": flops, "alg_bytes_per_launch": alg_bytes,
                "intensity_flop_per_byte": round(flops / alg_bytes, 1), "ridge_flop_per_byte": round(ridge, 1),
                "kernel": dom, "avg_launch_ms": round(avg_ms, 4),
                # the weight-gradient sweep's grad_W product alone (2HV per active
                # token), without the logits it recomputes
                "frac_grad_w_product_only": (round(0.5 * flops / (avg_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
                                             if dom == "wgrad_sweep" else None),
                "launches": n_launch,
                "sweep_ms_per_step": {n: round(v[3], 4) for n, v in per_launch.items()}}
    # the work the method itself does: the logits of every token (2HV) and
    # the two gradient products (2HV each) of the tokens with dL/dlogp != 0;
    # the 6NHV count charges the gradients of every token
    method_flops = 2.0 * H * V * (N + 2.0 * n_active)
    tflops_method = method_flops / (elapsed / args.steps) / 1e12
    line = {
        "metric": METRIC if not variant else METRIC.replace(
            "GMPO", spec.loss_type.upper() + (" (per-token advantages)" if tadv is not None else "")
            + (" (bias-corrected KL)" if spec.kl_bias_correction else "")),
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "tflops_6nhv": round(tflops, 2),
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "tflops_method_work": round(tflops_method, 2),
        "pct_bf16_peak_method_work": round(100.0 * tflops_method / PEAK_BF16_TFLOPS, 2),
        # what the path executes: the forward sweeps plus the weight-gradient
        # sweep's 4HV per token with a gradient (its logits are recomputed)
        "executed_tflops": round((fwd_flops + wg_flops) / (elapsed / args.steps) / 1e12, 2),
        "memory": {"inputs_bytes": int(mem_inputs), "workspace_bytes": int(ws.numel()),
                   "prepared_weight_bytes": int(wprep.numel()) if wprep is not None else 0,
                   "peak_bytes_beyond_inputs": int(peak_delta)},
        "config": {"workload": workload, "B": spec.B, "T": spec.T, "H": H, "V": V,
                   "loss_type": spec.loss_type, "bias": spec.bias, "beta": spec.beta,
                   "top_entropy_quantile": spec.top_entropy_quantile, "chunk_sequences": spec.chunk_sequences,
                   "token_advantages": tadv is not None, "kl_bias_correction": spec.kl_bias_correction,
                   "weight_prepared_outside_steps": wprep is not None,
                   "global_batch_tokens": N, "active_tokens_with_grad": n_active,
                   "event_ms_per_step": round(ev0.elapsed_time(ev1) / args.steps, 4)},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if flagged is not None:
        line["config"]["flagged_rows"] = flagged
    if not args.no_cpu_baseline and tadv is None:
        cb = _cpu_baseline(spec)
        # the whole workload at the sample's rate (not run: extrapolated)
        cb["extrapolated_full_workload_s"] = round(N / cb["value"], 1)
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
