/*
 * plp.h -- C ABI of the fused LM-head + GRPO-family policy loss for AMD
 * MI355X (gfx950).
 *
 * One hot path: hidden states h[N,H] and the LM-head weight W[V,H] (optional
 * bias b[V]) give the target-token log-probabilities and per-token entropies
 * through a streaming online log-sum-exp over vocabulary tiles (the
 * [N,V] logits are never stored), then the GMPO or GSPO-token objective with
 * an optional K3 KL penalty and an optional batch-global high-entropy token
 * mask, then grad_h, grad_W and grad_b.
 *
 * Definitions the entry points implement:
 *   - GMPO: Liger-Kernel PR #1320 "Add GMPO to fused linear GRPO loss",
 *     Summary and "The implementation" bullets (one-sided, advantage-dependent
 *     clipping of each token's log-ratio in log space [-eps_low, +eps_high];
 *     exp of the masked mean per completion; per-sample reduction; K3 KL;
 *     clipping metric; outer chunking; input/weight/bias gradients).
 *   - Streaming entropy and the high-entropy mask: Liger-Kernel PR #1558
 *     "support top_entropy_quantile", Details bullets (second accumulator
 *     sum exp(z-m)*z; H = log_z - sum_exp_z/sum_exp; threshold
 *     at 1-q of the active tokens' entropies, one per batch; the mask
 *     multiplies the policy term before the KL penalty; q validated to [0,1],
 *     q = 1 is the feature off).
 *   - GSPO-token: Tinker "GSPO" page, the sequence-ratio, per-token-ratio and
 *     objective equations, "Input tensors", "Output diagnostics" and
 *     "Choosing clipping thresholds".
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE memory owned by the caller. The library
 *     allocates nothing, never frees or retains a pointer after it returns,
 *     and uses only the caller's workspace (size from the matching
 *     *_workspace_size query; the workspace must be 256-byte aligned), except
 *     plp_entropy_quantile_mask_noalloc, whose scratch is a static device
 *     array of the library.
 *   - Calls only enqueue work on `stream`; outputs are valid once the stream
 *     has reached that point. Loss and metrics stay in device memory: no
 *     call synchronises with the host.
 *   - Every argument check happens on the host before any launch. On error
 *     nothing is enqueued, a negative PLP_E_* code is returned and
 *     plp_last_error() (thread-local) describes it.
 *   - Results are deterministic: the same inputs, sizes and build give
 *     bitwise-equal outputs (no floating-point atomics).
 *   - Calls from different host threads are safe when they use distinct
 *     workspaces; calls that share a workspace on overlapping streams race.
 *
 * Layouts: row-major. hidden [N,H] with the B sequences stored one after the
 * other, T rows each (row n = i*T + t); weight [V,H] (nn.Linear layout);
 * per-token arrays [N]; advantages [B]. hidden, weight, bias and the
 * gradient outputs must be 16-byte aligned (the kernels move 16-byte
 * chunks); a misaligned one is rejected with PLP_E_INVALID.
 */
#ifndef PLP_H
#define PLP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PLP_API __attribute__((visibility("default")))
#define PLP_ABI_VERSION 5

/* Return codes. */
#define PLP_OK 0
#define PLP_E_INVALID (-1)      /* bad shape, NULL where required, value out of range */
#define PLP_E_UNSUPPORTED (-2)  /* a combination the method excludes */
#define PLP_E_WORKSPACE (-3)    /* workspace NULL, misaligned or too small */
#define PLP_E_HIP (-4)          /* a HIP launch or runtime call failed */

typedef enum { PLP_DTYPE_F32 = 0, PLP_DTYPE_BF16 = 1 } plp_dtype;

/* GMPO: Liger PR #1320. GSPO_TOKEN: Tinker GSPO page (GSPO-token variant).
 * GRPO, BNPO, DAPO: the token-level clipped surrogate that Liger PR #1558
 * (Testing) and PR #1320 (Testing) name as loss types without printing it,
 * read as the Tinker GSPO page's objective with each token's own ratio
 * rho_t = exp(lp_t - old_t): per completion token
 * -min(rho_t A_i, clip(rho_t, 1-eps_low, 1+eps_high) A_i), a token held at a
 * bound passing no gradient (the predicate is exp(fp32(lp - old)) in fp64
 * against fp32(1-eps_low) and fp32(1+eps_high); ties are not clipped). They
 * differ only in the divisor of the token sum: GRPO the per-sample reduction
 * (masked mean per sequence, mean over B); BNPO the number of completion
 * tokens of the batch; DAPO args->global_tokens when > 0 (a count over a
 * larger accumulated batch), else the same as BNPO. The `reduction` field
 * does not apply to them; the ratio mask plays no part. */
typedef enum {
  PLP_LOSS_GMPO = 0,
  PLP_LOSS_GSPO_TOKEN = 1,
  PLP_LOSS_GRPO = 2,
  PLP_LOSS_BNPO = 3,
  PLP_LOSS_DAPO = 4
} plp_loss_type;

/* Importance-sampling level. GMPO rejects SEQUENCE (PR #1320: it clips at
 * token level before the sequence aggregation); GSPO_TOKEN is inherently a
 * sequence-level ratio and takes SEQUENCE; GRPO, BNPO and DAPO take TOKEN
 * (their sequence-level form is GSPO_TOKEN). */
typedef enum { PLP_IS_TOKEN = 0, PLP_IS_SEQUENCE = 1 } plp_is_level;

/* SEQ_MEAN: masked mean over each sequence's completion tokens, then the mean
 * over the B sequences (the per-sample reduction PR #1320 reuses).
 * TOKEN_SUM: plain sum over completion tokens (the Tinker page's loss:sum).
 * For GMPO and GSPO_TOKEN only. */
typedef enum { PLP_REDUCE_SEQ_MEAN = 0, PLP_REDUCE_TOKEN_SUM = 1 } plp_reduction;

/* Metrics layout (fp32, PLP_NUM_METRICS entries). */
enum {
  PLP_M_CLIP_FRACTION = 0,        /* clipped completion tokens / completion tokens (GSPO: a
                                     sequence's verdict counts for each of its tokens; GRPO,
                                     BNPO, DAPO: tokens whose ratio is held at a bound) */
  PLP_M_SEQ_LOG_RATIO_MEAN = 1,   /* mean over sequences of mean_{ratio tokens} (lp - old) */
  PLP_M_CLIPPED_SEQ_FRACTION = 2, /* GSPO: share of sequences whose ratio left the clip range
                                     (either side); other loss types: 0 */
  PLP_M_MEAN_KL = 3,              /* mean over sequences of the masked-mean K3 KL (0 without ref) */
  PLP_M_ENTROPY_THRESHOLD = 4,    /* batch-global entropy threshold; NaN when q = 1 or no
                                     completion token */
  PLP_M_ENTROPY_KEPT_FRACTION = 5,/* completion tokens kept by the entropy mask / completion tokens */
  PLP_M_ACTIVE_TOKENS = 6,        /* number of completion tokens */
  PLP_M_CLIPPED_TOKENS = 7,       /* number of clipped completion tokens */
  PLP_NUM_METRICS = 8
};

/* Inputs of the fused call. Versioned by struct_size (set it to
 * sizeof(plp_args)); fields are only ever appended, and a struct_size that
 * ends before an appended field leaves that field at its default. */
typedef struct plp_args {
  uint32_t struct_size;
  int32_t dtype;                /* plp_dtype of hidden, weight, bias and the gradients */
  int64_t B, T;                 /* sequences, tokens per sequence; N = B*T rows */
  int32_t H, V;                 /* hidden size, vocabulary size */
  const void* hidden;           /* [N,H] dtype */
  const void* weight;           /* [V,H] dtype */
  const void* bias;             /* [V] dtype, or NULL */
  const int64_t* targets;       /* [N] token ids in [0,V) */
  const float* old_logp;        /* [N] sampler log-probs, or NULL = on-policy (log-ratio 0) */
  const float* ref_logp;        /* [N] KL reference log-probs; required iff beta != 0 */
  const uint8_t* completion_mask; /* [N] nonzero = token enters the loss */
  const uint8_t* ratio_mask;    /* [N] nonzero = token enters the sequence ratio and clip;
                                   NULL = completion_mask (Tinker: sequence_ratio_mask) */
  const float* advantages;      /* [B] per-sequence advantage (NULL when token_advantages is given) */
  int32_t loss_type;            /* plp_loss_type */
  int32_t is_level;             /* plp_is_level */
  int32_t reduction;            /* plp_reduction */
  int32_t pad0;
  double epsilon_low;           /* GMPO: log-space lower bound -eps_low; GSPO: ratio 1-eps_low */
  double epsilon_high;          /* GMPO: log-space upper bound +eps_high; GSPO: ratio 1+eps_high */
  double beta;                  /* K3 KL weight (>= 0) */
  double temperature;           /* logits are divided by it (> 0) */
  double top_entropy_quantile;  /* q in [0,1]; 1 = no entropy mask */
  int64_t chunk_sequences;      /* outer chunk in whole sequences; 0 = all B at once */
  /* ---- ABI version 2 ---- */
  int64_t global_tokens;        /* DAPO divisor (>= 0); 0 = the batch's completion tokens.
                                   Ignored by the other loss types. Default 0. */
  const float* token_advantages;/* [N] one advantage per token (Tinker GSPO page, "Input
                                   tensors": advantages (N,)), or NULL (default) to use
                                   `advantages` [B]. When given, `advantages` is ignored and may
                                   be NULL; each token's min(ratio A_t, clip(ratio) A_t) takes its
                                   own A_t, so the clip binds per token by the sign of A_t.
                                   GSPO_TOKEN, GRPO, BNPO and DAPO only (GMPO's clip direction
                                   and geometric mean are per sequence: PLP_E_UNSUPPORTED). */
  /* ---- ABI version 3 ---- */
  int32_t kl_bias_correction;   /* nonzero: bias-corrected KL (Liger PR #1320, "The implementation"):
                                   each token's K3 term is multiplied by its importance ratio
                                   rho_t = exp(logp_t - old_logp_t), which is differentiated
                                   through, so dKL_t/dlogp_t = rho_t (logp_t - ref_logp_t).
                                   Without old_logp rho_t = 1 in value, its derivative still
                                   taken. The mean_kl metric reports the corrected term. Only
                                   read when beta != 0 or ref_logp is given. Default 0. */
  int32_t pad1;
  /* ---- ABI version 4 ---- */
  const void* weight_prepared;  /* the matrix-core copy of `weight` that plp_prepare_weight
                                   made from its current values, or NULL (default): the call
                                   then makes that copy itself, in its workspace. Given, the
                                   call reads the weight's tiles from it and skips the copy,
                                   and the workspace it needs shrinks by that copy's size; the
                                   caller keeps it in step with `weight` (prepare again after
                                   every change of the weight, e.g. once per optimizer step
                                   for all the micro-batches of a gradient accumulation).
                                   `weight` is still required: the target logit, the exact
                                   recompute and nothing else read it. bf16 with H a multiple
                                   of 128 up to 896 only (PLP_E_UNSUPPORTED otherwise);
                                   16-byte aligned. */
} plp_args;

/* Outputs of the fused call. Every pointer except loss and metrics may be
 * NULL to skip that output. Gradients have the input dtype. */
typedef struct plp_outputs {
  uint32_t struct_size;
  uint32_t pad0;
  float* loss;                  /* [1] */
  float* metrics;               /* [PLP_NUM_METRICS] */
  void* grad_hidden;            /* [N,H] */
  void* grad_weight;            /* [V,H] */
  void* grad_bias;              /* [V]; requires bias != NULL */
  float* logp_out;              /* [N] target log-probs */
  float* entropy_out;           /* [N] entropies */
  uint8_t* entropy_mask_out;    /* [N] 1 = kept by the entropy mask (all completion tokens when q=1) */
  float* dlogp_out;             /* [N] dL/dlogp */
} plp_outputs;

/* Version of this ABI (PLP_ABI_VERSION). */
PLP_API int plp_abi_version(void);

/* Message for the last non-zero return on this thread ("" if none). */
PLP_API const char* plp_last_error(void);

/* Workspace bytes needed by plp_fused_lmhead_policy_loss_fwd_bwd for these
 * arguments (only sizes, dtype, the NULL-ness of bias and weight_prepared, q
 * and chunk_sequences are read; pointers may be NULL). Host-only arithmetic:
 * needs no GPU. */
PLP_API int plp_workspace_size(const plp_args* args, size_t* bytes);

/* The whole path: forward statistics, entropy mask (q < 1), loss, metrics and
 * the gradients asked for in `out` (Liger PR #1320 fused linear GMPO; PR
 * #1558 entropy masking; Tinker GSPO-token). Outer chunks of
 * chunk_sequences whole sequences bound the per-chunk workspace; the entropy
 * threshold and the batch mean are global, so results do not depend on the
 * chunk size beyond rounding. Errors: PLP_E_INVALID (shapes, NULLs, q outside
 * [0,1], beta != 0 without ref_logp, temperature <= 0, negative eps or beta,
 * chunk_sequences < 0, global_tokens < 0), PLP_E_UNSUPPORTED (GMPO, GRPO,
 * BNPO or DAPO with SEQUENCE importance sampling; GSPO_TOKEN with TOKEN),
 * PLP_E_WORKSPACE, PLP_E_HIP. */
PLP_API int plp_fused_lmhead_policy_loss_fwd_bwd(const plp_args* args, const plp_outputs* out,
                                                 void* workspace, size_t workspace_bytes,
                                                 hipStream_t stream);

/* The weight's copy in the layout the matrix-core sweeps stream (Liger PR
 * #1320, "The implementation": the LM-head weight is read tile by tile in
 * the forward and again in the backward; this is the layout of those tiles):
 * 32-row tiles, each the four quarter-width column slices one after the
 * other, each slice in 16-column steps of 64 lanes x 8 bf16 (lane l: row
 * l % 32, columns 8 (l / 32) .. +7 of the step); rows past V up to a multiple
 * of 64 are zero. Layout and size are private to this library version; the
 * copy is only meant as plp_args.weight_prepared of calls on the same weight
 * values. plp_prepared_weight_size gives its bytes (host arithmetic; no GPU);
 * plp_prepare_weight writes it from weight [V,H] bf16 into `prepared`
 * (caller-owned device memory of at least that size, 256-byte aligned),
 * enqueued on `stream`. bf16 with H a multiple of 128 up to 896 only
 * (otherwise PLP_E_UNSUPPORTED); NULL or misaligned pointers, a short
 * buffer, V < 1: PLP_E_INVALID. */
PLP_API int plp_prepared_weight_size(int32_t H, int32_t V, int32_t dtype, size_t* bytes);
PLP_API int plp_prepare_weight(const void* weight, int32_t H, int32_t V, int32_t dtype, void* prepared,
                               size_t prepared_bytes, hipStream_t stream);

/* Streaming entropy and target log-prob over vocabulary tiles without
 * storing logits (PR #1558 "_selective_entropy_forward": running (m, sum
 * exp(z-m), sum exp(z-m) z), rescaled when the max moves;
 * H = log_z - sum_exp_z/sum_exp). hidden [N,H], weight [V,H], bias [V] or
 * NULL, all of `dtype`. targets [N] or NULL (then logp_out must be NULL).
 * entropy_out [N] fp32 (required), logp_out [N] fp32 or NULL. */
PLP_API int plp_selective_entropy_workspace_size(int64_t N, int32_t H, int32_t V, int32_t dtype,
                                                 size_t* bytes);
PLP_API int plp_selective_entropy(const void* hidden, const void* weight, const void* bias,
                                  int64_t N, int32_t H, int32_t V, int32_t dtype, float temperature,
                                  const int64_t* targets, float* entropy_out, float* logp_out,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* plp_selective_entropy on a weight whose matrix-core copy the caller made
 * with plp_prepare_weight (ABI version 5), for the no-grad passes between two
 * weight updates (PR #1558, Details: the entropy pre-pass runs over the same
 * LM-head weight as the loss that follows): the call reads weight_prepared
 * instead of making that copy, so its workspace
 * (plp_selective_entropy_prepared_workspace_size) has no copy of W. weight
 * [V,H] is still read (target logits, flagged rows) and must hold the values
 * weight_prepared was made from; the results are bit-identical to
 * plp_selective_entropy's. bf16 with H a multiple of 128 up to 896 only
 * (otherwise PLP_E_UNSUPPORTED); weight_prepared NULL or not 16-byte aligned:
 * PLP_E_INVALID; other arguments and errors as for plp_selective_entropy. */
PLP_API int plp_selective_entropy_prepared_workspace_size(int64_t N, int32_t H, int32_t V, int32_t dtype,
                                                          size_t* bytes);
PLP_API int plp_selective_entropy_prepared(const void* hidden, const void* weight, const void* weight_prepared,
                                           const void* bias, int64_t N, int32_t H, int32_t V, int32_t dtype,
                                           float temperature, const int64_t* targets, float* entropy_out,
                                           float* logp_out, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream);

/* Batch-global high-entropy mask (PR #1558, Details bullet 2):
 * thr = quantile(entropy[active], 1 - q) with torch.quantile's linear
 * interpolation evaluated in fp32; mask_out[n] = active[n] && entropy[n] >= thr.
 * No active entry: all-zero mask and thr = NaN. q = 1: mask = active, thr = NaN.
 * entropy [N] fp32, active [N] u8, mask_out [N] u8, threshold_out [1] fp32
 * (may be NULL). q outside [0,1] -> PLP_E_INVALID. */
PLP_API int plp_entropy_quantile_mask_workspace_size(int64_t N, size_t* bytes);
PLP_API int plp_entropy_quantile_mask(const float* entropy, const uint8_t* active, int64_t N, double q,
                                      uint8_t* mask_out, float* threshold_out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* The same mask without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Arguments, results and errors as for
 * plp_entropy_quantile_mask. The select state (16.4 KB) lives in a static
 * device array of 32 KB that the library holds on every device that runs the
 * call until the process ends; its address is looked up once per device on
 * the first call there. The call allocates nothing and enqueues on `stream`
 * (on the stream's device). The scratch does not grow with N, so the largest
 * input is the ABI's N < 2^31 (larger N: PLP_E_INVALID). Every call on one
 * device shares that device's array and resets it first: calls that overlap
 * on one device (concurrent streams, or threads) race and give wrong results.
 * PLP_E_HIP when the stream's device or the array's address cannot be
 * obtained. */
PLP_API int plp_entropy_quantile_mask_noalloc(const float* entropy, const uint8_t* active, int64_t N, double q,
                                              uint8_t* mask_out, float* threshold_out, hipStream_t stream);

/* The loss stage alone, from given per-token log-probs (the GMPO / GSPO-token
 * / GRPO / BNPO / DAPO / K3 KL objective without the LM head). args: as for the fused
 * call; hidden, weight, bias and targets are ignored, H and V may be 0.
 * logp [N] fp32. entropy [N] fp32 is required iff top_entropy_quantile < 1.
 * out: loss and metrics required; dlogp_out and entropy_mask_out optional;
 * the gradient, logp_out and entropy_out pointers are ignored. */
PLP_API int plp_policy_loss_workspace_size(const plp_args* args, size_t* bytes);
PLP_API int plp_policy_loss_from_logprobs(const plp_args* args, const float* logp, const float* entropy,
                                          const plp_outputs* out, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/* ---- Measurement helpers (not part of the method) -------------------------
 * Per-kernel timing of the two LM-head sweeps with HIP events recorded on the
 * stream of each call, for benchmarks and roofline reports.
 * plp_profile_start(max_records): pre-creates 2*max_records events and turns
 * recording on (PLP_E_INVALID if max_records < 1; PLP_E_HIP if event creation
 * fails). While on, every forward sweep over all rows of a chunk (kind 0),
 * weight-gradient sweep (kind 1) and, with the entropy mask, accumulator
 * pass over the compacted rows with a gradient (kind 2) is bracketed by an
 * event pair, up to max_records pairs. plp_profile_stop_n(ms[n], count[n],
 * n >= 2): waits for the recorded events, returns per kind the summed
 * milliseconds and the number of launches (with n = 2, kind 2 counts as kind
 * 0), destroys the events and turns recording off; plp_profile_stop(ms[2],
 * count[2]) is plp_profile_stop_n with n = 2. Process-global; not for
 * concurrent use. */
PLP_API int plp_profile_start(int32_t max_records);
PLP_API int plp_profile_stop(double* ms_out, int32_t* count_out);
PLP_API int plp_profile_stop_n(double* ms_out, int32_t* count_out, int32_t n_kinds);

#ifdef __cplusplus
}
#endif

#endif /* PLP_H */
