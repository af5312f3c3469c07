// Shared types and launcher declarations of the plp HIP library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace plp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Per (vocabulary split, row) result of the forward sweep: the reference m
// all exponentials are taken against, the largest logit zmax of the split,
// sum exp(z-m), sum exp(z-m) z, and a flag: a logit above m + 64, whose
// exponential the sweep clamped, so the row's statistics are to be taken
// again against its true maximum.
struct alignas(8) RowStats {
  double m;     // the reference, in natural units of the logits
  double s;
  double sz;
  float zmax;
  int flag;
};

// Per compacted token, what the weight-gradient sweep needs.
struct alignas(16) TokData {
  float lse;   // log-sum-exp of the token's logits
  float gs;    // dL/dlogp / temperature
  int y;       // target id
  int pad;
};

// Loss and metric accumulators carried across outer chunks (fp64 sums,
// integer counts) so the batch-level values are chunk independent.
struct LossAcc {
  double loss;
  double slr;          // sum over sequences of the mean ratio-token log-ratio
  double mkl;          // sum over sequences of the masked-mean KL
  unsigned long long n_active, n_clip, n_kept, n_clipseq;
  float thr;
  int pad;
};

// Per-sequence partial sums of the loss stage.
struct SeqPart {
  double sum_c;        // GMPO: sum over ratio tokens of the clipped log-ratio;
                       // token-clip losses: sum over kept completion tokens of the policy term
  double sum_lr;       // sum over ratio tokens of the log-ratio
  double sum_kl;       // sum over completion tokens of the K3 KL
  double sum_apos, sum_aneg;  // GSPO with per-token advantages: sums of A_t > 0 / A_t < 0 over kept
                              // completion tokens
  int cnt_m, cnt_r, cnt_k, cnt_clip;
  int cnt_pos, cnt_neg;       // completion tokens with A_t > 0 / A_t < 0 (per-token advantages)
};

// Per-sequence coefficients of dL/dlogp.
struct SeqCoef {
  double pol;          // policy-term coefficient applied to eligible tokens
  double wbeta;        // w_i * beta
  float adv;
  int pad;
};

struct LossParams {
  int64_t B_total;     // batch size dividing the per-sample reduction
  int64_t T;
  int loss_type;       // plp_loss_type: 0 GMPO, 1 GSPO_TOKEN, 2 GRPO, 3 BNPO, 4 DAPO
  int reduction;       // GMPO / GSPO: 0 seq mean, 1 token sum
  float eh32, el32;    // fp32(eps_high), fp32(eps_low)
  float lo32, hi32;    // ratio bounds fp32(1-eps_low), fp32(1+eps_high) (GSPO and the token-clip losses)
  double beta;
  int64_t norm_tokens; // BNPO / DAPO divisor when > 0 (DAPO's global count)
  const unsigned long long* ntok_dev;  // else: the batch's completion-token count (device)
  int token_adv;       // advantages are per token (the kernels' tadv argument)
  int kl_bc;           // KL term weighted by the token importance ratio
};

// Vocabulary splits of the forward sweep over `rows` token rows (64-row
// blocks x Sv contiguous vocabulary ranges, one workgroup each, one
// workgroup per compute unit): the Sv in [1, max_splits] (max_splits <= 64;
// every split holding at least one 32-row tile) with the shortest estimated
// time for a 4096-tile vocabulary, counted in hundredths of one workgroup's
// tile: ceil(blocks x Sv / 256) rounds of ceil(4096 / Sv) tiles, plus the
// split accumulators' write and merge, about 0.07 tile per row block and
// split (64 rows x H fp32 written and read again, against one tile's
// 64 x 32 x H x 4 matrix FLOP at the measured rates). The reference
// vocabulary keeps the choice, and so the workspace, a function of the row
// count alone (V only bounds Sv by its tile count). More than one split is
// taken only while row blocks x splits stay within kMaxSplitBlocks (four
// rounds), which bounds the split accumulators of a pass whose count lives on
// the device at 1024 x 64 rows. forward_split_key orders
// the candidates (time, then the smaller Sv); the host takes the least key in
// a loop, a wave on the device in one lane per candidate, so both pick the
// same Sv.
constexpr int64_t kMaxSplitBlocks = 1024;
__host__ __device__ inline unsigned long long forward_split_key(int64_t rows, int V, int max_splits, int sv) {
  const int64_t nrb = (rows + 63) / 64;
  const int n_tiles = (V + 31) / 32;
  if (sv < 1 || sv > max_splits || sv > n_tiles) return ~0ull;
  if (sv > 1 && nrb * sv > kMaxSplitBlocks) return ~0ull;  // bounds the split accumulators
  const int tps = (n_tiles + sv - 1) / sv;
  if ((n_tiles + tps - 1) / tps != sv) return ~0ull;  // a split would hold no tile
  const unsigned long long t = (unsigned long long)((nrb * sv + 255) / 256) * (unsigned long long)((4096 + sv - 1) / sv) *
                                   100ull +
                               7ull * (unsigned long long)(nrb * sv);
  return (t << 8) | (unsigned long long)sv;
}
// Largest Sv that can beat one split at nrb row blocks: one split costs at
// most 1600 nrb + 408000 + 7 nrb, any Sv at least 1600 nrb + 7 nrb Sv, so only
// nrb (Sv - 1) < 58286 can win; larger candidates need not be evaluated.
inline int forward_splits_useful(int64_t nrb) { return nrb < 1 ? 64 : (int)std::min<int64_t>(64, 1 + 58285 / nrb); }
inline int forward_splits(int64_t rows, int V, int max_splits) {
  unsigned long long best = ~0ull;
  const int top = forward_splits_useful((rows + 63) / 64);
  for (int sv = 1; sv <= top; ++sv) {
    const unsigned long long k = forward_split_key(rows, V, max_splits, sv);
    if (k < best) best = k;
  }
  return best == ~0ull ? 1 : (int)(best & 255ull);
}
// The same choice by one wave (all 64 lanes active, uniform arguments).
__device__ inline int forward_splits_wave(int64_t rows, int V, int max_splits) {
  unsigned long long k = forward_split_key(rows, V, max_splits, (int)(threadIdx.x & 63) + 1);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(k, off, 64);
    k = o < k ? o : k;
  }
  // the same in every lane: made scalar, so that what derives from it stays
  // in scalar registers
  return __builtin_amdgcn_readfirstlane(k == ~0ull ? 1 : (int)(k & 255ull));
}

// Largest number of (row block, split) pairs the sweep uses for any row
// count up to `rows` (the grid of a launch whose count lives on the device;
// the rows of its statistics are 64 times this). Host only; remembers its
// last few answers.
int64_t forward_blocks_max(int64_t rows, int V, int max_splits);

// Workgroup -> (row block, split) of the forward sweeps. Workgroup w runs on
// XCD w % 8; each XCD takes a contiguous range of the split-major order of
// the nrb x Sv blocks, so its compute units stream one vocabulary range of W
// together and share its tiles in their L2. Returns false for a workgroup
// with no block (grids are rounded up to a multiple of 8, or sized for the
// largest count).
__device__ inline bool forward_block(int64_t nrb, int Sv, int64_t& rb, int& sv) {
  // 32-bit arithmetic: grids stay below 2^31 workgroups
  const int nb = (int)nrb, total = nb * Sv, per = (total + 7) / 8;
  const int j = (int)(blockIdx.x / 8);
  const int g = (int)(blockIdx.x % 8) * per + j;
  if (j >= per || g >= total) return false;
  sv = g / nb;
  rb = g - sv * nb;
  return true;
}

// Token-level clipped losses (GRPO, BNPO, DAPO) share the per-token path.
__host__ __device__ inline bool token_clip_loss(int loss_type) { return loss_type >= 2; }
// Losses whose divisor is a token count rather than per-sample.
__host__ __device__ inline bool token_mean_loss(int loss_type) { return loss_type == 3 || loss_type == 4; }

// ---------------------------------------------------------------------------
// Launchers (each enqueues on `st`; return hipError_t of the launch)
// ---------------------------------------------------------------------------

// The bias as the accumulator sweep reads it: out[v] = fp32(b[v]) for v < V
// and 0 up to the next multiple of 64 (bias_f32_len(V) floats), so that a
// lane takes four rows with one 16-byte load and no bf16 unpacking.
hipError_t launch_bias_f32(const __bf16* b, int V, float* out, hipStream_t st);
inline int64_t bias_f32_len(int V) { return ((int64_t)V + 63) / 64 * 64; }

// Fragment-major copy of bf16 rows for the MFMA sweeps (the layout is given
// in mfma_tile.h): `tiles` 32-row tiles of X, or of X[idx[k]] when idx is
// given; rows at or past `rows` (*count_dev when given) are zero.
hipError_t launch_frag_copy(const __bf16* X, const int* idx, const int* count_dev, int64_t rows, int64_t tiles, int H,
                            __bf16* Xf, hipStream_t st);

// Forward sweep on MFMA (bf16, H a multiple of 128, H <= 896); Wf is the
// fragment-major copy of W; the bias, when there is one, comes as its fp32
// copy b32 (launch_bias_f32, read by the accumulator sweep) and as the
// caller's bf16 b16 (read by the statistics-only sweep), both or neither.
// With count_dev (an accumulator pass over a
// compacted row list, with_o only) the sweep runs over the first
// min(*count_dev, N) rows of h, or with row_idx over rows row_idx[k] of h
// (N is the list's capacity), with
// forward_splits(that count, V, Sv) splits, and stats / O use the row stride
// compact_stride(that count). With mref (natural-log units of the logits,
// row k's at mref[k * mref_stride]) every row takes its exponentials against
// that reference instead of its first tile's maximum; a reference at or
// above the row's largest logit leaves nothing to flag. clear_count (or
// NULL; not count_dev) is set to zero by the sweep, for a launch_flag_scan
// after it.
hipError_t launch_fwd_mfma(const __bf16* h, const __bf16* Wf, const float* b32, const __bf16* b16, int64_t N, int H,
                           int V, float inv_tau, int Sv, bool with_o, RowStats* stats, float* O, hipStream_t st,
                           const int* count_dev = nullptr, const float* mref = nullptr, int mref_stride = 1,
                           const int* row_idx = nullptr, int* clear_count = nullptr);
// Row stride of the compacted pass's stats and O (whole 64-row blocks).
__host__ __device__ inline int64_t compact_stride(int64_t rows) { return (rows + 63) / 64 * 64; }
// grad_h of the compacted rows k < *count_dev from the compacted pass:
// grad_h[idx[k]] = tok[k].gs (W_y - O/s) with y = tok[k].y (flagged rows
// recomputed exactly from h row idx[k]); the other rows are left as they are.
hipError_t launch_grad_h_compact(int dtype, const RowStats* stats, const float* O, int max_splits, int64_t cap, int H,
                                 int V, const void* h, const void* W, const void* b, float inv_tau, const int* idx,
                                 const TokData* tok, const int* count_dev, void* gh, hipStream_t st);

// Weight-gradient sweep on MFMA over the compacted tokens
// [tok_begin, tok_begin + tok_len) of the *count_dev (hcf and Wf are
// fragment-major; tok_begin a multiple of 32; hcf and tok point at token 0).
// tail_scratch (bwd_tail_scratch_floats(H) floats, or NULL to keep every
// vocabulary block in one workgroup) holds the fp32 partial sums of the
// blocks whose token tiles are split over several workgroups.
hipError_t launch_bwd_mfma(const __bf16* Wf, const __bf16* b, const __bf16* hcf, const TokData* tok,
                           const int* count_dev, int tok_begin, int tok_len, int H, int V, float inv_tau, int acc_mode,
                           float* gW_acc, float* gb_acc, __bf16* gW_out, __bf16* gb_out, float* tail_scratch,
                           hipStream_t st);
size_t bwd_tail_scratch_floats(int H);

// Generic (VALU) forward and weight-gradient sweeps for any H and fp32 or bf16.
hipError_t launch_fwd_generic(int dtype, const void* h, const void* W, const void* b, const int64_t* y,
                              int64_t N, int H, int V, float inv_tau, bool with_o, RowStats* stats,
                              float* O, hipStream_t st);
hipError_t launch_bwd_generic(int dtype, const void* W, const void* b, const void* hc,
                              const TokData* tok, const int* count_dev, int H, int V, float inv_tau,
                              int acc_mode, float* gW_acc, float* gb_acc, void* gW_out, void* gb_out,
                              hipStream_t st);

// The second forward pass over the rows the first one flagged: up to cap of
// them, listed by launch_flag_scan (idx, their largest logit mref, *count,
// and pos[row] = the row's place in the list or -1), taken again by the
// accumulator sweep against mref into stats / O (compacted layout, at most
// max_splits vocabulary splits).
struct FlaggedPass {
  int* idx;
  float* mref;
  int* pos;
  int* count;
  RowStats* stats;
  float* O;
  int cap;
  int max_splits;
};
// *count must be zero when the scan starts (the forward sweep before it
// clears it, see clear_count).
hipError_t launch_flag_scan(const RowStats* stats, int Sv, int64_t N, int cap2, int* idx, float* mref, int* pos,
                            int* count, hipStream_t st);

// Merge vocabulary splits: lp, H, lse per row and (when vout != NULL)
// v = W_y - sum_v p W_v as fp32 [N,H] (grad_h = g / tau * v). Rows listed
// by a second pass (fp) are merged from its results; rows still flagged are
// recomputed here from h, W, b with an exact online max.
hipError_t launch_combine(int dtype, const RowStats* stats, const float* O, int Sv, int64_t N, int H, int V,
                          const void* h, const void* W, const void* b, float inv_tau, const int64_t* y,
                          float* lp, float* ent, float* lse, float* vout, hipStream_t st,
                          const FlaggedPass* fp = nullptr);

// Loss stage (per outer chunk): per-sequence partial sums, the per-sequence
// merge (accumulators set on the first chunk; loss and metrics written on the
// last, with the threshold from thr_dev or NaN), then per-token dL/dlogp with
// per-32-token counts of nonzero gradients and grad_h = g / tau * v (gh and v
// may be NULL), and the in-order compaction of the tokens with g != 0.
// adv: per-sequence advantages [Bc]; tadv: per-token advantages [Bc*T] (used
// instead of adv when p.token_adv).
hipError_t launch_loss_seq_partial(const LossParams& p, int64_t Bc, const float* lp, const float* old,
                                   const float* ref, const uint8_t* comp, const uint8_t* ratio,
                                   const uint8_t* emask, const float* adv, const float* tadv, int St,
                                   SeqPart* part, hipStream_t st);
hipError_t launch_loss_seq_final(const LossParams& p, int64_t Bc, int St, const SeqPart* part, const float* adv,
                                 SeqCoef* coef, LossAcc* acc, bool init, const float* thr_dev, float* loss_out,
                                 float* metrics, hipStream_t st);
hipError_t launch_loss_tokens(int dtype, const LossParams& p, int64_t Bc, const float* lp, const float* old,
                              const float* ref, const uint8_t* comp, const uint8_t* ratio, const uint8_t* emask,
                              const float* tadv, const SeqCoef* coef, float* g, int* cnt32, const float* v, int H,
                              float inv_tau, void* gh, hipStream_t st);
size_t compact_scratch_bytes(int64_t N);
hipError_t launch_compact_scatter(const float* g, const float* lse, const int64_t* y, int64_t N, float inv_tau,
                                  const int* cnt32, int* idx, TokData* tok, int* count_dev, hipStream_t st);
hipError_t launch_gather_rows(int dtype, const void* X, const int* idx, const int* count_dev, int64_t cap,
                              int H, void* Xc, hipStream_t st);

// Entropy quantile mask: the radix select's state and histogram (the
// threshold first, so the later kernels read it as a float).
struct SelectState {
  float thr;                 // the threshold; NaN when no entry is active
  float w;                   // interpolation weight rank - floor(rank)
  unsigned pre[2];           // key prefixes of the two order statistics found so far
  unsigned long long n;      // active entries
  unsigned long long kk[2];  // ranks left within the current prefixes
  int done;                  // no active entry: the remaining passes do nothing
  int pad;
  unsigned hist[2][2048];    // digit histogram of the current pass (one per order statistic)
};
hipError_t launch_entropy_select(const float* ent, const uint8_t* active, int64_t N, float p32, SelectState* state,
                                 hipStream_t st);
hipError_t launch_entropy_mask(const float* ent, const uint8_t* active, int64_t N, const float* thr_dev,
                               uint8_t* mask, hipStream_t st);
hipError_t launch_store_thr(const float* thr_dev, float* thr_out, hipStream_t st);
// Number of nonzero bytes of m[0, N) into *out (one block, fixed order).
hipError_t launch_count_mask(const uint8_t* m, int64_t N, unsigned long long* out, hipStream_t st);
hipError_t launch_copy_mask(const uint8_t* src, int64_t N, uint8_t* dst, hipStream_t st);
hipError_t launch_set_nan(float* dst, hipStream_t st);

}  // namespace plp
