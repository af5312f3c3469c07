// Host side of the plp C ABI: argument checks, workspace planning and the
// order of the device passes. No allocation, no host synchronisation.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/plp.h"
#include "common.h"

using namespace plp;

int64_t plp::forward_blocks_max(int64_t rows, int V, int max_splits) {
  // the answers of the last few (rows, V, max_splits), per thread: the loop
  // runs up to rows / 64 x 64 key evaluations
  struct Memo {
    int64_t rows;
    int V, max_splits;
    int64_t blocks;
  };
  thread_local Memo memo[8] = {};
  thread_local int next = 0;
  for (const Memo& m : memo)
    if (m.blocks > 0 && m.rows == rows && m.V == V && m.max_splits == max_splits) return m.blocks;
  // several splits only while blocks x splits <= kMaxSplitBlocks, so past
  // that many row blocks the count of blocks is the row blocks themselves
  const int64_t nrb_cap = (rows + 63) / 64;
  int64_t best = nrb_cap;
  for (int64_t nrb = 1; nrb <= std::min<int64_t>(nrb_cap, kMaxSplitBlocks); ++nrb)
    best = std::max<int64_t>(best, nrb * forward_splits(nrb * 64, V, max_splits));
  memo[next] = Memo{rows, V, max_splits, best};
  next = (next + 1) % 8;
  return best;
}

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return PLP_OK;
}

constexpr size_t kAlign = 256;
constexpr int kBQ = 64, kBK = 32;
constexpr int kMaxSplits = 64;
// Rows of the second forward pass over flagged rows per call of the sweep
// (more flagged rows than this are recomputed by the merge on the vector
// ALU); its statistics and accumulator hold compact_rows_needed rows.
constexpr int64_t kFlagCap = 32768;
constexpr int64_t kMaxRows = (int64_t)1 << 31;
// plp_args as of ABI version 1 (fields up to chunk_sequences); later fields
// read as their defaults when struct_size ends before them.
constexpr size_t kArgsV1Size = offsetof(plp_args, global_tokens);

int64_t global_tokens(const plp_args* a) {
  return a->struct_size >= offsetof(plp_args, global_tokens) + sizeof(int64_t) ? a->global_tokens : 0;
}

const float* token_advantages(const plp_args* a) {
  return a->struct_size >= offsetof(plp_args, token_advantages) + sizeof(void*) ? a->token_advantages : nullptr;
}

int kl_bias_correction(const plp_args* a) {
  return a->struct_size >= offsetof(plp_args, kl_bias_correction) + sizeof(int32_t) && a->kl_bias_correction ? 1 : 0;
}

const void* weight_prepared(const plp_args* a) {
  return a->struct_size >= offsetof(plp_args, weight_prepared) + sizeof(void*) ? a->weight_prepared : nullptr;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Rows of stats / O a compacted accumulator pass over at most `cap` listed
// rows can use: the largest splits x row stride the sweep picks for any
// count up to cap (both depend on the count through its 64-row blocks only).
int64_t compact_rows_needed(int64_t cap, int V, int max_splits) { return 64 * forward_blocks_max(cap, V, max_splits); }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Sequential carving of the caller's workspace.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t count) {
    if (count == 0) return nullptr;
    T* p = base ? (T*)(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return p;
  }
};

bool mfma_eligible(int dtype, int H) { return dtype == PLP_DTYPE_BF16 && H % 128 == 0 && H >= 128 && H <= 896; }
bool generic_eligible(int H) { return H >= 1 && H <= 4096; }
size_t esize(int dtype) { return dtype == PLP_DTYPE_F32 ? 4 : 2; }

// Vocabulary splits of the forward sweep over all rows of a chunk
// (forward_splits); the generic path does not split.
int choose_splits(int64_t rows, int V, bool mfma) { return mfma ? forward_splits(rows, V, kMaxSplits) : 1; }

struct Plan {
  bool mfma = false;
  bool wprep = false;          // the caller passed the weight's matrix-core copy
  bool need_o = false, need_gw = false, need_gb = false;
  int64_t B = 0, T = 0, N = 0, Bc = 0, Nc = 0, nchunks = 0, cap = 0;
  int Sv = 1, St = 1;
  bool entropy = false;        // q < 1
  bool prepass = false;        // q < 1 with several chunks: stats-only pass first
  // q < 1 on the matrix cores with grad_h: statistics-only pass over every
  // row, then the grad_h accumulator pass over the compacted rows with g != 0
  bool o_compact = false;
  int64_t o2_rows = 0;         // row capacity of the compacted pass's stats / O (all splits)
  // weight-gradient launches: at most wg_sub compacted tokens each, so that
  // the rows one launch streams (wg_sub x H bf16, 128 MB) stay in the 256 MB
  // memory-side cache while every workgroup reads them; wg_launches in all
  int64_t wg_sub = 0, wg_launches = 0;
};

struct Bufs {
  __bf16* Wf = nullptr;        // fragment-major copy of W (MFMA path)
  float* bias2 = nullptr;      // the bias in fp32 for the forward sweeps (MFMA path with a bias)
  RowStats* stats = nullptr;
  float* O = nullptr;
  float* v = nullptr;
  float *lp = nullptr, *ent = nullptr, *lse = nullptr;
  uint8_t* emask = nullptr;
  SeqPart* part = nullptr;
  SeqCoef* coef = nullptr;
  float* g = nullptr;
  LossAcc* acc = nullptr;
  SelectState* sel = nullptr;  // radix select state; its first field is the threshold
  unsigned long long* ntok = nullptr;  // the batch's completion tokens (BNPO / DAPO divisor)
  int* idx = nullptr;
  TokData* tok = nullptr;
  int* count = nullptr;
  void* cscratch = nullptr;
  void* hc = nullptr;
  float* tail = nullptr;       // partial sums of the weight-gradient sweep's split tail blocks
  float* gW_acc = nullptr;
  float* gb_acc = nullptr;
  RowStats* stats2 = nullptr;  // compacted accumulator passes: the rows with g != 0 (o_compact) and the
  float* O2 = nullptr;         // flagged rows of a forward sweep (one at a time)
  FlaggedPass fp{};
};

Plan make_plan(const plp_args* a, bool need_o, bool need_gw, bool need_gb) {
  Plan p;
  p.mfma = mfma_eligible(a->dtype, a->H);
  p.wprep = p.mfma && weight_prepared(a) != nullptr;
  p.need_o = need_o;
  p.need_gw = need_gw || need_gb;
  p.need_gb = need_gb;
  p.B = a->B;
  p.T = a->T;
  p.N = a->B * a->T;
  p.Bc = (a->chunk_sequences > 0 && a->chunk_sequences < a->B) ? a->chunk_sequences : a->B;
  p.Nc = p.Bc * p.T;
  p.nchunks = (p.B + p.Bc - 1) / p.Bc;
  p.cap = round_up(p.Nc, kBK);
  p.Sv = choose_splits(p.Nc, a->V, p.mfma);
  p.St = (int)std::min<int64_t>(64, (p.T + 2047) / 2048);
  if (p.St < 1) p.St = 1;
  p.entropy = a->top_entropy_quantile < 1.0;
  p.o_compact = p.entropy && p.mfma && p.need_o;
  p.prepass = p.entropy && (p.nchunks > 1 || p.o_compact);
  // splits x row blocks < 512 while the splits are above one (forward_splits)
  p.o2_rows = p.mfma ? compact_rows_needed(p.o_compact ? p.cap : std::min(p.cap, kFlagCap), a->V, kMaxSplits) : 0;
  p.wg_sub = p.mfma ? std::max<int64_t>(32 * kBK, ((int64_t)128 << 20) / (2 * a->H) / kBK * kBK) : p.cap;
  for (int64_t c = 0; c < p.nchunks; ++c) {
    const int64_t capc = round_up(std::min(p.Bc, p.B - c * p.Bc) * p.T, kBK);
    p.wg_launches += (capc + p.wg_sub - 1) / p.wg_sub;
  }
  return p;
}

size_t carve(const plp_args* a, const Plan& p, void* ws, Bufs& b) {
  Carver c(ws);
  const int H = a->H, V = a->V;
  if (p.wprep)
    b.Wf = (__bf16*)weight_prepared(a);  // read only
  else if (p.mfma)
    b.Wf = c.take<__bf16>((size_t)round_up(V, 2 * kBK) * H);
  if (p.mfma && a->bias) b.bias2 = c.take<float>((size_t)bias_f32_len(V));
  b.stats = c.take<RowStats>((size_t)p.Sv * p.Nc);
  if (p.mfma) {
    const int64_t rows2 = p.o2_rows;
    b.stats2 = c.take<RowStats>((size_t)rows2);
    b.O2 = c.take<float>((size_t)rows2 * H);
    b.fp.cap = (int)std::min(p.cap, kFlagCap);
    b.fp.idx = c.take<int>((size_t)b.fp.cap);
    b.fp.mref = c.take<float>((size_t)b.fp.cap);
    b.fp.pos = c.take<int>((size_t)p.Nc);
    b.fp.count = c.take<int>(1);
    b.fp.stats = b.stats2;
    b.fp.O = b.O2;
    b.fp.max_splits = kMaxSplits;
  }
  if (p.need_o && !p.o_compact) {
    b.O = c.take<float>((size_t)p.Sv * p.Nc * H);
    b.v = p.Sv == 1 ? b.O : c.take<float>((size_t)p.Nc * H);
  }
  b.lp = c.take<float>(p.N);
  b.ent = c.take<float>(p.N);
  b.lse = c.take<float>(p.N);
  if (p.entropy) b.emask = c.take<uint8_t>(p.N);
  b.part = c.take<SeqPart>((size_t)p.Bc * p.St);
  b.coef = c.take<SeqCoef>(p.Bc);
  b.g = c.take<float>(p.Nc);
  b.acc = c.take<LossAcc>(1);
  b.sel = c.take<SelectState>(1);
  b.ntok = c.take<unsigned long long>(1);
  if (p.need_gw || p.o_compact) {
    b.idx = c.take<int>(p.cap);
    b.tok = c.take<TokData>(p.cap);
    b.count = c.take<int>(1);
    b.cscratch = c.take<char>(compact_scratch_bytes(p.Nc));
  }
  if (p.need_gw) {
    b.hc = c.take<char>((size_t)p.cap * H * esize(a->dtype));
    if (p.mfma) b.tail = c.take<float>(bwd_tail_scratch_floats(H));
    if (p.wg_launches > 1) {
      b.gW_acc = c.take<float>((size_t)V * H);
      if (p.need_gb) b.gb_acc = c.take<float>(V);
    }
  }
  return c.off + kAlign;
}

// Optional event timing of the two sweeps (plp_profile_start/stop).
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> ev;
  std::vector<int> kind;
  size_t used = 0;
};
Profiler g_prof;

// Returns the event pair for one launch of `k`, or nullptr when not recording.
hipEvent_t* prof_slot(int k) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.on || 2 * (g_prof.used + 1) > g_prof.ev.size()) return nullptr;
  hipEvent_t* p = &g_prof.ev[2 * g_prof.used];
  g_prof.kind[g_prof.used] = k;
  ++g_prof.used;
  return p;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(PLP_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

int check_ws(void* ws, size_t have, size_t need) {
  if (need > have) return fail(PLP_E_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", have, need);
  if (need > 0 && ws == nullptr) return fail(PLP_E_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)ws) % kAlign != 0) return fail(PLP_E_WORKSPACE, "workspace must be 256-byte aligned");
  return PLP_OK;
}

// Checks shared by the fused call and the loss-only call. `pointers`: also
// check the required pointers (the workspace queries read sizes only).
int check_loss_args(const plp_args* a, bool pointers = true) {
  if (!a) return fail(PLP_E_INVALID, "args is NULL");
  if (a->struct_size < kArgsV1Size)
    return fail(PLP_E_INVALID, "args->struct_size %u < %zu", a->struct_size, kArgsV1Size);
  if (a->B < 1 || a->T < 1) return fail(PLP_E_INVALID, "B and T must be >= 1 (B=%lld T=%lld)", (long long)a->B,
                                        (long long)a->T);
  if (a->B > kMaxRows / a->T) return fail(PLP_E_INVALID, "B*T must be < 2^31");
  if (a->loss_type < PLP_LOSS_GMPO || a->loss_type > PLP_LOSS_DAPO)
    return fail(PLP_E_INVALID, "unknown loss_type %d", a->loss_type);
  if (a->is_level != PLP_IS_TOKEN && a->is_level != PLP_IS_SEQUENCE)
    return fail(PLP_E_INVALID, "unknown is_level %d", a->is_level);
  if (a->loss_type == PLP_LOSS_GMPO && a->is_level == PLP_IS_SEQUENCE)
    return fail(PLP_E_UNSUPPORTED, "GMPO clips each token before it aggregates the sequence; "
                                   "sequence-level importance sampling is rejected");
  if (a->loss_type == PLP_LOSS_GSPO_TOKEN && a->is_level == PLP_IS_TOKEN)
    return fail(PLP_E_UNSUPPORTED, "GSPO_TOKEN uses the sequence-level ratio; set is_level = PLP_IS_SEQUENCE");
  if (token_clip_loss(a->loss_type) && a->is_level == PLP_IS_SEQUENCE)
    return fail(PLP_E_UNSUPPORTED, "GRPO, BNPO and DAPO clip each token's own ratio; their sequence-level form "
                                   "is GSPO_TOKEN");
  if (global_tokens(a) < 0) return fail(PLP_E_INVALID, "global_tokens must be >= 0");
  if (a->reduction != PLP_REDUCE_SEQ_MEAN && a->reduction != PLP_REDUCE_TOKEN_SUM)
    return fail(PLP_E_INVALID, "unknown reduction %d", a->reduction);
  if (!(a->epsilon_low >= 0.0) || !isfinite(a->epsilon_low) || !(a->epsilon_high >= 0.0) ||
      !isfinite(a->epsilon_high))
    return fail(PLP_E_INVALID, "epsilon_low and epsilon_high must be finite and >= 0");
  if (!(a->beta >= 0.0) || !isfinite(a->beta)) return fail(PLP_E_INVALID, "beta must be finite and >= 0");
  if (pointers && a->beta != 0.0 && a->ref_logp == nullptr) return fail(PLP_E_INVALID, "beta != 0 needs ref_logp");
  if (!(a->temperature > 0.0) || !isfinite(a->temperature)) return fail(PLP_E_INVALID, "temperature must be > 0");
  if (!(a->top_entropy_quantile >= 0.0 && a->top_entropy_quantile <= 1.0))
    return fail(PLP_E_INVALID, "top_entropy_quantile must lie in [0, 1] (got %g)", a->top_entropy_quantile);
  if (a->chunk_sequences < 0) return fail(PLP_E_INVALID, "chunk_sequences must be >= 0");
  if (pointers && (!a->completion_mask || (!a->advantages && !token_advantages(a))))
    return fail(PLP_E_INVALID, "completion_mask and advantages (or token_advantages) are required");
  if (token_advantages(a) && a->loss_type == PLP_LOSS_GMPO)
    return fail(PLP_E_UNSUPPORTED, "GMPO clips and averages per sequence and takes per-sequence advantages; "
                                   "token_advantages is for GSPO_TOKEN, GRPO, BNPO and DAPO");
  return PLP_OK;
}

// weight_prepared: only where the matrix-core sweeps run, 16-byte aligned.
int check_prepared(const plp_args* a) {
  const void* wp = weight_prepared(a);
  if (!wp) return PLP_OK;
  if (!mfma_eligible(a->dtype, a->H))
    return fail(PLP_E_UNSUPPORTED, "weight_prepared is for bf16 with H a multiple of 128 up to 896 (dtype %d, H=%d)",
                a->dtype, a->H);
  if ((uintptr_t)wp % 16 != 0) return fail(PLP_E_INVALID, "weight_prepared must be 16-byte aligned");
  return PLP_OK;
}

int check_fused_args(const plp_args* a) {
  int rc = check_loss_args(a);
  if (rc) return rc;
  if (a->dtype != PLP_DTYPE_F32 && a->dtype != PLP_DTYPE_BF16) return fail(PLP_E_INVALID, "unknown dtype %d", a->dtype);
  if (a->H < 1 || a->V < 1) return fail(PLP_E_INVALID, "H and V must be >= 1");
  if (!a->hidden || !a->weight || !a->targets) return fail(PLP_E_INVALID, "hidden, weight and targets are required");
  if (((uintptr_t)a->hidden | (uintptr_t)a->weight | (uintptr_t)a->bias) % 16 != 0)
    return fail(PLP_E_INVALID, "hidden, weight and bias must be 16-byte aligned");
  if (!mfma_eligible(a->dtype, a->H) && !generic_eligible(a->H))
    return fail(PLP_E_UNSUPPORTED, "H=%d is not supported (bf16 MFMA path: H multiple of 128 up to 896; "
                                   "generic path: H <= 4096)", a->H);
  return check_prepared(a);
}

// The batch's completion-token count, when the loss divides by it (BNPO, and
// DAPO without a global count), into *ntok.
int count_tokens_if_needed(const plp_args* a, unsigned long long* ntok, hipStream_t st) {
  if (token_mean_loss(a->loss_type) && !(a->loss_type == PLP_LOSS_DAPO && global_tokens(a) > 0))
    HIP_TRY(launch_count_mask(a->completion_mask, a->B * a->T, ntok, st));
  return PLP_OK;
}

LossParams loss_params(const plp_args* a, const unsigned long long* ntok_dev) {
  LossParams p;
  p.B_total = a->B;
  p.T = a->T;
  p.loss_type = a->loss_type;
  p.reduction = a->reduction;
  p.eh32 = (float)a->epsilon_high;
  p.el32 = (float)a->epsilon_low;
  p.lo32 = (float)(1.0 - a->epsilon_low);
  p.hi32 = (float)(1.0 + a->epsilon_high);
  p.beta = a->beta;
  p.norm_tokens = a->loss_type == PLP_LOSS_DAPO ? global_tokens(a) : 0;
  p.ntok_dev = ntok_dev;
  p.token_adv = token_advantages(a) != nullptr ? 1 : 0;
  p.kl_bc = kl_bias_correction(a);
  return p;
}

// The second forward pass: the rows the sweep flagged (up to fp.cap) listed
// with their largest logit and swept again, read through the list, with that logit as
// their exponent reference, which nothing can exceed; the merge takes their
// statistics and accumulator from this pass. A call with no flagged row
// costs the listing and the launches, whose workgroups find no row. The
// sweep before it has cleared fp.count (its clear_count).
hipError_t flagged_pass(const void* h, const __bf16* Wf, const float* b32, const __bf16* b16, const RowStats* stats,
                        int Sv, int64_t n, int H, int V, float inv_tau, const FlaggedPass& fp, hipStream_t st) {
  hipError_t e = launch_flag_scan(stats, Sv, n, fp.cap, fp.idx, fp.mref, fp.pos, fp.count, st);
  if (e != hipSuccess) return e;
  return launch_fwd_mfma((const __bf16*)h, Wf, b32, b16, fp.cap, H, V, inv_tau, fp.max_splits, true, fp.stats, fp.O,
                         st, fp.count, fp.mref, 1, fp.idx);
}

// A forward sweep over n rows of h. The statistics-only sweep (two workgroups
// per compute unit) with one vocabulary split goes out in launches of at
// most 4096 row blocks (eight rounds): over more rounds the workgroups drift
// apart, stop sharing W's tiles in L2 and lose up to 40 % at 4M rows; the
// accumulator sweep keeps its single launch (no such loss measured).
hipError_t forward_sweep(const void* h, const __bf16* Wf, const float* b32, const __bf16* b16, int64_t n, int H, int V,
                         float inv_tau, int Sv, bool with_o, RowStats* stats, float* O, int* clear_count,
                         hipStream_t st) {
  constexpr int64_t kRoundsRows = 4096 * (int64_t)kBQ;
  if (with_o || Sv != 1 || n <= kRoundsRows)
    return launch_fwd_mfma((const __bf16*)h, Wf, b32, b16, n, H, V, inv_tau, Sv, with_o, stats, O, st, nullptr,
                           nullptr, 1, nullptr, clear_count);
  for (int64_t o = 0; o < n; o += kRoundsRows) {
    const hipError_t e = launch_fwd_mfma((const __bf16*)h + o * H, Wf, b32, b16, std::min(kRoundsRows, n - o), H, V,
                                         inv_tau, 1, false, stats + o, nullptr, st, nullptr, nullptr, 1, nullptr,
                                         o == 0 ? clear_count : nullptr);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Workspace of plp_selective_entropy (sizes only when ws is NULL).
struct SelBufs {
  bool mfma = false;
  int sv = 1;
  RowStats* stats = nullptr;
  float* scratch_lp = nullptr;
  __bf16* Wf = nullptr;
  float* bias2 = nullptr;  // the bias in fp32 for the forward sweeps (when one is given)
  FlaggedPass fp{};
};

// prepared: the weight's matrix-core copy comes from the caller (no Wf here).
size_t carve_selective(void* ws, int64_t N, int H, int V, int dtype, bool prepared, SelBufs& sb) {
  Carver c(ws);
  sb.mfma = mfma_eligible(dtype, H);
  sb.sv = choose_splits(N, V, sb.mfma);
  sb.stats = c.take<RowStats>((size_t)sb.sv * N);
  sb.scratch_lp = c.take<float>(N);
  if (sb.mfma) {
    if (!prepared) sb.Wf = c.take<__bf16>((size_t)round_up(V, 2 * kBK) * H);
    sb.bias2 = c.take<float>((size_t)bias_f32_len(V));
    sb.fp.cap = (int)std::min(round_up(N, kBK), kFlagCap);
    sb.fp.idx = c.take<int>((size_t)sb.fp.cap);
    sb.fp.mref = c.take<float>((size_t)sb.fp.cap);
    sb.fp.pos = c.take<int>((size_t)N);
    sb.fp.count = c.take<int>(1);
    const int64_t rows2 = compact_rows_needed(sb.fp.cap, V, kMaxSplits);
    sb.fp.stats = c.take<RowStats>((size_t)rows2);
    sb.fp.O = c.take<float>((size_t)rows2 * H);
    sb.fp.max_splits = kMaxSplits;
  }
  return c.off + kAlign;
}

// Forward sweep + merge for rows [r0, r0 + n).
int forward_rows(const plp_args* a, const Plan& p, Bufs& b, int64_t r0, int64_t n, bool with_o, hipStream_t st) {
  const size_t es = esize(a->dtype);
  const char* h = (const char*)a->hidden + (size_t)r0 * a->H * es;
  const int64_t* y = a->targets + r0;
  const float inv_tau = (float)(1.0 / a->temperature);
  if (p.mfma) {
    hipEvent_t* ev = prof_slot(0);
    if (ev) HIP_TRY(hipEventRecord(ev[0], st));
    HIP_TRY(forward_sweep(h, b.Wf, b.bias2, (const __bf16*)a->bias, n, a->H, a->V, inv_tau, p.Sv, with_o, b.stats,
                          with_o ? b.O : nullptr, b.fp.count, st));
    if (ev) HIP_TRY(hipEventRecord(ev[1], st));
    HIP_TRY(flagged_pass(h, b.Wf, b.bias2, (const __bf16*)a->bias, b.stats, p.Sv, n, a->H, a->V, inv_tau, b.fp, st));
  } else {
    HIP_TRY(launch_fwd_generic(a->dtype, h, a->weight, a->bias, y, n, a->H, a->V, inv_tau, with_o, b.stats,
                               with_o ? b.O : nullptr, st));
  }
  HIP_TRY(launch_combine(a->dtype, b.stats, with_o ? b.O : nullptr, p.Sv, n, a->H, a->V, h, a->weight, a->bias,
                         inv_tau, y, b.lp + r0, b.ent + r0, b.lse + r0, with_o ? b.v : nullptr, st,
                         p.mfma ? &b.fp : nullptr));
  return PLP_OK;
}

int check_quantile_args(const float* entropy, const uint8_t* active, int64_t N, double q, const uint8_t* mask_out) {
  if (!(q >= 0.0 && q <= 1.0)) return fail(PLP_E_INVALID, "q must lie in [0, 1] (got %g)", q);
  if (N > 0 && (!entropy || !active || !mask_out)) return fail(PLP_E_INVALID, "entropy, active and mask_out are required");
  return PLP_OK;
}

// The batch-global mask with the select state in `sel` (whose contents the
// first kernel resets).
int quantile_mask(const float* entropy, const uint8_t* active, int64_t N, double q, uint8_t* mask_out,
                  float* threshold_out, SelectState* sel, hipStream_t st) {
  if (q == 1.0) {
    if (N > 0) HIP_TRY(launch_copy_mask(active, N, mask_out, st));
    if (threshold_out) HIP_TRY(launch_set_nan(threshold_out, st));
    return ok();
  }
  HIP_TRY(launch_entropy_select(entropy, active, N, (float)(1.0 - q), sel, st));
  if (N > 0) HIP_TRY(launch_entropy_mask(entropy, active, N, &sel->thr, mask_out, st));
  if (threshold_out) HIP_TRY(launch_store_thr(&sel->thr, threshold_out, st));
  return ok();
}

// Scratch of plp_entropy_quantile_mask_noalloc: the radix select's state in a
// device array rather than a workspace. Every device that runs the call holds
// its own copy until the process ends. On the host the array's name is only
// a stand-in for the symbol: its device address is taken once per device
// with hipGetSymbolAddress (with that device current) and only that address
// is handed to kernels.
constexpr size_t kStaticScratchBytes = 32768;
static_assert(sizeof(SelectState) <= kStaticScratchBytes, "the select state fits the static scratch");
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PLP_E_UNSUPPORTED, "device %d: the static scratch is kept for devices 0-%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    HIP_TRY(hipGetDevice(&cur));
    if (cur != dev) HIP_TRY(hipSetDevice(dev));
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) return fail(PLP_E_HIP, "hipSetDevice: %s", hipGetErrorString(e2));
    }
    if (e != hipSuccess) return fail(PLP_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    if (p == nullptr) return fail(PLP_E_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PLP_OK;
}

}  // namespace

extern "C" {

PLP_API int plp_abi_version(void) { return PLP_ABI_VERSION; }

PLP_API int plp_prepared_weight_size(int32_t H, int32_t V, int32_t dtype, size_t* bytes) {
  if (!bytes) return fail(PLP_E_INVALID, "bytes is NULL");
  if (V < 1 || H < 1) return fail(PLP_E_INVALID, "H and V must be >= 1");
  if (!mfma_eligible(dtype, H))
    return fail(PLP_E_UNSUPPORTED, "the prepared weight is for bf16 with H a multiple of 128 up to 896 (dtype %d, H=%d)",
                dtype, H);
  *bytes = (size_t)round_up(V, 2 * kBK) * H * sizeof(__bf16);
  return ok();
}

PLP_API int plp_prepare_weight(const void* weight, int32_t H, int32_t V, int32_t dtype, void* prepared,
                               size_t prepared_bytes, hipStream_t st) {
  size_t need = 0;
  int rc = plp_prepared_weight_size(H, V, dtype, &need);
  if (rc) return rc;
  if (!weight || !prepared) return fail(PLP_E_INVALID, "weight and prepared are required");
  if ((uintptr_t)weight % 16 != 0) return fail(PLP_E_INVALID, "weight must be 16-byte aligned");
  if ((uintptr_t)prepared % kAlign != 0) return fail(PLP_E_INVALID, "prepared must be 256-byte aligned");
  if (prepared_bytes < need)
    return fail(PLP_E_INVALID, "prepared buffer too small: %zu bytes given, %zu needed", prepared_bytes, need);
  HIP_TRY(launch_frag_copy((const __bf16*)weight, nullptr, nullptr, V, round_up(V, 2 * kBK) / kBK, H,
                           (__bf16*)prepared, st));
  return ok();
}

PLP_API int plp_profile_start(int32_t max_records) {
  if (max_records < 1) return fail(PLP_E_INVALID, "max_records must be >= 1");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.assign(2 * (size_t)max_records, nullptr);
  g_prof.kind.assign((size_t)max_records, 0);
  g_prof.used = 0;
  for (auto& e : g_prof.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      g_prof.on = false;
      return fail(PLP_E_HIP, "hipEventCreate: %s", hipGetErrorString(r));
    }
  }
  g_prof.on = true;
  return ok();
}

PLP_API int plp_profile_stop(double* ms_out, int32_t* count_out) { return plp_profile_stop_n(ms_out, count_out, 2); }

PLP_API int plp_profile_stop_n(double* ms_out, int32_t* count_out, int32_t n_kinds) {
  if (!ms_out || !count_out) return fail(PLP_E_INVALID, "ms_out and count_out are required");
  if (n_kinds < 2) return fail(PLP_E_INVALID, "n_kinds must be >= 2");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (int k = 0; k < n_kinds; ++k) {
    ms_out[k] = 0.0;
    count_out[k] = 0;
  }
  int rc = PLP_OK;
  for (size_t i = 0; i < g_prof.used; ++i) {
    float ms = 0.f;
    hipError_t r = hipEventSynchronize(g_prof.ev[2 * i + 1]);
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
    if (r != hipSuccess) {
      rc = fail(PLP_E_HIP, "event timing: %s", hipGetErrorString(r));
      break;
    }
    // with two kinds the compacted accumulator passes count as forward sweeps
    const int k = g_prof.kind[i] < n_kinds ? g_prof.kind[i] : 0;
    ms_out[k] += ms;
    count_out[k] += 1;
  }
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.kind.clear();
  g_prof.used = 0;
  g_prof.on = false;
  return rc == PLP_OK ? ok() : rc;
}

PLP_API const char* plp_last_error(void) { return g_last_error.c_str(); }

PLP_API int plp_workspace_size(const plp_args* a, size_t* bytes) {
  if (!bytes) return fail(PLP_E_INVALID, "bytes is NULL");
  int rc = check_loss_args(a, false);
  if (rc) return rc;
  if (a->H < 1 || a->V < 1) return fail(PLP_E_INVALID, "H and V must be >= 1");
  if (a->dtype != PLP_DTYPE_F32 && a->dtype != PLP_DTYPE_BF16) return fail(PLP_E_INVALID, "unknown dtype %d", a->dtype);
  if (weight_prepared(a) && !mfma_eligible(a->dtype, a->H))
    return fail(PLP_E_UNSUPPORTED, "weight_prepared is for bf16 with H a multiple of 128 up to 896 (dtype %d, H=%d)",
                a->dtype, a->H);
  // Sized for every gradient output, the largest request.
  Plan p = make_plan(a, true, true, a->bias != nullptr);
  Bufs b;
  *bytes = carve(a, p, nullptr, b);
  return ok();
}

PLP_API int plp_fused_lmhead_policy_loss_fwd_bwd(const plp_args* a, const plp_outputs* out, void* ws,
                                                 size_t ws_bytes, hipStream_t st) {
  int rc = check_fused_args(a);
  if (rc) return rc;
  if (!out || out->struct_size < sizeof(plp_outputs)) return fail(PLP_E_INVALID, "outputs NULL or struct_size too small");
  if (!out->loss || !out->metrics) return fail(PLP_E_INVALID, "loss and metrics outputs are required");
  if (out->grad_bias && !a->bias) return fail(PLP_E_INVALID, "grad_bias requested without bias");
  if (((uintptr_t)out->grad_hidden | (uintptr_t)out->grad_weight | (uintptr_t)out->grad_bias) % 16 != 0)
    return fail(PLP_E_INVALID, "gradient outputs must be 16-byte aligned");
  size_t need_full = 0;
  {
    Plan pf = make_plan(a, true, true, a->bias != nullptr);
    Bufs bf;
    need_full = carve(a, pf, nullptr, bf);
  }
  rc = check_ws(ws, ws_bytes, need_full);
  if (rc) return rc;

  const Plan p = make_plan(a, out->grad_hidden != nullptr, out->grad_weight != nullptr, out->grad_bias != nullptr);
  Bufs b;
  carve(a, p, ws, b);
  const int H = a->H, V = a->V;
  const size_t es = esize(a->dtype);
  const float inv_tau = (float)(1.0 / a->temperature);
  const LossParams lpar = loss_params(a, b.ntok);
  rc = count_tokens_if_needed(a, b.ntok, st);
  if (rc) return rc;

  if (p.mfma && !p.wprep)
    HIP_TRY(launch_frag_copy((const __bf16*)a->weight, nullptr, nullptr, V, round_up(V, 2 * kBK) / kBK, H, b.Wf, st));
  if (b.bias2) HIP_TRY(launch_bias_f32((const __bf16*)a->bias, V, b.bias2, st));

  bool first_chunk_done = false;
  if (p.entropy) {
    if (!p.prepass) {
      rc = forward_rows(a, p, b, 0, p.N, p.need_o, st);
      if (rc) return rc;
      first_chunk_done = true;
    } else {
      for (int64_t c = 0; c < p.nchunks; ++c) {
        const int64_t r0 = c * p.Nc, n = std::min(p.Nc, p.N - r0);
        rc = forward_rows(a, p, b, r0, n, false, st);
        if (rc) return rc;
      }
    }
    HIP_TRY(launch_entropy_select(b.ent, a->completion_mask, p.N, (float)(1.0 - a->top_entropy_quantile), b.sel,
                                  st));
    HIP_TRY(launch_entropy_mask(b.ent, a->completion_mask, p.N, &b.sel->thr, b.emask, st));
  }

  int64_t wg_launch = 0;
  for (int64_t c = 0; c < p.nchunks; ++c) {
    const int64_t s0 = c * p.Bc, bc = std::min(p.Bc, p.B - s0);
    const int64_t r0 = s0 * p.T, n = bc * p.T;
    // the statistics of every row are in place after the q < 1 passes; the
    // forward runs here for q = 1, and for q < 1 only to accumulate grad_h
    // over whole chunks (the generic path with several chunks)
    const bool fwd_here = !p.entropy || (p.need_o && !p.o_compact && !(c == 0 && first_chunk_done));
    if (fwd_here) {
      rc = forward_rows(a, p, b, r0, n, p.need_o, st);
      if (rc) return rc;
    }
    const float* old = a->old_logp ? a->old_logp + r0 : nullptr;
    const float* ref = a->ref_logp ? a->ref_logp + r0 : nullptr;
    const uint8_t* comp = a->completion_mask + r0;
    const uint8_t* ratio = a->ratio_mask ? a->ratio_mask + r0 : nullptr;
    const uint8_t* em = b.emask ? b.emask + r0 : nullptr;
    const float* adv = a->advantages ? a->advantages + s0 : nullptr;
    const float* tadv = token_advantages(a) ? token_advantages(a) + r0 : nullptr;
    HIP_TRY(launch_loss_seq_partial(lpar, bc, b.lp + r0, old, ref, comp, ratio, em, adv, tadv, p.St, b.part, st));
    const bool last = c == p.nchunks - 1;
    HIP_TRY(launch_loss_seq_final(lpar, bc, p.St, b.part, adv, b.coef, b.acc, c == 0, p.entropy ? &b.sel->thr : nullptr,
                                  last ? out->loss : nullptr, last ? out->metrics : nullptr, st));
    float* g = out->dlogp_out ? out->dlogp_out + r0 : b.g;
    int* cnt32 = (p.need_gw || p.o_compact) ? (int*)b.cscratch : nullptr;
    char* gh = p.need_o ? (char*)out->grad_hidden + (size_t)r0 * H * es : nullptr;
    // with the compacted accumulator pass the token kernel writes zero rows
    // and the rows with g != 0 are written after that pass
    HIP_TRY(launch_loss_tokens(a->dtype, lpar, bc, b.lp + r0, old, ref, comp, ratio, em, tadv, b.coef, g, cnt32,
                               p.need_o && !p.o_compact ? b.v : nullptr, H, inv_tau, gh, st));
    const char* hsrc = (const char*)a->hidden + (size_t)r0 * H * es;
    if (p.need_gw || p.o_compact)
      HIP_TRY(launch_compact_scatter(g, b.lse + r0, a->targets + r0, n, inv_tau, cnt32, b.idx, b.tok, b.count, st));
    if (p.o_compact) {
      hipEvent_t* ev = prof_slot(2);
      if (ev) HIP_TRY(hipEventRecord(ev[0], st));
      // each row's log-sum-exp (lse >= every logit of the row) as its
      // exponent reference: nothing to flag in this pass
      static_assert(offsetof(TokData, lse) == 0 && sizeof(TokData) == 4 * sizeof(float), "lse every 4 floats");
      HIP_TRY(launch_fwd_mfma((const __bf16*)hsrc, b.Wf, b.bias2, (const __bf16*)a->bias, p.cap, H, V, inv_tau,
                              kMaxSplits,
                              true, b.stats2, b.O2, st, b.count, (const float*)b.tok, 4, b.idx));
      if (ev) HIP_TRY(hipEventRecord(ev[1], st));
      HIP_TRY(launch_grad_h_compact(a->dtype, b.stats2, b.O2, kMaxSplits, p.cap, H, V, hsrc, a->weight, a->bias,
                                    inv_tau, b.idx, b.tok, b.count, gh, st));
    }
    if (p.need_gw) {
      if (p.mfma)
        HIP_TRY(launch_frag_copy((const __bf16*)hsrc, b.idx, b.count, n, p.cap / kBK, H, (__bf16*)b.hc, st));
      else
        HIP_TRY(launch_gather_rows(a->dtype, hsrc, b.idx, b.count, p.cap, H, b.hc, st));
      // accumulator modes over all weight-gradient launches of the call:
      // 0 the only launch writes grad_W; 1 the first stores the fp32
      // accumulator, 2 the middle ones add into it, 3 the last adds and
      // writes grad_W
      const int64_t capc = round_up(n, kBK);
      for (int64_t k0 = 0; k0 < capc; k0 += p.wg_sub) {
        const int mode = p.wg_launches == 1 ? 0 : (wg_launch == 0 ? 1 : (wg_launch == p.wg_launches - 1 ? 3 : 2));
        ++wg_launch;
        if (p.mfma) {
          hipEvent_t* ev = prof_slot(1);
          if (ev) HIP_TRY(hipEventRecord(ev[0], st));
          HIP_TRY(launch_bwd_mfma(b.Wf, (const __bf16*)a->bias, (const __bf16*)b.hc, b.tok, b.count, (int)k0,
                                  (int)std::min(p.wg_sub, capc - k0), H, V, inv_tau, mode, b.gW_acc, b.gb_acc,
                                  (__bf16*)out->grad_weight, (__bf16*)out->grad_bias, b.tail, st));
          if (ev) HIP_TRY(hipEventRecord(ev[1], st));
        } else
          HIP_TRY(launch_bwd_generic(a->dtype, a->weight, a->bias, b.hc, b.tok, b.count, H, V, inv_tau, mode,
                                     b.gW_acc, b.gb_acc, out->grad_weight, out->grad_bias, st));
      }
    }
  }
  if (out->logp_out) HIP_TRY(hipMemcpyAsync(out->logp_out, b.lp, p.N * sizeof(float), hipMemcpyDeviceToDevice, st));
  if (out->entropy_out)
    HIP_TRY(hipMemcpyAsync(out->entropy_out, b.ent, p.N * sizeof(float), hipMemcpyDeviceToDevice, st));
  if (out->entropy_mask_out)
    HIP_TRY(launch_copy_mask(p.entropy ? b.emask : a->completion_mask, p.N, out->entropy_mask_out, st));
  return ok();
}

namespace {

int selective_workspace_size(int64_t N, int32_t H, int32_t V, int32_t dtype, bool prepared, size_t* bytes) {
  if (!bytes) return fail(PLP_E_INVALID, "bytes is NULL");
  if (N < 1 || N >= kMaxRows || H < 1 || V < 1) return fail(PLP_E_INVALID, "bad sizes N=%lld H=%d V=%d", (long long)N, H, V);
  if (dtype != PLP_DTYPE_F32 && dtype != PLP_DTYPE_BF16) return fail(PLP_E_INVALID, "unknown dtype %d", dtype);
  if (prepared && !mfma_eligible(dtype, H))
    return fail(PLP_E_UNSUPPORTED, "weight_prepared is for bf16 with H a multiple of 128 up to 896 (dtype %d, H=%d)",
                dtype, H);
  SelBufs sb;
  *bytes = carve_selective(nullptr, N, H, V, dtype, prepared, sb);
  return ok();
}

// Both selective-entropy entry points; wprep is the caller's matrix-core copy
// of the weight or NULL (then the call makes its own in the workspace).
int selective_entropy(const void* hidden, const void* weight, const void* wprep, bool prepared, const void* bias,
                      int64_t N, int32_t H, int32_t V, int32_t dtype, float temperature, const int64_t* targets,
                      float* entropy_out, float* logp_out, void* ws, size_t ws_bytes, hipStream_t st) {
  size_t need = 0;
  int rc = selective_workspace_size(N, H, V, dtype, prepared, &need);
  if (rc) return rc;
  if (prepared && (!wprep || (uintptr_t)wprep % 16 != 0))
    return fail(PLP_E_INVALID, "weight_prepared must be non-NULL and 16-byte aligned");
  if (!hidden || !weight || !entropy_out) return fail(PLP_E_INVALID, "hidden, weight and entropy_out are required");
  if (((uintptr_t)hidden | (uintptr_t)weight | (uintptr_t)bias) % 16 != 0)
    return fail(PLP_E_INVALID, "hidden, weight and bias must be 16-byte aligned");
  if (logp_out && !targets) return fail(PLP_E_INVALID, "logp_out needs targets");
  if (!(temperature > 0.f) || !isfinite(temperature)) return fail(PLP_E_INVALID, "temperature must be > 0");
  if (!mfma_eligible(dtype, H) && !generic_eligible(H)) return fail(PLP_E_UNSUPPORTED, "H=%d is not supported", H);
  rc = check_ws(ws, ws_bytes, need);
  if (rc) return rc;
  SelBufs sb;
  carve_selective(ws, N, H, V, dtype, prepared, sb);
  const int64_t* y = targets;  // may be NULL: no target logit is taken
  const float inv_tau = 1.0f / temperature;
  if (sb.mfma) {
    if (prepared)
      sb.Wf = (__bf16*)wprep;  // read only
    else
      HIP_TRY(launch_frag_copy((const __bf16*)weight, nullptr, nullptr, V, round_up(V, 2 * kBK) / kBK, H, sb.Wf, st));
    if (bias) HIP_TRY(launch_bias_f32((const __bf16*)bias, V, sb.bias2, st));
    const float* bias2 = bias ? sb.bias2 : nullptr;
    HIP_TRY(forward_sweep(hidden, sb.Wf, bias2, (const __bf16*)bias, N, H, V, inv_tau, sb.sv, false, sb.stats, nullptr,
                          sb.fp.count, st));
    HIP_TRY(flagged_pass(hidden, sb.Wf, bias2, (const __bf16*)bias, sb.stats, sb.sv, N, H, V, inv_tau, sb.fp, st));
  }
  else
    HIP_TRY(launch_fwd_generic(dtype, hidden, weight, bias, y, N, H, V, inv_tau, false, sb.stats, nullptr, st));
  HIP_TRY(launch_combine(dtype, sb.stats, nullptr, sb.sv, N, H, V, hidden, weight, bias, inv_tau, y,
                         logp_out ? logp_out : (y ? sb.scratch_lp : nullptr), entropy_out, nullptr, nullptr, st,
                         sb.mfma ? &sb.fp : nullptr));
  return ok();
}

}  // namespace

PLP_API int plp_selective_entropy_workspace_size(int64_t N, int32_t H, int32_t V, int32_t dtype, size_t* bytes) {
  return selective_workspace_size(N, H, V, dtype, false, bytes);
}

PLP_API int plp_selective_entropy(const void* hidden, const void* weight, const void* bias, int64_t N, int32_t H,
                                  int32_t V, int32_t dtype, float temperature, const int64_t* targets,
                                  float* entropy_out, float* logp_out, void* ws, size_t ws_bytes, hipStream_t st) {
  return selective_entropy(hidden, weight, nullptr, false, bias, N, H, V, dtype, temperature, targets, entropy_out,
                           logp_out, ws, ws_bytes, st);
}

PLP_API int plp_selective_entropy_prepared_workspace_size(int64_t N, int32_t H, int32_t V, int32_t dtype,
                                                          size_t* bytes) {
  return selective_workspace_size(N, H, V, dtype, true, bytes);
}

PLP_API int plp_selective_entropy_prepared(const void* hidden, const void* weight, const void* weight_prepared,
                                           const void* bias, int64_t N, int32_t H, int32_t V, int32_t dtype,
                                           float temperature, const int64_t* targets, float* entropy_out,
                                           float* logp_out, void* ws, size_t ws_bytes, hipStream_t st) {
  return selective_entropy(hidden, weight, weight_prepared, true, bias, N, H, V, dtype, temperature, targets,
                           entropy_out, logp_out, ws, ws_bytes, st);
}

PLP_API int plp_entropy_quantile_mask_workspace_size(int64_t N, size_t* bytes) {
  if (!bytes) return fail(PLP_E_INVALID, "bytes is NULL");
  if (N < 0 || N >= kMaxRows) return fail(PLP_E_INVALID, "bad N=%lld", (long long)N);
  *bytes = align_up(sizeof(SelectState)) + kAlign;
  return ok();
}

PLP_API int plp_entropy_quantile_mask(const float* entropy, const uint8_t* active, int64_t N, double q,
                                      uint8_t* mask_out, float* threshold_out, void* ws, size_t ws_bytes,
                                      hipStream_t st) {
  size_t need = 0;
  int rc = plp_entropy_quantile_mask_workspace_size(N, &need);
  if (rc) return rc;
  rc = check_quantile_args(entropy, active, N, q, mask_out);
  if (rc) return rc;
  rc = check_ws(ws, ws_bytes, need);
  if (rc) return rc;
  return quantile_mask(entropy, active, N, q, mask_out, threshold_out, (SelectState*)ws, st);
}

PLP_API int plp_entropy_quantile_mask_noalloc(const float* entropy, const uint8_t* active, int64_t N, double q,
                                              uint8_t* mask_out, float* threshold_out, hipStream_t st) {
  if (N < 0 || N >= kMaxRows)
    return fail(PLP_E_INVALID, "N=%lld outside [0, 2^31), the largest input of the static scratch", (long long)N);
  int rc = check_quantile_args(entropy, active, N, q, mask_out);
  if (rc) return rc;
  int dev = 0;
  HIP_TRY(hipStreamGetDevice(st, &dev));
  void* sel = nullptr;
  rc = static_scratch(dev, &sel);
  if (rc) return rc;
  return quantile_mask(entropy, active, N, q, mask_out, threshold_out, (SelectState*)sel, st);
}

PLP_API int plp_policy_loss_workspace_size(const plp_args* a, size_t* bytes) {
  if (!bytes) return fail(PLP_E_INVALID, "bytes is NULL");
  int rc = check_loss_args(a, false);
  if (rc) return rc;
  const int64_t N = a->B * a->T;
  const int St = (int)std::max<int64_t>(1, std::min<int64_t>(64, (a->T + 2047) / 2048));
  Carver c(nullptr);
  c.take<uint8_t>(N);
  c.take<SeqPart>((size_t)a->B * St);
  c.take<SeqCoef>(a->B);
  c.take<float>(N);
  c.take<LossAcc>(1);
  c.take<SelectState>(1);
  c.take<unsigned long long>(1);
  *bytes = c.off + kAlign;
  return ok();
}

PLP_API int plp_policy_loss_from_logprobs(const plp_args* a, const float* logp, const float* entropy,
                                          const plp_outputs* out, void* ws, size_t ws_bytes, hipStream_t st) {
  size_t need = 0;
  int rc = check_loss_args(a);
  if (rc) return rc;
  rc = plp_policy_loss_workspace_size(a, &need);
  if (rc) return rc;
  if (!logp) return fail(PLP_E_INVALID, "logp is required");
  if (!out || out->struct_size < sizeof(plp_outputs) || !out->loss || !out->metrics)
    return fail(PLP_E_INVALID, "outputs with loss and metrics are required");
  const bool q_on = a->top_entropy_quantile < 1.0;
  if (q_on && !entropy) return fail(PLP_E_INVALID, "entropy is required when top_entropy_quantile < 1");
  rc = check_ws(ws, ws_bytes, need);
  if (rc) return rc;
  const int64_t N = a->B * a->T;
  const int St = (int)std::max<int64_t>(1, std::min<int64_t>(64, (a->T + 2047) / 2048));
  Carver c(ws);
  uint8_t* emask = c.take<uint8_t>(N);
  SeqPart* part = c.take<SeqPart>((size_t)a->B * St);
  SeqCoef* coef = c.take<SeqCoef>(a->B);
  float* gbuf = c.take<float>(N);
  LossAcc* acc = c.take<LossAcc>(1);
  SelectState* sel = c.take<SelectState>(1);
  unsigned long long* ntok = c.take<unsigned long long>(1);
  const LossParams lpar = loss_params(a, ntok);
  rc = count_tokens_if_needed(a, ntok, st);
  if (rc) return rc;
  if (q_on) {
    HIP_TRY(launch_entropy_select(entropy, a->completion_mask, N, (float)(1.0 - a->top_entropy_quantile), sel, st));
    HIP_TRY(launch_entropy_mask(entropy, a->completion_mask, N, &sel->thr, emask, st));
  }
  const uint8_t* em = q_on ? emask : nullptr;
  HIP_TRY(launch_loss_seq_partial(lpar, a->B, logp, a->old_logp, a->ref_logp, a->completion_mask, a->ratio_mask, em,
                                  a->advantages, token_advantages(a), St, part, st));
  HIP_TRY(launch_loss_seq_final(lpar, a->B, St, part, a->advantages, coef, acc, true, q_on ? &sel->thr : nullptr, out->loss,
                                out->metrics, st));
  float* g = out->dlogp_out ? out->dlogp_out : gbuf;
  HIP_TRY(launch_loss_tokens(PLP_DTYPE_F32, lpar, a->B, logp, a->old_logp, a->ref_logp, a->completion_mask,
                             a->ratio_mask, em, token_advantages(a), coef, g, nullptr, nullptr, 0, 1.0f, nullptr, st));
  if (out->entropy_mask_out) HIP_TRY(launch_copy_mask(q_on ? emask : a->completion_mask, N, out->entropy_mask_out, st));
  return ok();
}

}  // extern "C"
