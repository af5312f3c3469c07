// Everything after the logits: split merge, the GMPO / GSPO-token / K3 KL
// loss stage, grad_h, token compaction for the weight-gradient sweep, and the
// batch-global entropy quantile mask. All reductions run in a fixed order, so
// results are bitwise reproducible.
#include "common.h"
#include "generic_row.h"

#include <math.h>

namespace plp {

namespace {

constexpr int NT = 256;
constexpr int kEarlySplits = 32;  // split accumulators a merge thread loads up front

template <typename T>
__device__ __forceinline__ float ldf(const T* p, int64_t i) {
  return (float)p[i];
}

// Four consecutive elements p[i .. i+3] as floats (i a multiple of 4, p
// 16-byte aligned): one 16-byte load for fp32, one 8-byte load for bf16.
__device__ __forceinline__ f32x4 ld4f(const float* p, int64_t i) { return *reinterpret_cast<const f32x4*>(p + i); }
__device__ __forceinline__ f32x4 ld4f(const __bf16* p, int64_t i) {
  const uint2 u = *reinterpret_cast<const uint2*>(p + i);
  return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
               __uint_as_float(u.y & 0xffff0000u)};
}

// Sum over the block's NT threads, the same order on every call: a butterfly
// within each 64-lane wave, then the four wave sums as (w0 + w1) + (w2 + w3).
static_assert(NT == 256, "block_sum combines four waves");
template <typename V_>
__device__ V_ block_sum(V_ v, V_* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const V_ r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Merge of vocabulary splits (per row): lse = M + log sum_j e^{m_j-M} s_j,
// lp = z_y - lse, H = lse - (sum_j e^{m_j-M} sz_j) / (sum_j e^{m_j-M} s_j)
// (PR #1558: H = log_z - sum_exp_z / sum_exp), and v = W_y - O/s, so that
// grad_h = (g / tau) v since d lp / d z_v = [v = y] - p_v. The target logit
// z_y = (h . W_y + b_y) / tau is one dot product per row, taken here rather
// than gathered inside the sweeps. A row any split flagged is recomputed
// exactly (row_exact).
// ---------------------------------------------------------------------------
//
// Rows the sweep flagged and a second pass took again against their largest
// logit (pos[row] = k >= 0) are merged from that pass's statistics and
// accumulator at position k (row stride compact_stride(n2) and
// forward_splits(n2, V, max_splits2) splits, n2 = min(*count2, cap2)).
template <typename T, bool EARLY>
__global__ __launch_bounds__(NT) void combine_kernel(const RowStats* __restrict__ stats, const float* __restrict__ O,
                                                     int Sv, int64_t N, int H, int V, const T* __restrict__ h,
                                                     const T* __restrict__ W, const T* __restrict__ b, float inv_tau,
                                                     const int64_t* __restrict__ y, float* __restrict__ lp,
                                                     float* __restrict__ ent, float* __restrict__ lse_out,
                                                     float* __restrict__ vout, const int* __restrict__ pos,
                                                     const RowStats* __restrict__ stats2,
                                                     const float* __restrict__ O2, const int* __restrict__ count2,
                                                     int cap2, int max_splits2) {
  extern __shared__ float sm[];
  const int64_t row = blockIdx.x;
  __shared__ double s_c[64];  // per-split weights e^{m_j - M}, up to 64 splits
  __shared__ double s_red[NT];
  __shared__ double s_res[4];
  __shared__ int s_flag;
  const int64_t yv = y ? y[row] : -1;
  // targets outside [0, V) are invalid input; clamp the index so they cannot
  // address memory outside W
  const int64_t yc = yv < 0 ? 0 : (yv >= V ? V - 1 : yv);
  const RowStats* st_ = stats;
  const float* O_ = O;
  int Sv_ = Sv;
  int64_t stride = N, srow = row;
  // EARLY (several splits, up to 32, one 4-column group per thread): each
  // thread's split accumulators are loaded first, so their latency overlaps
  // the split statistics and the target-logit dot product below. It costs
  // registers (two waves per SIMD), so a single split takes the plain form.
  const bool vec = (H & 3) == 0;
  bool early = EARLY && vout != nullptr && vec && Sv <= kEarlySplits && H / 4 <= NT;
  f32x4 opre[EARLY ? kEarlySplits : 1];
  if (early && (int)threadIdx.x < H / 4) {
#pragma unroll
    for (int j = 0; j < (EARLY ? kEarlySplits : 1); ++j)
      if (j < Sv) opre[j] = *reinterpret_cast<const f32x4*>(O + ((int64_t)j * N + row) * H + 4 * threadIdx.x);
  }
  // split statistics (one lane per split; butterfly reductions in a fixed order)
  auto merge_stats = [&]() {
    if (threadIdx.x < 64) {
      const int j = threadIdx.x;
      const bool have = j < Sv_;
      RowStats rs;
      if (have) rs = st_[(int64_t)j * stride + srow];
      int f = have ? rs.flag : 0;
      double M = have ? rs.m : -INFINITY;
      for (int o = 32; o > 0; o >>= 1) {
        M = fmax(M, __shfl_xor(M, o, 64));
        f |= __shfl_xor(f, o, 64);
      }
      const double c = (have && rs.s > 0.0) ? exp(rs.m - M) : 0.0;
      double cs = have ? c * rs.s : 0.0, csz = have ? c * rs.sz : 0.0;
      for (int o = 32; o > 0; o >>= 1) {
        cs += __shfl_xor(cs, o, 64);
        csz += __shfl_xor(csz, o, 64);
      }
      s_c[j] = c;
      if (j == 0) {
        s_flag = f;
        s_res[0] = M;
        s_res[1] = cs;
        s_res[2] = csz;
      }
    }
    __syncthreads();
  };
  merge_stats();
  if (s_flag && pos != nullptr) {  // uniform: a flagged row the second pass may have taken
    const int k = pos[row];
    if (k >= 0) {
      const int64_t n2 = min((int64_t)*count2, (int64_t)cap2);
      st_ = stats2;
      O_ = O2;
      Sv_ = forward_splits_wave(n2, V, max_splits2);
      stride = compact_stride(n2);
      srow = k;
      early = false;
      __syncthreads();  // every thread has read s_flag
      merge_stats();
    }
  }
  if (s_flag) {
    const RowResult r = row_exact<T>(h + row * H, W, b, yv, H, V, inv_tau, vout != nullptr, sm);
    const double l = (double)r.m + log(r.s);
    if (threadIdx.x == 0) {
      if (lp) lp[row] = (float)((double)r.zy - l);
      ent[row] = (float)(l - r.sz / r.s);
      if (lse_out) lse_out[row] = (float)l;
    }
    if (vout) {
      const float* os = sm + H;
      const double inv_s = 1.0 / r.s;
      for (int d = threadIdx.x; d < H; d += NT)
        vout[row * H + d] = (float)((double)ldf<T>(W, yc * H + d) - (double)os[d] * inv_s);
    }
    return;
  }
  // Rows of H a multiple of 4 go four columns per thread and step (wide
  // loads, more bytes in flight per thread); others one column at a time.
  double zp = 0.0;
  if (lp) {
    if (vec) {
      for (int d4 = threadIdx.x; d4 < H / 4; d4 += NT) {
        const f32x4 hv = ld4f(h, row * H + 4 * d4), wv = ld4f(W, yc * H + 4 * d4);
#pragma unroll
        for (int k = 0; k < 4; ++k) zp += (double)hv[k] * (double)wv[k];
      }
    } else {
      for (int d = threadIdx.x; d < H; d += NT) zp += (double)ldf<T>(h, row * H + d) * (double)ldf<T>(W, yc * H + d);
    }
  }
  zp = block_sum(zp, s_red);
  if (threadIdx.x == 0) {
    const double S = s_res[1], SZ = s_res[2];
    const double l = s_res[0] + log(S);
    if (lp) {
      const float zy = (float)((zp + (b ? (double)ldf<T>(b, yc) : 0.0)) * (double)inv_tau);
      lp[row] = (float)((double)zy - l);
    }
    ent[row] = (float)(l - SZ / S);
    if (lse_out) lse_out[row] = (float)l;
    s_res[3] = 1.0 / S;
  }
  __syncthreads();
  if (vout) {
    const double inv_s = s_res[3];
    const float* Orow = O_ + srow * H;
    const int64_t sstride = stride * H;
    if (early) {
      const int d4 = threadIdx.x;
      if (d4 < H / 4) {
        double o[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int j = 0; j < (EARLY ? kEarlySplits : 1); ++j) {
          if (j < Sv_) {
            const double c = s_c[j];
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] += c * (double)opre[j][k];
          }
        }
        const f32x4 wy = ld4f(W, yc * H + 4 * d4);
        f32x4 r;
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = (float)((double)wy[k] - o[k] * inv_s);
        *reinterpret_cast<f32x4*>(vout + row * H + 4 * d4) = r;
      }
    } else if (vec) {
      for (int d4 = threadIdx.x; d4 < H / 4; d4 += NT) {
        double o[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
        for (int j = 0; j < Sv_; ++j) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(Orow + j * sstride + 4 * d4);
          const double c = s_c[j];
#pragma unroll
          for (int k = 0; k < 4; ++k) o[k] += c * (double)x[k];
        }
        const f32x4 wy = ld4f(W, yc * H + 4 * d4);
        f32x4 r;
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = (float)((double)wy[k] - o[k] * inv_s);
        *reinterpret_cast<f32x4*>(vout + row * H + 4 * d4) = r;
      }
    } else {
      for (int d = threadIdx.x; d < H; d += NT) {
        double o = 0.0;
#pragma unroll 8
        for (int j = 0; j < Sv_; ++j) o += s_c[j] * (double)Orow[j * sstride + d];
        vout[row * H + d] = (float)((double)ldf<T>(W, yc * H + d) - o * inv_s);
      }
    }
  }
}


// grad_h of the compacted rows k < *count_dev after the accumulator pass over
// them (stats and O with the row stride compact_stride(count) and
// forward_splits(count, V, max_splits) splits): the split merge of the
// accumulator as in combine_kernel, v = W_y - O/s, and
// grad_h[idx[k]] = (g_k / tau) v with g_k / tau = tok[k].gs and y = tok[k].y.
// A row any split flagged is recomputed exactly from h row idx[k].
template <typename T>
__global__ __launch_bounds__(NT) void grad_h_compact_kernel(const RowStats* __restrict__ stats,
                                                            const float* __restrict__ O, int max_splits, int H, int V,
                                                            const T* __restrict__ h, const T* __restrict__ W,
                                                            const T* __restrict__ b, float inv_tau,
                                                            const int* __restrict__ idx,
                                                            const TokData* __restrict__ tok,
                                                            const int* __restrict__ count_dev, T* __restrict__ gh) {
  extern __shared__ float sm[];
  const int64_t n = *count_dev;
  const int64_t k = blockIdx.x;
  if (k >= n) return;  // uniform
  const int Sv = forward_splits_wave(n, V, max_splits);
  const int64_t stride = compact_stride(n);
  __shared__ double s_c[64];
  __shared__ double s_res[2];
  __shared__ int s_flag;
  const int64_t src = idx[k];
  const TokData td = tok[k];
  const int64_t yc = td.y < 0 ? 0 : (td.y >= V ? V - 1 : td.y);
  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    const bool have = j < Sv;
    RowStats rs;
    if (have) rs = stats[(int64_t)j * stride + k];
    int f = have ? rs.flag : 0;
    double M = have ? rs.m : -INFINITY;
    for (int o = 32; o > 0; o >>= 1) {
      M = fmax(M, __shfl_xor(M, o, 64));
      f |= __shfl_xor(f, o, 64);
    }
    const double c = (have && rs.s > 0.0) ? exp(rs.m - M) : 0.0;
    double cs = have ? c * rs.s : 0.0;
    for (int o = 32; o > 0; o >>= 1) cs += __shfl_xor(cs, o, 64);
    s_c[j] = c;
    if (j == 0) {
      s_flag = f;
      s_res[0] = 1.0 / cs;
    }
  }
  __syncthreads();
  const float gs = td.gs;
  T* out = gh + src * H;
  if (s_flag) {
    const RowResult r = row_exact<T>(h + src * H, W, b, td.y, H, V, inv_tau, true, sm);
    const float* os = sm + H;
    const double inv_s = 1.0 / r.s;
    for (int d = threadIdx.x; d < H; d += NT)
      out[d] = (T)(gs * (float)((double)ldf<T>(W, yc * H + d) - (double)os[d] * inv_s));
    return;
  }
  const double inv_s = s_res[0];
  const float* Orow = O + k * H;
  const int64_t sstride = stride * H;
  for (int d = threadIdx.x; d < H; d += NT) {
    double o = 0.0;
    for (int j = 0; j < Sv; ++j) o += s_c[j] * (double)Orow[j * sstride + d];
    out[d] = (T)(gs * (float)((double)ldf<T>(W, yc * H + d) - o * inv_s));
  }
}
// Rows the forward sweep flagged (a logit above the split's reference by more
// than the slack, in any split): numbered with an integer counter (their
// order varies between calls, each row's results do not), up to cap2 of them
// listed with their largest logit as the reference for the second pass;
// pos[row] = its number, or -1 (not flagged, or past cap2: then the merge
// recomputes the row on the vector ALU).
// The counter starts at zero: the forward sweep before the scan clears it.
__global__ __launch_bounds__(NT) void flag_scan_kernel(const RowStats* __restrict__ stats, int Sv, int64_t N,
                                                       int cap2, int* __restrict__ idx, float* __restrict__ mref,
                                                       int* __restrict__ pos, int* __restrict__ count) {
  static_assert(offsetof(RowStats, flag) == offsetof(RowStats, zmax) + 4, "zmax and flag adjacent");
  for (int64_t r = (int64_t)blockIdx.x * NT + threadIdx.x; r < N; r += (int64_t)gridDim.x * NT) {
    int f = 0;
    float zm = -INFINITY;
    // (zmax, flag) of each split, eight loads in flight at a time
    auto zf = [&](int j) { return *reinterpret_cast<const float2*>(&stats[(int64_t)j * N + r].zmax); };
    int j = 0;
    for (; j + 8 <= Sv; j += 8) {
      float2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = zf(j + u);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        zm = fmaxf(zm, v[u].x);
        f |= __float_as_int(v[u].y);
      }
    }
    for (; j < Sv; ++j) {
      const float2 v = zf(j);
      zm = fmaxf(zm, v.x);
      f |= __float_as_int(v.y);
    }
    int k = -1;
    if (f) {
      k = atomicAdd(count, 1);
      if (k < cap2) {
        idx[k] = (int)r;
        mref[k] = zm;
      } else {
        k = -1;
      }
    }
    pos[r] = k;
  }
}

// ---------------------------------------------------------------------------
// Loss stage
// ---------------------------------------------------------------------------
struct TokEval {
  bool M, R, E;
  bool clipped;   // GMPO: token predicate on ratio tokens; token-clip losses: ratio held at a bound
  double c;       // GMPO: clipped log-ratio; token-clip losses: policy term -min(rho A, clip(rho) A)
  double rho;     // token-clip losses: the token ratio exp(lr32)
  double lr;      // log-ratio value
  double kl, dkl;
};

// Per-token quantities. GMPO (Liger PR #1320): clip in log space, advantage
// dependent and one sided. GRPO / BNPO / DAPO: the Tinker GSPO page's clipped
// objective with the token's own ratio, decided on exp(lr32) in fp64 against
// the fp32 ratio bounds. K3 KL, optionally bias corrected (Liger PR #1320,
// "The implementation"): weighted by the token's importance ratio. lr32 = fp32(lp - old) is the predicate
// operand; ties are not clipped; A = 0 gives no term.
__device__ __forceinline__ TokEval eval_tok(const LossParams& p, int64_t t, const float* lp, const float* old,
                                            const float* ref, const uint8_t* comp, const uint8_t* ratio,
                                            const uint8_t* emask, float A) {
  TokEval e;
  const float lp32 = lp[t];
  const float old32 = old ? old[t] : lp32;
  const float lr32 = __fsub_rn(lp32, old32);
  e.M = comp[t] != 0;
  e.R = ratio ? ratio[t] != 0 : e.M;
  e.E = emask ? emask[t] != 0 : true;
  e.lr = (double)lr32;
  if (token_clip_loss(p.loss_type)) {
    const double rho = exp((double)lr32);
    const double hi64 = (double)p.hi32, lo64 = (double)p.lo32, A64 = (double)A;
    const bool hi = A > 0.f && rho > hi64;
    const bool lo = A < 0.f && rho < lo64;
    e.clipped = e.M && (hi || lo);
    e.rho = rho;
    e.c = A == 0.f ? 0.0 : (hi ? -hi64 * A64 : (lo ? -lo64 * A64 : -rho * A64));
  } else {
    const bool hi = A > 0.f && lr32 > p.eh32;
    const bool lo = A < 0.f && lr32 < -p.el32;
    e.clipped = e.R && (hi || lo);
    e.rho = 0.0;
    e.c = hi ? (double)p.eh32 : (lo ? -(double)p.el32 : (double)lr32);
  }
  if (ref) {
    const double x = (double)ref[t] - (double)lp32;
    const double ex = exp(x);
    const double k3 = ex - x - 1.0;
    if (p.kl_bc) {
      // rho K3 with rho = exp(lp - old): d/dlp = rho K3 + rho (1 - e^x) = -rho x
      const double rho = old ? exp((double)lp32 - (double)old32) : 1.0;
      e.kl = rho * k3;
      e.dkl = -rho * x;
    } else {
      e.kl = k3;
      e.dkl = 1.0 - ex;
    }
  } else {
    e.kl = 0.0;
    e.dkl = 0.0;
  }
  return e;
}

// grid (Bc, St): partial sums of sequence i over token segment s.
__global__ __launch_bounds__(NT) void seq_partial_kernel(LossParams p, const float* __restrict__ lp,
                                                         const float* __restrict__ old, const float* __restrict__ ref,
                                                         const uint8_t* __restrict__ comp,
                                                         const uint8_t* __restrict__ ratio,
                                                         const uint8_t* __restrict__ emask,
                                                         const float* __restrict__ adv,
                                                         const float* __restrict__ tadv, int St,
                                                         SeqPart* __restrict__ part) {
  __shared__ double redd[NT];
  __shared__ int redi[NT];
  const int i = blockIdx.x, s = blockIdx.y;
  const int64_t T = p.T;
  const int64_t L = (T + St - 1) / St;
  const int64_t a = (int64_t)s * L, b = min(T, a + L);
  const float Aseq = p.token_adv ? 0.f : adv[i];
  double sc = 0.0, slr = 0.0, skl = 0.0, sap = 0.0, san = 0.0;
  int cm = 0, cr = 0, ck = 0, cc = 0, cp = 0, cn = 0;
  for (int64_t k = a + threadIdx.x; k < b; k += NT) {
    const int64_t t = (int64_t)i * T + k;
    const float A = p.token_adv ? tadv[t] : Aseq;
    const TokEval e = eval_tok(p, t, lp, old, ref, comp, ratio, emask, A);
    if (p.token_adv && e.M) {
      cp += A > 0.f ? 1 : 0;
      cn += A < 0.f ? 1 : 0;
      if (e.E) {
        sap += A > 0.f ? (double)A : 0.0;
        san += A < 0.f ? (double)A : 0.0;
      }
    }
    if (e.R) {
      if (!token_clip_loss(p.loss_type)) sc += e.c;
      slr += e.lr;
      cr += 1;
    }
    if (token_clip_loss(p.loss_type) && e.M && e.E) sc += e.c;
    if (e.M) {
      skl += e.kl;
      cm += 1;
      ck += e.E ? 1 : 0;
      cc += e.clipped ? 1 : 0;
    }
  }
  SeqPart out;
  out.sum_c = block_sum(sc, redd);
  out.sum_lr = block_sum(slr, redd);
  out.sum_kl = block_sum(skl, redd);
  out.cnt_m = block_sum(cm, redi);
  out.cnt_r = block_sum(cr, redi);
  out.cnt_k = block_sum(ck, redi);
  out.cnt_clip = block_sum(cc, redi);
  out.sum_apos = block_sum(sap, redd);
  out.sum_aneg = block_sum(san, redd);
  out.cnt_pos = block_sum(cp, redi);
  out.cnt_neg = block_sum(cn, redi);
  if (threadIdx.x == 0) part[(int64_t)i * St + s] = out;
}

// One block: per-sequence scalars (GMPO r_i, GSPO s_i; the token-clip
// losses' masked sum of policy terms), gradient coefficients, loss and metric
// contributions of the chunk. The first chunk
// (init) sets the batch accumulators instead of adding to them; the last one
// (loss_out != NULL) also writes the loss and the metrics, with the entropy
// threshold from thr_dev (NaN when NULL: the mask is off).
__global__ __launch_bounds__(NT) void seq_final_kernel(LossParams p, int64_t Bc, int St,
                                                       const SeqPart* __restrict__ part,
                                                       const float* __restrict__ adv, SeqCoef* __restrict__ coef,
                                                       LossAcc* __restrict__ acc, int init,
                                                       const float* __restrict__ thr_dev, float* __restrict__ loss_out,
                                                       float* __restrict__ metrics) {
  __shared__ double redd[NT];
  __shared__ unsigned long long redu[NT];
  double loss = 0.0, slr = 0.0, mkl = 0.0;
  unsigned long long na = 0, nc = 0, nk = 0, ncs = 0;
  for (int64_t i = threadIdx.x; i < Bc; i += NT) {
    double sum_c = 0.0, sum_lr = 0.0, sum_kl = 0.0, sum_ap = 0.0, sum_an = 0.0;
    long long cm = 0, cr = 0, ck = 0, cc = 0, cpos = 0, cneg = 0;
    for (int s = 0; s < St; ++s) {
      const SeqPart q = part[i * St + s];
      sum_c += q.sum_c;
      sum_lr += q.sum_lr;
      sum_kl += q.sum_kl;
      sum_ap += q.sum_apos;
      sum_an += q.sum_aneg;
      cm += q.cnt_m;
      cr += q.cnt_r;
      ck += q.cnt_k;
      cc += q.cnt_clip;
      cpos += q.cnt_pos;
      cneg += q.cnt_neg;
    }
    const double n = (double)(cm > 0 ? cm : 1);
    const double nt = (double)(cr > 0 ? cr : 1);
    const double K = (double)ck;
    const float A32 = p.token_adv ? 0.f : adv[i];
    const double A = (double)A32;
    double w;
    if (token_mean_loss(p.loss_type))
      w = 1.0 / (double)(p.norm_tokens > 0 ? (unsigned long long)p.norm_tokens
                                           : (*p.ntok_dev > 0 ? *p.ntok_dev : 1ull));
    else if (p.loss_type == 2 || p.reduction == 0)
      w = 1.0 / ((double)p.B_total * n);
    else
      w = 1.0;
    const double seq_lr = sum_lr / nt;
    double policy_seq, pol;
    long long clip_tok;
    int clip_any = 0;
    int held = 0;  // GSPO with per-token advantages: bit 0 s > hi (A_t > 0 held), bit 1 s < lo (A_t < 0 held)
    if (token_clip_loss(p.loss_type)) {
      // GRPO / BNPO / DAPO: sum_c already holds the masked policy terms
      policy_seq = 0.0;
      pol = -w;  // times the token's A_t and ratio where it is not held at a bound
      clip_tok = cc;
    } else if (p.token_adv) {
      // GSPO-token with per-token advantages: min(s A_t, clip(s) A_t) is
      // s A_t except min(s, hi) A_t for A_t > 0 and max(s, lo) A_t for A_t < 0
      const double sr = exp(seq_lr);
      const double lo = (double)p.lo32, hi = (double)p.hi32;
      const bool hp = sr > hi, hn = sr < lo;
      policy_seq = 0.0;
      sum_c = (sum_ap != 0.0 ? -sum_ap * fmin(sr, hi) : 0.0) + (sum_an != 0.0 ? -sum_an * fmax(sr, lo) : 0.0);
      pol = -sr * w;  // times A_t where the token is not held
      clip_tok = (hp ? cpos : 0) + (hn ? cneg : 0);
      clip_any = (hp || hn) ? 1 : 0;
      held = (hp ? 1 : 0) | (hn ? 2 : 0);
    } else if (p.loss_type == 0) {
      // GMPO: r = exp(masked mean of the clipped log-ratios) (PR #1320)
      const double r = A32 != 0.f ? exp(sum_c / nt) : 1.0;
      policy_seq = A32 != 0.f ? -A * r : 0.0;
      pol = A32 != 0.f ? -A * r * K * w / nt : 0.0;
      clip_tok = cc;
    } else {
      // GSPO-token: s = exp(mean log-ratio), clip(s, 1-eps_l, 1+eps_h) (Tinker GSPO)
      const double sr = exp(seq_lr);
      const double lo = (double)p.lo32, hi = (double)p.hi32;
      const bool clipped = (A32 > 0.f && sr > hi) || (A32 < 0.f && sr < lo);
      const double scl = fmin(fmax(sr, lo), hi);
      policy_seq = -fmin(sr * A, scl * A);
      pol = clipped ? 0.0 : -A * sr * w;
      clip_tok = clipped ? cm : 0;
      clip_any = (sr < lo || sr > hi) ? 1 : 0;
    }
    const bool tok_terms = token_clip_loss(p.loss_type) || p.token_adv;
    loss += tok_terms ? w * (sum_c + p.beta * sum_kl) : w * (policy_seq * K + p.beta * sum_kl);
    slr += seq_lr;
    mkl += sum_kl / n;
    na += (unsigned long long)cm;
    nc += (unsigned long long)clip_tok;
    nk += (unsigned long long)ck;
    ncs += (unsigned long long)clip_any;
    SeqCoef sc;
    sc.pol = pol;
    sc.wbeta = w * p.beta;
    sc.adv = A32;
    sc.pad = held;
    coef[i] = sc;
  }
  loss = block_sum(loss, redd);
  slr = block_sum(slr, redd);
  mkl = block_sum(mkl, redd);
  na = block_sum(na, redu);
  nc = block_sum(nc, redu);
  nk = block_sum(nk, redu);
  ncs = block_sum(ncs, redu);
  if (threadIdx.x == 0) {
    LossAcc a;
    if (init) {
      a.loss = loss;
      a.slr = slr;
      a.mkl = mkl;
      a.n_active = na;
      a.n_clip = nc;
      a.n_kept = nk;
      a.n_clipseq = ncs;
    } else {
      a = *acc;
      a.loss += loss;
      a.slr += slr;
      a.mkl += mkl;
      a.n_active += na;
      a.n_clip += nc;
      a.n_kept += nk;
      a.n_clipseq += ncs;
    }
    a.thr = 0.f;
    a.pad = 0;
    *acc = a;
    if (loss_out) {
      loss_out[0] = (float)a.loss;
      const float den = (float)(a.n_active > 0 ? a.n_active : 1ull);
      metrics[0] = (float)a.n_clip / den;
      metrics[1] = (float)(a.slr / (double)p.B_total);
      metrics[2] = (float)((double)a.n_clipseq / (double)p.B_total);
      metrics[3] = (float)(a.mkl / (double)p.B_total);
      metrics[4] = thr_dev ? *thr_dev : __int_as_float(0x7fc00000);
      metrics[5] = a.n_active > 0 ? (float)a.n_kept / den : 0.f;
      metrics[6] = (float)a.n_active;
      metrics[7] = (float)a.n_clip;
    }
  }
}

// Per 32-token block: g_t = dL/dlp_t (GMPO: pol on unclipped ratio tokens;
// GSPO-token: pol on kept completion tokens; GRPO / BNPO / DAPO: pol times the
// token's ratio on kept completion tokens not held at a bound; plus
// w beta (1 - e^{ref - lp})
// on completion tokens), the block's count of g != 0 (cnt32, when given) and,
// when gh is given, grad_h = (g / tau) v for its rows.
constexpr int TB = 32;  // tokens per block of the token kernel

template <typename T>
__global__ __launch_bounds__(NT) void token_kernel(LossParams p, int64_t Nc, const float* __restrict__ lp,
                                                   const float* __restrict__ old, const float* __restrict__ ref,
                                                   const uint8_t* __restrict__ comp, const uint8_t* __restrict__ ratio,
                                                   const uint8_t* __restrict__ emask,
                                                   const float* __restrict__ tadv,
                                                   const SeqCoef* __restrict__ coef, float* __restrict__ g,
                                                   int* __restrict__ cnt32, const float* __restrict__ v, int H,
                                                   float inv_tau, T* __restrict__ gh) {
  __shared__ float s_g[TB];
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  // blockIdx.y = column slice of grad_h; every slice evaluates g for its 32
  // tokens (cheap), slice 0 alone writes g and the counts
  const bool writer = blockIdx.y == 0;
  if (threadIdx.x < TB) {
    const int64_t t = t0 + threadIdx.x;
    float gv32 = 0.f;
    if (t < Nc) {
      const int64_t i = t / p.T;
      const SeqCoef c = coef[i];
      const float A = p.token_adv ? tadv[t] : c.adv;
      const TokEval e = eval_tok(p, t, lp, old, ref, comp, ratio, emask, A);
      double gv = 0.0;
      if (token_clip_loss(p.loss_type)) {
        if (e.M && e.E && !e.clipped && A != 0.f) gv = c.pol * (double)A * e.rho;
      } else if (p.token_adv) {
        const bool held = (A > 0.f && (c.pad & 1)) || (A < 0.f && (c.pad & 2));
        if (e.M && e.E && !held && A != 0.f) gv = c.pol * (double)A;
      } else if (p.loss_type == 0) {
        if (e.R && !e.clipped) gv = c.pol;
      } else {
        if (e.M && e.E) gv = c.pol;
      }
      if (e.M) gv += c.wbeta * e.dkl;
      gv32 = (float)gv;
      if (writer) g[t] = gv32;
    }
    s_g[threadIdx.x] = gv32;
    if (cnt32 && writer) {
      const unsigned long long m = __ballot(gv32 != 0.f);
      if (threadIdx.x == 0) cnt32[blockIdx.x] = __popcll(m);
    }
  }
  if (gh == nullptr) return;  // uniform
  __syncthreads();
  const int rows = (int)min((int64_t)TB, Nc - t0);
  const int HS = gridDim.y, Hs = H / HS, c0 = blockIdx.y * Hs;  // the launcher makes Hs a multiple of 4
  const int64_t base = t0 * H + c0;
  if (v == nullptr) {  // uniform: grad_h of the rows with g != 0 comes later (compacted pass); zeros here
    for (int e = threadIdx.x; e < rows * Hs; e += NT) {
      const int r = e / Hs, col = e - r * Hs;
      gh[base + (int64_t)r * H + col] = (T)0.f;
    }
    return;
  }
  if ((Hs & 3) == 0) {
    for (int e = threadIdx.x * 4; e < rows * Hs; e += NT * 4) {
      const int r = e / Hs, col = e - r * Hs;
      const float sc = s_g[r] * inv_tau;
      const int64_t k = base + (int64_t)r * H + col;
      const float4 x = *reinterpret_cast<const float4*>(v + k);
      if constexpr (sizeof(T) == 2) {
        bf16x4 u;
        u[0] = (__bf16)(sc * x.x);
        u[1] = (__bf16)(sc * x.y);
        u[2] = (__bf16)(sc * x.z);
        u[3] = (__bf16)(sc * x.w);
        *reinterpret_cast<bf16x4*>(gh + k) = u;
      } else {
        *reinterpret_cast<float4*>(gh + k) = make_float4(sc * x.x, sc * x.y, sc * x.z, sc * x.w);
      }
    }
  } else {
    for (int e = threadIdx.x; e < rows * Hs; e += NT) {
      const int r = e / Hs, col = e - r * Hs;
      gh[base + (int64_t)r * H + col] = (T)(s_g[r] * inv_tau * v[base + (int64_t)r * H + col]);
    }
  }
}

// ---------------------------------------------------------------------------
// Token compaction: tokens with g != 0, in order.
// ---------------------------------------------------------------------------
constexpr int CB = 1024;  // tokens per compaction block (32 token-kernel blocks)

// Each block sums the g != 0 counts of the 32-token blocks before it (fixed
// order), then each thread owns CB/NT = 4 consecutive tokens; an exclusive
// scan of the per-thread counts gives every kept token its slot. The last
// block writes the total.
__global__ __launch_bounds__(NT) void compact_scatter_kernel(const float* __restrict__ g, const float* __restrict__ lse,
                                                             const int64_t* __restrict__ y, int64_t N, float inv_tau,
                                                             const int* __restrict__ cnt32, int* __restrict__ idx,
                                                             TokData* __restrict__ tok, int* __restrict__ total) {
  __shared__ int sc[NT];
  __shared__ int red[NT];
  constexpr int PER = CB / NT;
  const int nprev = blockIdx.x * (CB / TB);
  int pre = 0;
  for (int k = threadIdx.x; k < nprev; k += NT) pre += cnt32[k];
  pre = block_sum(pre, red);
  const int64_t base = (int64_t)blockIdx.x * CB + (int64_t)threadIdx.x * PER;
  int c = 0;
  bool f[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int64_t t = base + k;
    f[k] = t < N && g[t] != 0.f;
    c += f[k] ? 1 : 0;
  }
  sc[threadIdx.x] = c;
  __syncthreads();
  for (int s = 1; s < NT; s <<= 1) {  // Hillis-Steele inclusive scan
    const int v = threadIdx.x >= s ? sc[threadIdx.x - s] : 0;
    __syncthreads();
    sc[threadIdx.x] += v;
    __syncthreads();
  }
  int pos = pre + sc[threadIdx.x] - c;
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == NT - 1) *total = pre + sc[NT - 1];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (f[k]) {
      const int64_t t = base + k;
      idx[pos] = (int)t;
      TokData td;
      td.lse = lse[t];
      td.gs = g[t] * inv_tau;
      td.y = (int)y[t];
      td.pad = 0;
      tok[pos] = td;
      ++pos;
    }
  }
}

// Natural-layout gather of compacted rows (generic path); rows past the count
// are zero.
template <typename T>
__global__ __launch_bounds__(NT) void gather_rows_kernel(const T* __restrict__ X, const int* __restrict__ idx,
                                                         const int* __restrict__ count_dev, int64_t cap, int H,
                                                         T* __restrict__ Xc) {
  const int n = *count_dev;
  for (int64_t k = blockIdx.x; k < cap; k += gridDim.x) {
    if (k >= ((int64_t)n + 31) / 32 * 32) return;
    for (int d = threadIdx.x; d < H; d += NT) Xc[k * H + d] = k < n ? X[(int64_t)idx[k] * H + d] : (T)0.f;
  }
}

// ---------------------------------------------------------------------------
// Batch-global quantile of the active entropies (torch.quantile linear
// interpolation in fp32), by MSB-first radix select over the whole grid on
// order-preserving integer keys: three digit passes (11, 11 and 10 bits),
// each a histogram kernel over all entries (workgroup histograms in LDS,
// added into one global histogram with integer atomics, so the counts do
// not depend on the order of the additions) and a one-workgroup scan that
// picks the digit of each of the two order statistics floor(rank) and
// ceil(rank). The scratch is a SelectState (thr first, so the threshold is
// read through a float pointer by the later kernels).
// ---------------------------------------------------------------------------
constexpr int SEL_BINS = 2048;

__device__ __forceinline__ unsigned f2key(float f) {
  const unsigned u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// Digit of pass p: bits [shift, shift + width) of the key.
__device__ __forceinline__ int sel_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ int sel_width(int pass) { return pass == 2 ? 10 : 11; }

__global__ __launch_bounds__(NT) void select_init_kernel(SelectState* __restrict__ s) {
  unsigned* hist = &s->hist[0][0];
  for (int k = threadIdx.x; k < 2 * SEL_BINS; k += NT) hist[k] = 0u;
  if (threadIdx.x == 0) {
    s->thr = __int_as_float(0x7fc00000);
    s->w = 0.f;
    s->pre[0] = s->pre[1] = 0u;
    s->n = 0ull;
    s->kk[0] = s->kk[1] = 0ull;
    s->done = 0;
  }
}

// Histogram of pass `pass` over the active entries whose key carries the
// prefix found so far (one histogram while both order statistics share it).
__global__ __launch_bounds__(NT) void select_hist_kernel(const float* __restrict__ ent,
                                                         const uint8_t* __restrict__ active, int64_t N,
                                                         SelectState* __restrict__ s, int pass) {
  __shared__ unsigned lh[2][SEL_BINS];
  if (s->done) return;  // uniform: no active entry
  const int shift = sel_shift(pass);
  const unsigned dmask = (1u << sel_width(pass)) - 1u;
  const int top = shift + sel_width(pass);
  const unsigned hmask = top >= 32 ? 0u : (0xffffffffu << top);
  const unsigned p0 = s->pre[0], p1 = s->pre[1];
  const bool same = p0 == p1;
  for (int k = threadIdx.x; k < 2 * SEL_BINS; k += NT) (&lh[0][0])[k] = 0u;
  __syncthreads();
  for (int64_t t = (int64_t)blockIdx.x * NT + threadIdx.x; t < N; t += (int64_t)gridDim.x * NT) {
    if (active[t] == 0) continue;
    const unsigned key = f2key(ent[t]);
    const unsigned d = (key >> shift) & dmask;
    if ((key & hmask) == p0) atomicAdd(&lh[0][d], 1u);
    if (!same && (key & hmask) == p1) atomicAdd(&lh[1][d], 1u);
  }
  __syncthreads();
  for (int k = threadIdx.x; k < (same ? 1 : 2) * SEL_BINS; k += NT) {
    const unsigned v = (&lh[0][0])[k];
    if (v != 0u) atomicAdd(&s->hist[0][0] + k, v);
  }
}

// Digit of pass `pass` for both order statistics from the global histogram;
// clears the histogram for the next pass. Pass 0 also counts the active
// entries and fixes the ranks; the last pass writes the threshold.
__global__ __launch_bounds__(NT) void select_scan_kernel(SelectState* __restrict__ s, int pass, float p32) {
  // The rank, its fraction and the interpolation are each rounded to fp32 as
  // torch.quantile rounds them: no multiply-add contraction here (it would
  // take the fraction of the unrounded product).
#pragma clang fp contract(off)
  constexpr int PER = SEL_BINS / NT;
  __shared__ unsigned long long red[4];
  __shared__ unsigned long long tsum[NT];
  // the state this kernel updates is kept in LDS and written back at the end
  // (no global value is read back after a write within the kernel)
  __shared__ unsigned long long sk[2];
  __shared__ unsigned spre[2];
  __shared__ float sw;
  if (s->done) return;  // uniform
  const int shift = sel_shift(pass);
  const unsigned p0 = s->pre[0], p1 = s->pre[1];
  const bool same = p0 == p1;
  if (pass == 0) {
    unsigned long long c = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) c += s->hist[0][threadIdx.x * PER + k];
    const unsigned long long n = block_sum(c, red);
    if (n == 0) {
      if (threadIdx.x == 0) {
        s->done = 1;
        s->thr = __int_as_float(0x7fc00000);
      }
      return;
    }
    // rank = p (n - 1) in fp32 as torch.quantile forms it; past 2^24 entries
    // fp32(n - 1) can round up to n, so both order statistics are clamped to
    // the last one
    const float rank = p32 * (float)(n - 1);
    const float rlo = floorf(rank);
    if (threadIdx.x == 0) {
      s->n = n;
      sw = rank - rlo;
      sk[0] = min((unsigned long long)rlo, n - 1);
      sk[1] = min((unsigned long long)ceilf(rank), n - 1);
    }
  } else if (threadIdx.x == 0) {
    sw = s->w;
    sk[0] = s->kk[0];
    sk[1] = s->kk[1];
  }
  if (threadIdx.x == 0) {
    spre[0] = p0;
    spre[1] = p1;
  }
  __syncthreads();
  for (int r = 0; r < 2; ++r) {
    const unsigned* hw = s->hist[same ? 0 : r];
    unsigned long long loc = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) loc += hw[threadIdx.x * PER + k];
    tsum[threadIdx.x] = loc;
    __syncthreads();
    for (int o = 1; o < NT; o <<= 1) {  // inclusive scan of the thread sums
      const unsigned long long v = threadIdx.x >= o ? tsum[threadIdx.x - o] : 0ull;
      __syncthreads();
      tsum[threadIdx.x] += v;
      __syncthreads();
    }
    const unsigned long long k = sk[r];
    unsigned long long cum = tsum[threadIdx.x] - loc;  // bins before this thread's
    __syncthreads();
    if (k >= cum && k < cum + loc) {  // exactly one thread holds the rank
      int b = threadIdx.x * PER;
      for (int j = 0; j < PER - 1; ++j, ++b) {
        if (k < cum + hw[b]) break;
        cum += hw[b];
      }
      sk[r] = k - cum;
      spre[r] |= (unsigned)b << shift;
    }
    __syncthreads();
  }
  for (int k = threadIdx.x; k < 2 * SEL_BINS; k += NT) (&s->hist[0][0])[k] = 0u;
  if (threadIdx.x == 0) {
    s->pre[0] = spre[0];
    s->pre[1] = spre[1];
    s->kk[0] = sk[0];
    s->kk[1] = sk[1];
    s->w = sw;
    if (pass == 2) {
      const float a = key2f(spre[0]);
      const float b = key2f(spre[1]);
      const float d = b - a;
      s->thr = sw < 0.5f ? __builtin_fmaf(sw, d, a) : __builtin_fmaf(sw - 1.0f, d, b);
    }
  }
}

__global__ __launch_bounds__(NT) void mask_kernel(const float* __restrict__ ent, const uint8_t* __restrict__ active,
                                                  int64_t N, const float* __restrict__ thr_dev,
                                                  uint8_t* __restrict__ mask) {
  const float thr = *thr_dev;
  for (int64_t t = (int64_t)blockIdx.x * NT + threadIdx.x; t < N; t += (int64_t)gridDim.x * NT)
    mask[t] = (active[t] != 0 && ent[t] >= thr) ? 1 : 0;
}

// Number of nonzero mask bytes (one block, fixed-order sum): the batch's
// completion tokens, the divisor of BNPO and of DAPO without a global count.
__global__ __launch_bounds__(NT) void count_mask_kernel(const uint8_t* __restrict__ m, int64_t N,
                                                        unsigned long long* __restrict__ out) {
  __shared__ unsigned long long red[NT];
  unsigned long long c = 0;
  const int64_t n16 = N / 16;
  const uint4* m16 = reinterpret_cast<const uint4*>(m);
  const bool aligned = (reinterpret_cast<uintptr_t>(m) & 15) == 0;
  int64_t done = 0;
  if (aligned) {
    for (int64_t k = threadIdx.x; k < n16; k += NT) {
      const uint4 v = m16[k];
      const unsigned w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) c += ((w4[j] >> (8 * b)) & 0xffu) != 0u;
    }
    done = n16 * 16;
  }
  for (int64_t k = done + threadIdx.x; k < N; k += NT) c += m[k] != 0;
  c = block_sum(c, red);
  if (threadIdx.x == 0) *out = c;
}

__global__ void store_thr_kernel(const float* __restrict__ thr_dev, float* __restrict__ thr_out) {
  if (threadIdx.x == 0) *thr_out = *thr_dev;
}

__global__ __launch_bounds__(NT) void copy_mask_kernel(const uint8_t* __restrict__ src, int64_t N,
                                                       uint8_t* __restrict__ dst) {
  for (int64_t t = (int64_t)blockIdx.x * NT + threadIdx.x; t < N; t += (int64_t)gridDim.x * NT)
    dst[t] = src[t] != 0 ? 1 : 0;
}

__global__ void set_nan_kernel(float* dst) {
  if (threadIdx.x == 0) *dst = __int_as_float(0x7fc00000);
}

inline unsigned grid_for(int64_t n, int per_block) {
  int64_t b = (n + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > 65535 * 16) b = 65535 * 16;
  return (unsigned)b;
}

}  // namespace

hipError_t launch_flag_scan(const RowStats* stats, int Sv, int64_t N, int cap2, int* idx, float* mref, int* pos,
                            int* count, hipStream_t st) {
  if (N > 0)
    hipLaunchKernelGGL(flag_scan_kernel, dim3(grid_for(N, NT)), dim3(NT), 0, st, stats, Sv, N, cap2, idx, mref, pos,
                       count);
  return hipGetLastError();
}

hipError_t launch_combine(int dtype, const RowStats* stats, const float* O, int Sv, int64_t N, int H, int V,
                          const void* h, const void* W, const void* b, float inv_tau, const int64_t* y, float* lp,
                          float* ent, float* lse, float* vout, hipStream_t st, const FlaggedPass* fp) {
  const int* pos = fp ? fp->pos : nullptr;
  const RowStats* st2 = fp ? fp->stats : nullptr;
  const float* O2 = fp ? fp->O : nullptr;
  const int* cnt2 = fp ? fp->count : nullptr;
  const int cap2 = fp ? fp->cap : 0, ms2 = fp ? fp->max_splits : 1;
  if (N <= 0) return hipSuccess;
  const size_t lds = row_exact_smem_bytes(H);
  const bool early = Sv > 1 && Sv <= kEarlySplits && vout != nullptr;
  if (dtype == 0) {
    const float *hh = (const float*)h, *WW = (const float*)W, *bb = (const float*)b;
    if (early)
      hipLaunchKernelGGL((combine_kernel<float, true>), dim3((unsigned)N), dim3(NT), lds, st, stats, O, Sv, N, H, V,
                         hh, WW, bb, inv_tau, y, lp, ent, lse, vout, pos, st2, O2, cnt2, cap2, ms2);
    else
      hipLaunchKernelGGL((combine_kernel<float, false>), dim3((unsigned)N), dim3(NT), lds, st, stats, O, Sv, N, H, V,
                         hh, WW, bb, inv_tau, y, lp, ent, lse, vout, pos, st2, O2, cnt2, cap2, ms2);
  } else {
    const __bf16 *hh = (const __bf16*)h, *WW = (const __bf16*)W, *bb = (const __bf16*)b;
    if (early)
      hipLaunchKernelGGL((combine_kernel<__bf16, true>), dim3((unsigned)N), dim3(NT), lds, st, stats, O, Sv, N, H, V,
                         hh, WW, bb, inv_tau, y, lp, ent, lse, vout, pos, st2, O2, cnt2, cap2, ms2);
    else
      hipLaunchKernelGGL((combine_kernel<__bf16, false>), dim3((unsigned)N), dim3(NT), lds, st, stats, O, Sv, N, H,
                         V, hh, WW, bb, inv_tau, y, lp, ent, lse, vout, pos, st2, O2, cnt2, cap2, ms2);
  }
  return hipGetLastError();
}

hipError_t launch_grad_h_compact(int dtype, const RowStats* stats, const float* O, int max_splits, int64_t cap, int H,
                                 int V, const void* h, const void* W, const void* b, float inv_tau, const int* idx,
                                 const TokData* tok, const int* count_dev, void* gh, hipStream_t st) {
  if (cap <= 0) return hipSuccess;
  const size_t lds = row_exact_smem_bytes(H);
  if (dtype == 0)
    hipLaunchKernelGGL((grad_h_compact_kernel<float>), dim3((unsigned)cap), dim3(NT), lds, st, stats, O, max_splits,
                       H, V, (const float*)h, (const float*)W, (const float*)b, inv_tau, idx, tok, count_dev,
                       (float*)gh);
  else
    hipLaunchKernelGGL((grad_h_compact_kernel<__bf16>), dim3((unsigned)cap), dim3(NT), lds, st, stats, O, max_splits,
                       H, V, (const __bf16*)h, (const __bf16*)W, (const __bf16*)b, inv_tau, idx, tok, count_dev,
                       (__bf16*)gh);
  return hipGetLastError();
}

hipError_t launch_loss_seq_partial(const LossParams& p, int64_t Bc, const float* lp, const float* old,
                                   const float* ref, const uint8_t* comp, const uint8_t* ratio,
                                   const uint8_t* emask, const float* adv, const float* tadv, int St,
                                   SeqPart* part, hipStream_t st) {
  hipLaunchKernelGGL(seq_partial_kernel, dim3((unsigned)Bc, (unsigned)St), dim3(NT), 0, st, p, lp, old, ref, comp,
                     ratio, emask, adv, tadv, St, part);
  return hipGetLastError();
}

hipError_t launch_loss_seq_final(const LossParams& p, int64_t Bc, int St, const SeqPart* part, const float* adv,
                                 SeqCoef* coef, LossAcc* acc, bool init, const float* thr_dev, float* loss_out,
                                 float* metrics, hipStream_t st) {
  hipLaunchKernelGGL(seq_final_kernel, dim3(1), dim3(NT), 0, st, p, Bc, St, part, adv, coef, acc, init ? 1 : 0,
                     thr_dev, loss_out, metrics);
  return hipGetLastError();
}

hipError_t launch_loss_tokens(int dtype, const LossParams& p, int64_t Bc, const float* lp, const float* old,
                              const float* ref, const uint8_t* comp, const uint8_t* ratio, const uint8_t* emask,
                              const float* tadv, const SeqCoef* coef, float* g, int* cnt32, const float* v, int H,
                              float inv_tau, void* gh, hipStream_t st) {
  const int64_t Nc = Bc * p.T;
  const unsigned grid = (unsigned)((Nc + TB - 1) / TB);
  // few token blocks: split grad_h's columns over more workgroups (slices of
  // a multiple of 4 columns) so the copy-like part fills the chip
  unsigned hs = 1;
  if (gh != nullptr)
    while (grid * hs * 2 <= 2048 && H % (int)(8 * hs) == 0) hs *= 2;
  const dim3 grid2(grid, hs);
  if (dtype == 0)
    hipLaunchKernelGGL((token_kernel<float>), grid2, dim3(NT), 0, st, p, Nc, lp, old, ref, comp, ratio, emask,
                       tadv, coef, g, cnt32, v, H, inv_tau, (float*)gh);
  else
    hipLaunchKernelGGL((token_kernel<__bf16>), grid2, dim3(NT), 0, st, p, Nc, lp, old, ref, comp, ratio, emask,
                       tadv, coef, g, cnt32, v, H, inv_tau, (__bf16*)gh);
  return hipGetLastError();
}

size_t compact_scratch_bytes(int64_t N) { return (size_t)((N + TB - 1) / TB) * sizeof(int); }

hipError_t launch_compact_scatter(const float* g, const float* lse, const int64_t* y, int64_t N, float inv_tau,
                                  const int* cnt32, int* idx, TokData* tok, int* count_dev, hipStream_t st) {
  const int64_t nb = (N + CB - 1) / CB;
  hipLaunchKernelGGL(compact_scatter_kernel, dim3((unsigned)nb), dim3(NT), 0, st, g, lse, y, N, inv_tau, cnt32, idx,
                     tok, count_dev);
  return hipGetLastError();
}

hipError_t launch_gather_rows(int dtype, const void* X, const int* idx, const int* count_dev, int64_t cap, int H,
                              void* Xc, hipStream_t st) {
  // the rows are known only on the device: a bounded grid walks them
  const unsigned grid = (unsigned)(cap < 4096 ? (cap > 0 ? cap : 1) : 4096);
  if (dtype == 0)
    hipLaunchKernelGGL((gather_rows_kernel<float>), dim3(grid), dim3(NT), 0, st, (const float*)X, idx, count_dev,
                       cap, H, (float*)Xc);
  else
    hipLaunchKernelGGL((gather_rows_kernel<__bf16>), dim3(grid), dim3(NT), 0, st, (const __bf16*)X, idx, count_dev,
                       cap, H, (__bf16*)Xc);
  return hipGetLastError();
}

hipError_t launch_entropy_select(const float* ent, const uint8_t* active, int64_t N, float p32, SelectState* state,
                                 hipStream_t st) {
  // workgroups: about eight entries per thread, at most 1024 workgroups
  int64_t g = (N + NT * 8 - 1) / (NT * 8);
  g = g < 1 ? 1 : (g > 1024 ? 1024 : g);
  hipLaunchKernelGGL(select_init_kernel, dim3(1), dim3(NT), 0, st, state);
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(select_hist_kernel, dim3((unsigned)g), dim3(NT), 0, st, ent, active, N, state, pass);
    hipLaunchKernelGGL(select_scan_kernel, dim3(1), dim3(NT), 0, st, state, pass, p32);
  }
  return hipGetLastError();
}

hipError_t launch_entropy_mask(const float* ent, const uint8_t* active, int64_t N, const float* thr_dev,
                               uint8_t* mask, hipStream_t st) {
  hipLaunchKernelGGL(mask_kernel, dim3(grid_for(N, NT)), dim3(NT), 0, st, ent, active, N, thr_dev, mask);
  return hipGetLastError();
}

hipError_t launch_count_mask(const uint8_t* m, int64_t N, unsigned long long* out, hipStream_t st) {
  hipLaunchKernelGGL(count_mask_kernel, dim3(1), dim3(NT), 0, st, m, N, out);
  return hipGetLastError();
}

hipError_t launch_store_thr(const float* thr_dev, float* thr_out, hipStream_t st) {
  hipLaunchKernelGGL(store_thr_kernel, dim3(1), dim3(64), 0, st, thr_dev, thr_out);
  return hipGetLastError();
}

hipError_t launch_copy_mask(const uint8_t* src, int64_t N, uint8_t* dst, hipStream_t st) {
  hipLaunchKernelGGL(copy_mask_kernel, dim3(grid_for(N, NT)), dim3(NT), 0, st, src, N, dst);
  return hipGetLastError();
}

hipError_t launch_set_nan(float* dst, hipStream_t st) {
  hipLaunchKernelGGL(set_nan_kernel, dim3(1), dim3(64), 0, st, dst);
  return hipGetLastError();
}

}  // namespace plp
