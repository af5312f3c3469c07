// Forward sweep of the LM head on the matrix cores (gfx950): the kernel
// templates and their launches over the supported hidden sizes. The
// single-role kernel (four waves) serves the statistics-only passes; the
// two-role kernel (eight waves) the passes with the grad_h accumulator. The
// tile machinery and the schedule are described in mfma_tile.h.
#pragma once

#include "mfma_tile.h"

namespace plp {

namespace {

// Forward sweep, statistics only: per token row, running
// (sum 2^{z2-m2}, sum 2^{z2-m2} z2) against the reference m2 (z2 = z log2 e).
// Grid: (row blocks) x Sv vocabulary splits in the order of forward_block.
template <int KB, bool HAS_BIAS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_mfma_kernel(const __bf16* __restrict__ h, const __bf16* __restrict__ Wf,
                     const __bf16* __restrict__ bias, int64_t N, int V, float inv_tau, int Sv,
                     int tiles_per_split, RowStats* __restrict__ stats, int* __restrict__ clear_count) {
  constexpr int H = 128 * KB;
  if (clear_count && blockIdx.x == 0 && threadIdx.x == 0) *clear_count = 0;  // for the flag scan that follows
  constexpr int DS = Stage<KB>::DS;  // columns per wave
  constexpr int KS = DS / 16;        // 16-wide contraction steps per wave
  __shared__ f32x4 s_part[NW][2][4][64];
  __shared__ float s_x[2 * NW * 64];
  // the partials buffer is reused for the final cross-wave sums
  double* s_xd = reinterpret_cast<double*>(&s_part[0][0][0][0]);   // [NW][2][64]

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, c = lane & 31;
  const int nbq = w & 1, kh = w >> 1;  // quarter this wave reduces: row block nbq, tile-row half kh
  int64_t rb;
  int sv;
  if (!forward_block((N + BQ - 1) / BQ, Sv, rb, sv)) return;  // uniform: no block for this workgroup
  const int64_t q0 = rb * BQ;
  const int d0 = w * DS;
  const int n_tiles = (V + BK - 1) / BK;
  const int t_begin = sv * tiles_per_split;
  const int t_end = min(n_tiles, t_begin + tiles_per_split);

  // Resident h fragments (B operand of S^T): rows q0 + 32nb + c, cols
  // d0 + 16ks + 8hh; rows past N repeat row N - 1 (their results are never
  // stored). The first streamed tile is loaded in the same k-step order, so
  // the first MFMAs wait only for their own operands.
  const bool any = t_begin < t_end;
  bf16x8 q[2][KS];
  bf16x8 a[KS];
  {
    const auto rh = frag_rsrc(h + q0 * H, BQ * H * 2);
    const int row0 = (int)min((int64_t)c, N - 1 - q0), row1 = (int)min((int64_t)(32 + c), N - 1 - q0);
    // an empty split loads nothing (zero range)
    const auto ra = frag_rsrc(frag_ptr<KB>(Wf, any ? t_begin : 0, w, 0, 0), any ? KS * 1024 : 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      q[0][ks] = ld_buf(rh, (row0 * H + d0 + 8 * hh) * 2, 32 * ks);
      q[1][ks] = ld_buf(rh, (row1 * H + d0 + 8 * hh) * 2, 32 * ks);
      a[ks] = ld_buf(ra, lane * 16, ks * 1024);
    }
  }

  const int64_t my_row = q0 + 32 * nbq + c;  // row whose epilogue this lane runs (with 3 other lanes)
  // The epilogue works in base 2: z2 = z log2(e), p = 2^(z2 - m2). Base-2
  // values go back to natural units of the logits with the inverse of the
  // factor that made them (inv_tau / c2 in fp64), so the fp32 rounding of
  // log2(e) in c2 does not shift the reference.
  const float c2 = inv_tau * kLog2e;
  const double to_nat = (double)inv_tau / (double)c2;
  float m2 = -INFINITY;
  double s_acc = 0.0, sz_acc = 0.0;  // this lane's share of sum p, sum p z2
  bool flag = false;
  float zmx = -INFINITY;             // the largest logit (base 2) this lane saw

  // Bias of tile rows kvq(kh, hh, 0..7), kept as packed bf16 (two groups of
  // four consecutive rows, one 8-byte load each when inside the vocabulary).
  const auto bias_r = frag_rsrc(bias, HAS_BIAS ? V * 2 : 0);
  auto load_bias = [&](int t, uint2 (&bv)[2]) {
    if constexpr (HAS_BIAS) {
      if ((t + 1) * BK <= V) {  // uniform: the whole tile lies inside the vocabulary
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int r0 = t * BK + 16 * kh + 8 * hf + 4 * hh;
          bv[hf] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(bias_r, r0 * 2, 0, 0));
        }
      } else {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int r0 = t * BK + 16 * kh + 8 * hf + 4 * hh;
          unsigned e[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) e[j] = __builtin_amdgcn_raw_buffer_load_b16(bias_r, min(r0 + j, V - 1) * 2, 0, 0);
          bv[hf] = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
        }
      }
    } else {
      bv[0] = bv[1] = make_uint2(0u, 0u);
    }
  };
  auto bias_at = [&](const uint2 (&bv)[2], int j) -> float {
    const uint2 u = bv[j >> 2];
    const unsigned wd = (j & 2) ? u.y : u.x;
    return __uint_as_float((j & 1) ? (wd & 0xffff0000u) : (wd << 16));
  };
  // S^T of the tile held in `a` (tile rows past V are zero in the
  // fragment-major copy and masked in the epilogue); each k-slice of `a`,
  // once its MFMAs are issued, is reloaded with the same slice of tile
  // `t_next`.
  auto s_step = [&](bf16x8 (&a)[KS], f32x16 (&acc)[2], int t_next) {
    const auto r = frag_rsrc(frag_ptr<KB>(Wf, t_next, w, 0, 0), KS * 1024);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[nb] = mfma32(a[ks], q[nb][ks], ks == 0 ? zero16() : acc[nb]);
      a[ks] = ld_buf(r, lane * 16, ks * 1024);
    }
  };
  // The partial S^T in four groups of four rows per row block; the wave
  // reducing quarter (nb, kh) reads groups 2kh and 2kh+1 of block nb.
  auto write_part = [&](const f32x16 (&acc)[2]) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig)
        s_part[w][nb][ig][lane] = f32x4{acc[nb][4 * ig], acc[nb][4 * ig + 1], acc[nb][4 * ig + 2], acc[nb][4 * ig + 3]};
  };
  auto reduce_part = [&](f32x4 (&sf)[2]) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
      sf[e] = (s_part[0][nbq][2 * kh + e][lane] + s_part[1][nbq][2 * kh + e][lane]) +
              (s_part[2][nbq][2 * kh + e][lane] + s_part[3][nbq][2 * kh + e][lane]);
  };
  // Logits (base 2) of the eight tile rows this lane holds; rows past the
  // vocabulary get -1e30 (2^(-1e30 - m2) = 0 and 0 * z = 0).
  auto logits = [&](int v0, const f32x4 (&sf)[2], const uint2 (&bv)[2], float (&z)[8]) {
    const int lim = V - v0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float sv_ = sf[j >> 2][j & 3];
      const float zz = HAS_BIAS ? (sv_ + bias_at(bv, j)) * c2 : sv_ * c2;
      z[j] = kvq(kh, hh, j) < lim ? zz : -1e30f;
    }
  };

  f32x16 acc[2];
  f32x4 sf[2];
  uint2 bv[2];
  if (any) {
    load_bias(t_begin, bv);
    s_step(a, acc, min(t_begin + 1, t_end - 1));
    write_part(acc);
  }
  __syncthreads();
  if (t_begin < t_end) {
    reduce_part(sf);
    // reference m2: the row's max over its first tile, from the four lanes
    // (two lane halves of two waves) that hold the row
    float z[8];
    logits(t_begin * BK, sf, bv, z);
    float mx = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
    mx = fmaxf(mx, other_half(mx, hh));
    if (hh == 0) s_x[w * 64 + c] = mx;
  }
  __syncthreads();
  if (t_begin < t_end) m2 = fmaxf(s_x[w * 64 + c], s_x[(w ^ 2) * 64 + c]);
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int v0 = t * BK;
    const int tn = min(t + 1, t_end - 1);
    const int tnn = min(t + 2, t_end - 1);
    uint2 bvn[2];
    load_bias(tn, bvn);
    // ---- epilogue of tile t (vector ALU; the scheduler interleaves it with
    //      the logit MFMAs of tile t+1 below) -------------------------------
    float z[8];
    logits(v0, sf, bv, z);
    float sp = 0.f, szp = 0.f;
    // the tile's largest logit in this lane: the flag test and the row max
    const float tm = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
    flag |= tm > m2 + kRefSlack2;
    zmx = fmaxf(zmx, tm);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float pj = __builtin_amdgcn_exp2f(fminf(z[j] - m2, kRefSlack2));
      sp += pj;
      szp = fmaf(pj, z[j], szp);
    }
    s_acc += (double)sp;
    sz_acc += (double)szp;
    // ---- logits of tile t+1 on the matrix cores, load t+2 ------------------
    s_step(a, acc, tnn);
    __builtin_amdgcn_sched_barrier(0);
    exec_barrier();
    write_part(acc);
    __syncthreads();
    // ---- reduce of tile t+1 ------------------------------------------------
    reduce_part(sf);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) bv[hf] = bvn[hf];
  }

  // ---- results: combine the four holders of each row ----------------------
  double sx = s_acc + (double)__shfl_xor(s_acc, 32, 64);
  double szx = sz_acc + (double)__shfl_xor(sz_acc, 32, 64);
  int fl = flag ? 1 : 0;
  fl |= __shfl_xor(fl, 32, 64);
  const float zm = fmaxf(zmx, other_half(zmx, hh));
  __syncthreads();
  if (hh == 0) {
    s_xd[(2 * w) * 64 + c] = sx;
    s_xd[(2 * w + 1) * 64 + c] = szx;
    s_x[w * 64 + c] = __int_as_float(fl);
    s_x[NW * 64 + w * 64 + c] = zm;
  }
  __syncthreads();
  if (kh == 0 && hh == 0 && my_row < N) {
    RowStats rs;
    rs.m = (double)m2 * to_nat;
    rs.zmax = (float)((double)fmaxf(zm, s_x[NW * 64 + (w ^ 2) * 64 + c]) * to_nat);
    rs.s = sx + s_xd[(2 * (w ^ 2)) * 64 + c];
    rs.sz = (szx + s_xd[(2 * (w ^ 2) + 1) * 64 + c]) * to_nat;
    rs.flag = (fl | __float_as_int(s_x[(w ^ 2) * 64 + c])) ? 1 : 0;
    stats[(int64_t)sv * N + my_row] = rs;
  }
}

// Forward sweep with the grad_h accumulator, as two roles on every SIMD
// (8 waves, two per SIMD, 256 registers each): waves 0-3 (S role) keep the
// resident rows of their H quarter, compute the logits of tile t+1 with its
// stage writes and loads, reduce the partials and run the epilogue; waves
// 4-7 (PV role) keep the accumulator of the same quarter and compute P KV of
// tile t, its two contraction steps split over the two phases between the
// barriers, so that one role's MFMAs fill the other's stalls:
//
//   prologue (S): logits of t0, reduce, reference m2, epilogue -> P(t0)
//   loop t:  barrier A
//            S: logits of t+1, stage t+1, loads of t+2, partials -> LDS
//            PV: P KV(t), first contraction step
//            barrier B
//            S: reduce of t+1, epilogue -> P(t+1)
//            PV: P KV(t), second contraction step
//
// P is double buffered (P(t+1) is written while P KV(t) still reads P(t)),
// and so are the staged tiles. The statistics are bit-identical to the
// statistics-only kernel's: every sum runs in the same order.
//
// With count_dev the rows are the first min(*count_dev, N) rows of a
// compacted list (rows row_idx[k] of h when row_idx is given), the splits
// forward_splits(that count, V, Sv) and the row stride of stats and O
// compact_stride(that count); the grid is sized for the largest count
// (forward_blocks_max) and workgroups with no block exit at once.
// With mref the exponent reference of row k is mref[k * mref_stride]
// (natural units) instead of the maximum of its first tile. clear_count, when
// given (never the count_dev of the same launch), is set to zero.
template <int KB, bool HAS_BIAS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_pp_kernel(const __bf16* __restrict__ h, const __bf16* __restrict__ Wf, const float* __restrict__ bias2,
                   int64_t N_, int V, float inv_tau, int Sv_, int tiles_per_split_, RowStats* __restrict__ stats,
                   float* __restrict__ O, const int* __restrict__ count_dev, const float* __restrict__ mref,
                   int mref_stride, const int* __restrict__ row_idx, int* __restrict__ clear_count) {
  constexpr int H = 128 * KB;
  if (clear_count && blockIdx.x == 0 && threadIdx.x == 0) *clear_count = 0;  // for the flag scan that follows
  int64_t N = N_, stride = N_;
  int Sv = Sv_, tiles_per_split = tiles_per_split_;
  if (count_dev) {
    N = min((int64_t)*count_dev, N_);
    if (N <= 0) return;  // uniform: an empty list (the usual second pass)
    Sv = forward_splits_wave(N, V, Sv_);
    tiles_per_split = ((V + BK - 1) / BK + Sv - 1) / Sv;
    stride = compact_stride(N);
  }
  int64_t rb;
  int sv;
  if (!forward_block((N + BQ - 1) / BQ, Sv, rb, sv)) return;  // uniform: no rows for this workgroup
  constexpr int DS = Stage<KB>::DS;
  constexpr int TS = Stage<KB>::TS;
  constexpr int KS = DS / 16;
  constexpr int DB = DS / 32;
  __shared__ f32x4 s_part[NW][2][4][64];
  __shared__ bf16x8 s_p[2][4][64];  // P of tiles t (even / odd)
  __shared__ unsigned short s_t[NW][2][BK * TS];
  float* s_x = reinterpret_cast<float*>(&s_p[0][0][0]);           // [NW][64]
  double* s_xd = reinterpret_cast<double*>(&s_part[0][0][0][0]);   // [NW][2][64]

  const int lane = threadIdx.x & 63;
  const int wall = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool srole = wall < 4;
  const int w = wall & 3;  // H quarter
  const int hh = lane >> 5, c = lane & 31;
  const int nbq = w & 1, kh = w >> 1;
  const int64_t q0 = rb * BQ;
  const int d0 = w * DS;
  const int n_tiles = (V + BK - 1) / BK;
  const int t_begin = sv * tiles_per_split;
  const int t_end = min(n_tiles, t_begin + tiles_per_split);
  const bool any = t_begin < t_end;
  const float c2 = inv_tau * kLog2e;
  const double to_nat = (double)inv_tau / (double)c2;  // base 2 back to natural units (see above)

  if (srole) {
    // ======================= S role =======================
    int sw_base[2];
    {
      const int x = hh ^ ((c >> 1) & 3);
      sw_base[0] = c * TS + 8 * x;
      sw_base[1] = c * TS + 8 * (x ^ 2) - 16;
    }
    bf16x8 q[2][KS];
    bf16x8 a[KS];
    {
      const int row0 = (int)min((int64_t)c, N - 1 - q0), row1 = (int)min((int64_t)(32 + c), N - 1 - q0);
      const auto ra = frag_rsrc(frag_ptr<KB>(Wf, any ? t_begin : 0, w, 0, 0), any ? KS * 1024 : 0);
      if (row_idx) {  // uniform: the resident rows are rows row_idx[q0 + r] of h
        const __bf16* p0 = h + (int64_t)row_idx[q0 + row0] * H + d0 + 8 * hh;
        const __bf16* p1 = h + (int64_t)row_idx[q0 + row1] * H + d0 + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          q[0][ks] = ld16(p0 + 16 * ks);
          q[1][ks] = ld16(p1 + 16 * ks);
          a[ks] = ld_buf(ra, lane * 16, ks * 1024);
        }
      } else {
        const auto rh = frag_rsrc(h + q0 * H, BQ * H * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          q[0][ks] = ld_buf(rh, (row0 * H + d0 + 8 * hh) * 2, 32 * ks);
          q[1][ks] = ld_buf(rh, (row1 * H + d0 + 8 * hh) * 2, 32 * ks);
          a[ks] = ld_buf(ra, lane * 16, ks * 1024);
        }
      }
    }
    const int64_t my_row = q0 + 32 * nbq + c;
    float m2 = -INFINITY;
    double s_acc = 0.0, sz_acc = 0.0;
    bool flag = false;
    float zmx = -INFINITY;  // the largest logit (base 2) this lane saw
    auto s_step = [&](f32x16 (&acc)[2], int buf, int t_next) {
      const auto r = frag_rsrc(frag_ptr<KB>(Wf, t_next, w, 0, 0), KS * 1024);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[nb] = mfma32(a[ks], q[nb][ks], ks == 0 ? zero16() : acc[nb]);
        *reinterpret_cast<bf16x8*>(&s_t[w][buf][sw_base[ks & 1] + 16 * ks]) = a[ks];
        a[ks] = ld_buf(r, lane * 16, ks * 1024);
      }
    };
    auto write_part = [&](const f32x16 (&acc)[2]) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig)
          s_part[w][nb][ig][lane] = f32x4{acc[nb][4 * ig], acc[nb][4 * ig + 1], acc[nb][4 * ig + 2], acc[nb][4 * ig + 3]};
    };
    auto reduce_part = [&](f32x4 (&sf)[2]) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
        sf[e] = (s_part[0][nbq][2 * kh + e][lane] + s_part[1][nbq][2 * kh + e][lane]) +
                (s_part[2][nbq][2 * kh + e][lane] + s_part[3][nbq][2 * kh + e][lane]);
    };
    // Bias of tile rows kvq(kh, hh, 0..7) from its fp32 copy (as above).
    const auto bias_r = f32_rsrc(bias2, HAS_BIAS ? ((V + 63) / 64) * 64 * 4 : 0);
    auto load_bias = [&](int t, f32x4 (&bv)[2]) {
      if constexpr (HAS_BIAS) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) bv[hf] = ld_f4(bias_r, (t * BK + 16 * kh + 8 * hf + 4 * hh) * 4);
      } else {
        bv[0] = bv[1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    };
    // Logits (base 2) of the eight tile rows this lane holds; rows past the
    // vocabulary get -1e30 (2^(-1e30 - m2) = 0 and 0 * z = 0).
    auto logits = [&](int v0, const f32x4 (&sf)[2], const f32x4 (&bv)[2], float (&z)[8]) {
      const int lim = V - v0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float sv_ = sf[j >> 2][j & 3];
        const float zz = HAS_BIAS ? (sv_ + bv[j >> 2][j & 3]) * c2 : sv_ * c2;
        z[j] = kvq(kh, hh, j) < lim ? zz : -1e30f;
      }
    };
    f32x4 bv[2];
    auto epilogue = [&](int t, const f32x4 (&sf)[2]) {
      float z[8];
      logits(t * BK, sf, bv, z);
      float sp = 0.f, szp = 0.f;
      bf16x8 pa;
      // the tile's largest logit in this lane: the flag test and the row max
      const float tm =
          fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
      flag |= tm > m2 + kRefSlack2;
      zmx = fmaxf(zmx, tm);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pj = __builtin_amdgcn_exp2f(fminf(z[j] - m2, kRefSlack2));
        sp += pj;
        szp = fmaf(pj, z[j], szp);
        pa[j] = (__bf16)pj;
      }
      s_acc += (double)sp;
      sz_acc += (double)szp;
      s_p[t & 1][w][lane] = pa;
    };

    f32x16 acc[2];
    f32x4 sf[2];
    if (any) {
      load_bias(t_begin, bv);
      s_step(acc, t_begin & 1, min(t_begin + 1, t_end - 1));
      write_part(acc);
    }
    __syncthreads();  // P0
    if (any) {
      reduce_part(sf);
      float z[8];
      logits(t_begin * BK, sf, bv, z);
      float mx = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
      mx = fmaxf(mx, other_half(mx, hh));
      if (hh == 0) s_x[w * 64 + c] = mx;
    }
    __syncthreads();  // P1
    if (any) {
      m2 = mref ? (float)((double)mref[min(my_row, N - 1) * mref_stride] / to_nat)
                : fmaxf(s_x[w * 64 + c], s_x[(w ^ 2) * 64 + c]);
    }
    __syncthreads();  // P2
    if (any) epilogue(t_begin, sf);
    for (int t = t_begin; t < t_end; ++t) {
      __syncthreads();  // A
      const bool more = t + 1 < t_end;
      if (more) {
        load_bias(t + 1, bv);
        s_step(acc, (t + 1) & 1, min(t + 2, t_end - 1));
        write_part(acc);
      }
      __syncthreads();  // B
      if (more) {
        reduce_part(sf);
        epilogue(t + 1, sf);
      }
    }
    // results
    double sx = s_acc + (double)__shfl_xor(s_acc, 32, 64);
    double szx = sz_acc + (double)__shfl_xor(sz_acc, 32, 64);
    int fl = flag ? 1 : 0;
    fl |= __shfl_xor(fl, 32, 64);
    const float zm = fmaxf(zmx, other_half(zmx, hh));
    __syncthreads();  // R0
    if (hh == 0) {
      s_xd[(2 * w) * 64 + c] = sx;
      s_xd[(2 * w + 1) * 64 + c] = szx;
      s_x[w * 64 + c] = __int_as_float(fl);
      s_x[NW * 64 + w * 64 + c] = zm;
    }
    __syncthreads();  // R1
    if (kh == 0 && hh == 0 && my_row < N) {
      RowStats rs;
      rs.m = (double)m2 * to_nat;
      rs.zmax = (float)((double)fmaxf(zm, s_x[NW * 64 + (w ^ 2) * 64 + c]) * to_nat);
      rs.s = sx + s_xd[(2 * (w ^ 2)) * 64 + c];
      rs.sz = (szx + s_xd[(2 * (w ^ 2) + 1) * 64 + c]) * to_nat;
      rs.flag = (fl | __float_as_int(s_x[(w ^ 2) * 64 + c])) ? 1 : 0;
      stats[(int64_t)sv * stride + my_row] = rs;
    }
  } else {
    // ======================= PV role =======================
    int tr_base[2];
    {
      const int p = lane & 15, G = lane >> 4;
      const int r = 4 * (G >> 1) + (p >> 2);
      const int b = 2 * (G & 1) + ((p >> 1) & 1);
      const int s = (r >> 1) & 3;
      tr_base[0] = r * TS + 8 * (b ^ s) + 4 * (p & 1);
      tr_base[1] = (r + 8) * TS + 8 * (b ^ s) + 4 * (p & 1);
    }
    f32x16 o[2][DB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int db = 0; db < DB; ++db) o[qb][db] = zero16();
    // P KV of tile t, contraction step ks (16 tile rows)
    auto pv = [&](int t, int ks) {
      const int buf = t & 1;
      const unsigned short* tb = &s_t[w][buf][0];
      {
        const bf16x8 p0 = s_p[buf][0 + 2 * ks][lane], p1 = s_p[buf][1 + 2 * ks][lane];
        auto frag = [&](int db) {
          return ld_tr(tb + tr_base[0] + 16 * ks * TS + 32 * db, tb + tr_base[1] + 16 * ks * TS + 32 * db);
        };
        bf16x8 b0 = frag(0);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 b1 = frag(db + 1 < DB ? db + 1 : DB - 1);
          o[0][db] = mfma32(p0, b0, o[0][db]);
          o[1][db] = mfma32(p1, b0, o[1][db]);
          b0 = b1;
        }
      }
    };
    __syncthreads();  // P0
    __syncthreads();  // P1
    __syncthreads();  // P2
    for (int t = t_begin; t < t_end; ++t) {
      __syncthreads();  // A
      pv(t, 0);
      __syncthreads();  // B
      pv(t, 1);
    }
    __syncthreads();  // R0
    __syncthreads();  // R1
    float* Ob = O + (int64_t)sv * stride * H;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t row = q0 + 32 * qb + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (row < N) {
          float* dst = Ob + row * H + d0 + c;
#pragma unroll
          for (int db = 0; db < DB; ++db) dst[32 * db] = o[qb][db][i];
        }
      }
  }
}

template <bool HAS_BIAS>
hipError_t fwd_pp_launch(const __bf16* h, const __bf16* Wf, const float* b, int64_t N, int H, int V, float inv_tau,
                         int Sv, RowStats* stats, float* O, const int* count_dev, const float* mref, int mref_stride,
                         const int* row_idx, int* clear_count, hipStream_t st) {
  if (clear_count && clear_count == count_dev) return hipErrorInvalidValue;
  const int n_tiles = (V + BK - 1) / BK;
  const int tps = (n_tiles + Sv - 1) / Sv;
  const int64_t nrb = (N + BQ - 1) / BQ;
  // with a device row count, enough workgroups for any count up to N
  int64_t blocks = count_dev ? forward_blocks_max(N, V, Sv) : nrb * Sv;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)((blocks + 7) / 8 * 8)), block(512);
  switch (H / 128) {
#define PLP_PP_CASE(K)                                                                                                \
  case K:                                                                                                             \
    hipLaunchKernelGGL((fwd_pp_kernel<K, HAS_BIAS>), grid, block, 0, st, h, Wf, b, N, V, inv_tau, Sv, tps, stats, O,  \
                       count_dev, mref, mref_stride, row_idx, clear_count);                                           \
    break;
    PLP_PP_CASE(1)
    PLP_PP_CASE(2)
    PLP_PP_CASE(3)
    PLP_PP_CASE(4)
    PLP_PP_CASE(5)
    PLP_PP_CASE(6)
    PLP_PP_CASE(7)
#undef PLP_PP_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool HAS_BIAS>
hipError_t fwd_stats_launch(const __bf16* h, const __bf16* Wf, const __bf16* b, int64_t N, int H, int V,
                            float inv_tau, int Sv, RowStats* stats, int* clear_count, hipStream_t st) {
  const int n_tiles = (V + BK - 1) / BK;
  const int tps = (n_tiles + Sv - 1) / Sv;
  const int64_t nrb = (N + BQ - 1) / BQ;
  const dim3 grid((unsigned)((nrb * Sv + 7) / 8 * 8)), block(256);
  switch (H / 128) {
#define PLP_FWD_CASE(K)                                                                                              \
  case K:                                                                                                            \
    hipLaunchKernelGGL((fwd_mfma_kernel<K, HAS_BIAS>), grid, block, 0, st, h, Wf, b, N, V, inv_tau, Sv, tps, stats,   \
                       clear_count);                                                                                 \
    break;
    PLP_FWD_CASE(1)
    PLP_FWD_CASE(2)
    PLP_FWD_CASE(3)
    PLP_FWD_CASE(4)
    PLP_FWD_CASE(5)
    PLP_FWD_CASE(6)
    PLP_FWD_CASE(7)
#undef PLP_FWD_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// The variants with the grad_h accumulator (two-role form), from
// lmhead_fwd_o.hip; b (the bias's fp32 copy, launch_bias_f32) may be NULL.
hipError_t launch_fwd_mfma_o(const __bf16* h, const __bf16* Wf, const float* b, int64_t N, int H, int V, float inv_tau,
                             int Sv, RowStats* stats, float* O, const int* count_dev, const float* mref,
                             int mref_stride, const int* row_idx, int* clear_count, hipStream_t st);

}  // namespace plp
