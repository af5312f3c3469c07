// MFMA (bf16, gfx950) sweeps of the LM head.
//
// Both the forward sweep and the weight-gradient sweep have the shape of an
// attention block with a very wide head (head dim = hidden size H):
//   resident rows  Q [64, H]        (forward: 64 token rows of h;
//                                     weight grad: 64 vocabulary rows of W)
//   streamed tiles KV[32, H]        (forward: 32 vocabulary rows of W;
//                                     weight grad: 32 compacted token rows of h)
//   S^T = KV Q^T                    logits of the tile, contraction over H
//   P   = epilogue(S)               forward: exp(z - m) with the row's reference m
//                                   weight grad: g (onehot - softmax) / tau
//   Acc += P KV                     forward: sum_v e^{z-m} W_v (for grad_h)
//                                   weight grad: sum_t dz h_t  (grad_W)
//
// H is split across the 4 waves of a workgroup: wave w owns columns
// [w*H/4, (w+1)*H/4) of Q, of every KV tile and of Acc. Its slice of Q stays
// in registers for the whole sweep and Acc in accumulation registers. The
// partial S^T of each wave (its slice of the contraction) is reduce-scattered
// through LDS: wave w ends up with the complete logits of resident-row block
// w, runs the epilogue on them, and the bf16 P fragments are all-gathered
// through LDS for the P KV product.
//
// Each KV tile is read from global memory once. The P KV product contracts
// over tile rows, so its KV operand needs the 8 tile rows of one column in a
// lane: after a wave has used its slice of the tile for S^T, it stores that
// slice row-major into a wave-private LDS buffer and reads it back with the
// gfx950 transposing load ds_read_b64_tr_b16, which, within each 16-lane
// group, hands lane l element l%4 of the 64-bit chunk that lane 4j + l/4
// addressed, for j = 0..3. Pointing lane p at row r0 + p/4, columns
// c0 + 4(p%4) .. +3 gives lane l the column c0 + l of rows r0 .. r0 + 3, the
// MFMA B-operand layout.
//
// MFMA: v_mfma_f32_16x16x32_bf16. Lane l holds A[l%16][8(l/16)+j],
// B[8(l/16)+j][l%16] (j = 0..7) and D[4(l/16)+i][l%16] (i = 0..3).
// The rows of a 32-row tile that lane-group g = l/16 holds after the S^T
// product are kv(g,j) = 4g+j (j<4) and 16+4g+(j-4) (j>=4); the same order is
// used as the contraction index of the P KV product, for both operands.
#include "common.h"

#include <math.h>

namespace plp {

namespace {

constexpr int BQ = 64;   // resident rows per workgroup
constexpr int BK = 32;   // streamed rows per tile
constexpr int NW = 4;    // waves per workgroup
// The forward sweep fixes each row's exponent reference m at the max of the
// row's first tile and never rescales the accumulator (a rescale of the
// register-resident accumulator does not fit the register file). A later
// logit above m + kRefSlack would make e^{z-m} exceed e^64; the row is then
// flagged and the merge kernel recomputes it exactly. e^64 ~ 6e27 keeps every
// running sum far inside fp32 and bf16 range.
constexpr float kRefSlack = 64.0f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int kv_of(int g, int j) { return j < 4 ? 4 * g + j : 12 + 4 * g + j; }

__device__ __forceinline__ bf16x8 ld16(const __bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// Two transposing LDS loads (rows r0..r0+3 and r0+16..r0+19 of a row-major
// bf16 tile, see the header) form one B-operand fragment.
__device__ __forceinline__ bf16x8 ld_tr(const unsigned short* p0, const unsigned short* p1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Reductions over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48) with the gfx950 lane swaps: permlane16_swap(x, x) hands every lane the
// values of rows {0,1} or {2,3} as (even row, odd row), permlane32_swap(y, y)
// the values of halves (low, high). Every lane combines the same operands in
// the same order, so all four lanes hold bitwise-identical results.
__device__ __forceinline__ float xg_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const unsigned v = __float_as_uint(y);
  const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

__device__ __forceinline__ float xg_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const unsigned v = __float_as_uint(y);
  const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Row stride (elements) of a wave's staged tile slice: the slice width plus
// 16 elements, so the rows a 16-lane group writes and the four rows each
// quarter of it reads in a transposing load start on different banks.
template <int KB>
struct Stage {
  static constexpr int DS = 32 * KB;
  static constexpr int TS = DS + 16;
};

// ---------------------------------------------------------------------------
// Row gather: Xc[k] = X[idx[k]] for k < count, zero rows up to the next
// multiple of 32 (16-byte vector copies).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather16_kernel(const __bf16* __restrict__ X, const int* __restrict__ idx,
                                                       const int* __restrict__ count_dev, int64_t cap, int H,
                                                       __bf16* __restrict__ Xc) {
  const int64_t n = *count_dev;
  const int64_t rows = min(cap, (n + BK - 1) / BK * BK);
  const int cpr = H / 8;
  const int64_t total = rows * cpr;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = e / cpr;
    const int c = (int)(e - k * cpr);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (k < n) v = *reinterpret_cast<const uint4*>(X + (int64_t)idx[k] * H + c * 8);
    *reinterpret_cast<uint4*>(Xc + k * H + c * 8) = v;
  }
}

// ---------------------------------------------------------------------------
// Schedule shared by both sweeps (per workgroup, per tile t of the sweep):
//
//   prologue: S^T(t0) -> LDS partials, barrier, reduce -> sf
//   loop t:   S^T(t+1) MFMAs          | interleaved with the epilogue of tile t
//             stage tile t+1 for the transposing load, loads for tile t+2
//             barrier
//             P(t) -> LDS, partials of t+1 -> LDS
//             barrier
//             P KV(t) MFMAs            | interleaved with the reduce of t+1
//
// so the matrix cores work while the vector unit runs the epilogue, and every
// load has a whole phase to arrive. Two barriers per tile; the partials and P
// buffers are reused every tile (each write follows a barrier that all reads
// of the previous contents precede). The staged tile slices are double
// buffered per wave: slice t+1 is written after the wave's last read of the
// buffer (P KV of tile t-1), and read in P KV(t+1).
// ---------------------------------------------------------------------------

// Forward sweep: per token row, running (sum e^{z-m}, sum e^{z-m} z) against
// the reference m, the target logit, and (WITH_O) the accumulator
// O = sum_v e^{z-m} W_v. Grid: (row blocks) x Sv vocabulary splits, block
// id = rb * Sv + split.
template <int KB, bool WITH_O, bool HAS_BIAS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_mfma_kernel(const __bf16* __restrict__ h, const __bf16* __restrict__ W,
                     const __bf16* __restrict__ bias, const int64_t* __restrict__ y, int64_t N, int V,
                     float inv_tau, int Sv, int tiles_per_split, RowStats* __restrict__ stats,
                     float* __restrict__ O) {
  constexpr int H = 128 * KB;
  constexpr int DS = Stage<KB>::DS;  // columns per wave
  constexpr int TS = Stage<KB>::TS;
  constexpr int DB = 2 * KB;         // 16-wide column blocks per wave
  __shared__ f32x4 s_part[NW][2][4][64];
  __shared__ bf16x8 s_p[4][64];
  __shared__ unsigned short s_t[WITH_O ? NW : 1][2][BK][WITH_O ? TS : 8];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int rb = blockIdx.x / Sv, sv = blockIdx.x - rb * Sv;
  const int64_t q0 = (int64_t)rb * BQ;
  const int d0 = w * DS;
  const int n_tiles = (V + BK - 1) / BK;
  const int t_begin = sv * tiles_per_split;
  const int t_end = min(n_tiles, t_begin + tiles_per_split);

  // Resident h fragments (B operand of S^T), rows q0+16nb+c16, cols d0+32kb+8g.
  bf16x8 q[4][KB];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int64_t row = min(q0 + 16 * nb + c16, N - 1);
    const __bf16* src = h + row * H + d0 + 8 * g;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) q[nb][kb] = ld16(src + 32 * kb);
  }

  f32x4 o[4][WITH_O ? DB : 1];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int db = 0; db < (WITH_O ? DB : 1); ++db) o[qb][db] = zero4();

  const int64_t my_row = q0 + 16 * w + c16;  // row whose epilogue this lane runs
  const int64_t yv = (y != nullptr && my_row < N) ? y[my_row] : -1;
  float m_ref = -INFINITY;
  double s_run = 0.0, sz_run = 0.0;
  float zy = 0.f;
  bool have_y = false, flag = false;

  auto load_a = [&](int t, bf16x8 (&a)[2][KB]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int v = min(t * BK + 16 * mb + c16, V - 1);  // rows past V are masked in the epilogue
      const __bf16* src = W + (int64_t)v * H + d0 + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) a[mb][kb] = ld16(src + 32 * kb);
    }
  };
  // Bias of tile rows kv(g, 0..7), kept as packed bf16 (two groups of four
  // consecutive rows, one 8-byte load each when inside the vocabulary).
  auto load_bias = [&](int t, uint2 (&bv)[2]) {
    if constexpr (HAS_BIAS) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int r0 = t * BK + 16 * hf + 4 * g;
        if (r0 + 3 < V) {
          bv[hf] = *reinterpret_cast<const uint2*>(bias + r0);
        } else {
          unsigned short e[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) e[j] = __builtin_bit_cast(unsigned short, bias[min(r0 + j, V - 1)]);
          bv[hf] = make_uint2(e[0] | ((unsigned)e[1] << 16), e[2] | ((unsigned)e[3] << 16));
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
  // S^T of the tile held in `a`; each k-slice of `a`, once its MFMAs are
  // issued, is staged for the transposing load (WITH_O) and reloaded with
  // the same slice of tile `t_next`.
  auto s_step = [&](bf16x8 (&a)[2][KB], f32x4 (&acc)[2][4], int buf, int t_next) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = zero4();
    const __bf16* src[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int v = min(t_next * BK + 16 * mb + c16, V - 1);
      src[mb] = W + (int64_t)v * H + d0 + 8 * g;
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma16(a[mb][kb], q[nb][kb], acc[mb][nb]);
      if constexpr (WITH_O) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          *reinterpret_cast<bf16x8*>(&s_t[w][buf][16 * mb + c16][32 * kb + 8 * g]) = a[mb][kb];
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) a[mb][kb] = ld16(src[mb] + 32 * kb);
    }
  };
  auto write_part = [&](const f32x4 (&acc)[2][4]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) s_part[w][mb][nb][lane] = acc[mb][nb];
  };
  auto reduce_part = [&](f32x4 (&sf)[2]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      sf[mb] = (s_part[0][mb][w][lane] + s_part[1][mb][w][lane]) + (s_part[2][mb][w][lane] + s_part[3][mb][w][lane]);
  };
  // P KV of the staged tile in `buf`, with the reduce of the next tile's
  // partials issued four column blocks before the end.
  auto pv_reduce = [&](int buf, f32x4 (&sf)[2]) {
    f32x4 r[NW];
    if constexpr (WITH_O) {
      bf16x8 pf[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) pf[qb] = s_p[qb][lane];
      const unsigned short* base = &s_t[w][buf][4 * g + (c16 >> 2)][4 * (c16 & 3)];
      // operand fragments two column blocks ahead of the MFMAs that use them
      bf16x8 b0 = ld_tr(base, base + 16 * TS);
      bf16x8 b1 = ld_tr(base + 16, base + 16 * TS + 16);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int dn = db + 2 < DB ? db + 2 : DB - 1;
        const bf16x8 b2 = ld_tr(base + 16 * dn, base + 16 * TS + 16 * dn);
        if (db == (DB > 4 ? DB - 4 : 0)) {
#pragma unroll
          for (int src = 0; src < NW; ++src) r[src] = s_part[src][0][w][lane];
        }
        if (db == (DB > 2 ? DB - 2 : 0)) {
          sf[0] = (r[0] + r[1]) + (r[2] + r[3]);
#pragma unroll
          for (int src = 0; src < NW; ++src) r[src] = s_part[src][1][w][lane];
        }
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) o[qb][db] = mfma16(pf[qb], b0, o[qb][db]);
        b0 = b1;
        b1 = b2;
      }
    } else {
#pragma unroll
      for (int src = 0; src < NW; ++src) r[src] = s_part[src][0][w][lane];
      sf[0] = (r[0] + r[1]) + (r[2] + r[3]);
#pragma unroll
      for (int src = 0; src < NW; ++src) r[src] = s_part[src][1][w][lane];
    }
    sf[1] = (r[0] + r[1]) + (r[2] + r[3]);
  };

  bf16x8 a[2][KB];
  f32x4 acc[2][4], sf[2];
  uint2 bv[2];
  if (t_begin < t_end) {
    load_a(t_begin, a);
    load_bias(t_begin, bv);
    s_step(a, acc, t_begin & 1, min(t_begin + 1, t_end - 1));
    write_part(acc);
  }
  __syncthreads();
  if (t_begin < t_end) reduce_part(sf);

  for (int t = t_begin; t < t_end; ++t) {
    const int v0 = t * BK;
    const int tn = min(t + 1, t_end - 1);
    const int tnn = min(t + 2, t_end - 1);
    // ---- logits of tile t+1 on the matrix cores, stage t+1, load t+2 -------
    s_step(a, acc, (t + 1) & 1, tnn);
    uint2 bvn[2];
    load_bias(tn, bvn);
    // ---- epilogue of tile t on row my_row, tile rows kv(g, j) -------------
    float z[8];
    bool ok[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int v = v0 + kv_of(g, j);
      ok[j] = v < V;
      const float sv_ = j < 4 ? sf[0][j] : sf[1][j - 4];
      z[j] = ok[j] ? (sv_ + bias_at(bv, j)) * inv_tau : -INFINITY;
    }
    float mx = z[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, z[j]);
    mx = xg_max(mx);
    m_ref = t == t_begin ? mx : m_ref;
    flag |= mx > m_ref + kRefSlack;
    float p[8], sp = 0.f, szp = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = ok[j] ? __expf(fminf(z[j] - m_ref, kRefSlack)) : 0.f;
      sp += p[j];
      szp += ok[j] ? p[j] * z[j] : 0.f;
    }
    s_run += (double)xg_sum(sp);
    sz_run += (double)xg_sum(szp);
    {
      const int64_t rel = yv - v0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool hit = (int64_t)kv_of(g, j) == rel;
        zy = hit ? z[j] : zy;
        have_y |= hit;
      }
    }
    bf16x8 pa;
#pragma unroll
    for (int j = 0; j < 8; ++j) pa[j] = (__bf16)p[j];
    __syncthreads();
    if constexpr (WITH_O) s_p[w][lane] = pa;
    write_part(acc);
    __syncthreads();
    // ---- accumulator product of tile t, reduce of tile t+1 -----------------
    pv_reduce(t & 1, sf);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) bv[hf] = bvn[hf];
  }

  // ---- results ---------------------------------------------------------------
  const float zyv = xg_sum(have_y ? zy : 0.f);
  if (g == 0 && my_row < N) {
    RowStats rs;
    rs.m = m_ref;
    rs.zy = zyv;
    rs.s = s_run;
    rs.sz = sz_run;
    rs.flag = flag ? 1 : 0;
    rs.pad = 0;
    stats[(int64_t)sv * N + my_row] = rs;
  }
  if constexpr (WITH_O) {
    float* Ob = O + (int64_t)sv * N * H;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = q0 + 16 * qb + 4 * g + i;
        if (row < N) {
          float* dst = Ob + row * H + d0 + c16;
#pragma unroll
          for (int db = 0; db < DB; ++db) dst[16 * db] = o[qb][db][i];
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Weight-gradient sweep: per vocabulary row v, over compacted tokens t,
//   dz[t,v] = gs_t ([v = y_t] - exp(z[t,v] - lse_t)),  gs_t = g_t / tau
//   grad_W[v] += sum_t dz[t,v] h_t,   grad_b[v] += sum_t dz[t,v]
// acc_mode: 0 write the output dtype; 1 store fp32 accumulator; 2 add into it;
// 3 add the fp32 accumulator and write the output dtype.
// ---------------------------------------------------------------------------
template <int KB, bool HAS_BIAS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_mfma_kernel(const __bf16* __restrict__ W, const __bf16* __restrict__ bias,
                     const __bf16* __restrict__ hc, const TokData* __restrict__ tok,
                     const int* __restrict__ count_dev, int V, float inv_tau, int acc_mode,
                     float* __restrict__ gW_acc, float* __restrict__ gb_acc, __bf16* __restrict__ gW_out,
                     __bf16* __restrict__ gb_out) {
  constexpr int H = 128 * KB;
  constexpr int DS = Stage<KB>::DS;
  constexpr int TS = Stage<KB>::TS;
  constexpr int DB = 2 * KB;
  __shared__ f32x4 s_part[NW][2][4][64];
  __shared__ bf16x8 s_p[4][64];
  __shared__ TokData s_tok[2][BK];
  __shared__ unsigned short s_t[NW][2][BK][TS];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int q0 = blockIdx.x * BQ;
  const int d0 = w * DS;
  const int n_tok = *count_dev;
  const int n_tiles = (n_tok + BK - 1) / BK;

  // Resident W fragments (B operand of S^T), rows q0+16nb+c16, cols d0+32kb+8g.
  bf16x8 q[4][KB];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int v = min(q0 + 16 * nb + c16, V - 1);
    const __bf16* src = W + (int64_t)v * H + d0 + 8 * g;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) q[nb][kb] = ld16(src + 32 * kb);
  }
  f32x4 o[4][DB];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = zero4();

  const int my_v = q0 + 16 * w + c16;
  const float bvl = HAS_BIAS ? (float)bias[min(my_v, V - 1)] : 0.f;
  double gb_run = 0.0;

  auto load_a = [&](int t, bf16x8 (&a)[2][KB]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const __bf16* src = hc + (int64_t)(t * BK + 16 * mb + c16) * H + d0 + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) a[mb][kb] = ld16(src + 32 * kb);
    }
  };
  auto stage_tok = [&](int t) {
    if (w == 0 && lane < BK) s_tok[t & 1][lane] = tok[t * BK + lane];
  };
  auto s_step = [&](bf16x8 (&a)[2][KB], f32x4 (&acc)[2][4], int buf, int t_next) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = zero4();
    const __bf16* src[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) src[mb] = hc + (int64_t)(t_next * BK + 16 * mb + c16) * H + d0 + 8 * g;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma16(a[mb][kb], q[nb][kb], acc[mb][nb]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        *reinterpret_cast<bf16x8*>(&s_t[w][buf][16 * mb + c16][32 * kb + 8 * g]) = a[mb][kb];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) a[mb][kb] = ld16(src[mb] + 32 * kb);
    }
  };
  auto write_part = [&](const f32x4 (&acc)[2][4]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) s_part[w][mb][nb][lane] = acc[mb][nb];
  };
  auto reduce_part = [&](f32x4 (&sf)[2]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      sf[mb] = (s_part[0][mb][w][lane] + s_part[1][mb][w][lane]) + (s_part[2][mb][w][lane] + s_part[3][mb][w][lane]);
  };
  auto pv_reduce = [&](int buf, f32x4 (&sf)[2]) {
    f32x4 r[NW];
    bf16x8 pf[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) pf[qb] = s_p[qb][lane];
    const unsigned short* base = &s_t[w][buf][4 * g + (c16 >> 2)][4 * (c16 & 3)];
    bf16x8 b0 = ld_tr(base, base + 16 * TS);
    bf16x8 b1 = ld_tr(base + 16, base + 16 * TS + 16);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int dn = db + 2 < DB ? db + 2 : DB - 1;
      const bf16x8 b2 = ld_tr(base + 16 * dn, base + 16 * TS + 16 * dn);
      if (db == (DB > 4 ? DB - 4 : 0)) {
#pragma unroll
        for (int src = 0; src < NW; ++src) r[src] = s_part[src][0][w][lane];
      }
      if (db == (DB > 2 ? DB - 2 : 0)) {
        sf[0] = (r[0] + r[1]) + (r[2] + r[3]);
#pragma unroll
        for (int src = 0; src < NW; ++src) r[src] = s_part[src][1][w][lane];
      }
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) o[qb][db] = mfma16(pf[qb], b0, o[qb][db]);
      b0 = b1;
      b1 = b2;
    }
    sf[1] = (r[0] + r[1]) + (r[2] + r[3]);
  };

  bf16x8 a[2][KB];
  f32x4 acc[2][4], sf[2];
  if (n_tiles > 0) {
    stage_tok(0);
    load_a(0, a);
    s_step(a, acc, 0, min(1, n_tiles - 1));
    write_part(acc);
  }
  __syncthreads();
  if (n_tiles > 0) reduce_part(sf);

  for (int t = 0; t < n_tiles; ++t) {
    const int t0 = t * BK;
    const int tn = min(t + 1, n_tiles - 1);
    const int tnn = min(t + 2, n_tiles - 1);
    s_step(a, acc, (t + 1) & 1, tnn);
    bf16x8 pa;
    float gsum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kv = kv_of(g, j);
      const TokData td = s_tok[t & 1][kv];
      const float sv_ = j < 4 ? sf[0][j] : sf[1][j - 4];
      const float z = (sv_ + bvl) * inv_tau;
      const float pr = __expf(z - td.lse);
      float dz = td.gs * ((td.y == my_v ? 1.f : 0.f) - pr);
      dz = (t0 + kv < n_tok && my_v < V) ? dz : 0.f;
      gsum += dz;
      pa[j] = (__bf16)dz;
    }
    gb_run += (double)gsum;
    __syncthreads();
    s_p[w][lane] = pa;
    write_part(acc);
    stage_tok(tn);
    __syncthreads();
    pv_reduce(t & 1, sf);
  }

  // grad_b: the four lane groups of a row hold disjoint token subsets
  double gbv = gb_run;
  gbv += __shfl_xor(gbv, 16, 64);
  gbv += __shfl_xor(gbv, 32, 64);
  const bool from_acc = acc_mode == 2 || acc_mode == 3;
  const bool to_acc = acc_mode == 1 || acc_mode == 2;
  if (g == 0 && my_v < V && (to_acc ? gb_acc != nullptr : gb_out != nullptr)) {
    double val = gbv;
    if (from_acc) val += (double)gb_acc[my_v];
    if (to_acc) gb_acc[my_v] = (float)val;
    else gb_out[my_v] = (__bf16)(float)val;
  }
  if (to_acc ? gW_acc == nullptr : gW_out == nullptr) return;
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = q0 + 16 * qb + 4 * g + i;
      if (v < V) {
        const int64_t base = (int64_t)v * H + d0 + c16;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          float val = o[qb][db][i];
          const int64_t k = base + 16 * db;
          if (from_acc) val += gW_acc[k];
          if (to_acc) gW_acc[k] = val;
          else gW_out[k] = (__bf16)val;
        }
      }
    }
}

template <int KB>
hipError_t fwd_dispatch(const __bf16* h, const __bf16* W, const __bf16* b, const int64_t* y, int64_t N, int V,
                        float inv_tau, int Sv, int tps, bool with_o, RowStats* stats, float* O, hipStream_t st) {
  const int64_t nrb = (N + BQ - 1) / BQ;
  dim3 grid((unsigned)(nrb * Sv)), block(256);
  if (with_o && b)
    hipLaunchKernelGGL((fwd_mfma_kernel<KB, true, true>), grid, block, 0, st, h, W, b, y, N, V, inv_tau, Sv, tps,
                       stats, O);
  else if (with_o)
    hipLaunchKernelGGL((fwd_mfma_kernel<KB, true, false>), grid, block, 0, st, h, W, b, y, N, V, inv_tau, Sv, tps,
                       stats, O);
  else if (b)
    hipLaunchKernelGGL((fwd_mfma_kernel<KB, false, true>), grid, block, 0, st, h, W, b, y, N, V, inv_tau, Sv, tps,
                       stats, O);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<KB, false, false>), grid, block, 0, st, h, W, b, y, N, V, inv_tau, Sv, tps,
                       stats, O);
  return hipGetLastError();
}

template <int KB>
hipError_t bwd_dispatch(const __bf16* W, const __bf16* b, const __bf16* hc, const TokData* tok, const int* count_dev,
                        int V, float inv_tau, int acc_mode, float* gW_acc, float* gb_acc, __bf16* gW_out,
                        __bf16* gb_out, hipStream_t st) {
  dim3 grid((unsigned)((V + BQ - 1) / BQ)), block(256);
  if (b)
    hipLaunchKernelGGL((bwd_mfma_kernel<KB, true>), grid, block, 0, st, W, b, hc, tok, count_dev, V, inv_tau,
                       acc_mode, gW_acc, gb_acc, gW_out, gb_out);
  else
    hipLaunchKernelGGL((bwd_mfma_kernel<KB, false>), grid, block, 0, st, W, b, hc, tok, count_dev, V, inv_tau,
                       acc_mode, gW_acc, gb_acc, gW_out, gb_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_bf16(const __bf16* X, const int* idx, const int* count_dev, int64_t cap, int H, __bf16* Xc,
                              hipStream_t st) {
  if (cap <= 0) return hipSuccess;
  const int64_t chunks = cap * (H / 8);
  const int64_t blocks = (chunks + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL(gather16_kernel, dim3(grid), dim3(256), 0, st, X, idx, count_dev, cap, H, Xc);
  return hipGetLastError();
}

hipError_t launch_fwd_mfma(const __bf16* h, const __bf16* W, const __bf16* b, const int64_t* y, int64_t N, int H,
                           int V, float inv_tau, int Sv, bool with_o, RowStats* stats, float* O, hipStream_t st) {
  const int n_tiles = (V + BK - 1) / BK;
  const int tps = (n_tiles + Sv - 1) / Sv;
  switch (H / 128) {
    case 1: return fwd_dispatch<1>(h, W, b, y, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    case 2: return fwd_dispatch<2>(h, W, b, y, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    case 3: return fwd_dispatch<3>(h, W, b, y, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    case 4: return fwd_dispatch<4>(h, W, b, y, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    case 5: return fwd_dispatch<5>(h, W, b, y, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    case 6: return fwd_dispatch<6>(h, W, b, y, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    case 7: return fwd_dispatch<7>(h, W, b, y, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_mfma(const __bf16* W, const __bf16* b, const __bf16* hc, const TokData* tok,
                           const int* count_dev, int H, int V, float inv_tau, int acc_mode, float* gW_acc,
                           float* gb_acc, __bf16* gW_out, __bf16* gb_out, hipStream_t st) {
  switch (H / 128) {
    case 1: return bwd_dispatch<1>(W, b, hc, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out, st);
    case 2: return bwd_dispatch<2>(W, b, hc, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out, st);
    case 3: return bwd_dispatch<3>(W, b, hc, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out, st);
    case 4: return bwd_dispatch<4>(W, b, hc, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out, st);
    case 5: return bwd_dispatch<5>(W, b, hc, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out, st);
    case 6: return bwd_dispatch<6>(W, b, hc, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out, st);
    case 7: return bwd_dispatch<7>(W, b, hc, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace plp
