// Weight-gradient sweep of the LM head on the matrix cores (gfx950), its
// tail reduction, and the fragment-major copies both sweeps read; the tile
// machinery and the schedule are described in mfma_tile.h.
#include <atomic>

#include "mfma_tile.h"

namespace plp {

namespace {

// ---------------------------------------------------------------------------
// Fragment-major copy of 32-row tiles of X (rows X[idx[k]] when idx is given),
// rows at or past `rows` (= *count_dev when given) zero. Each thread copies
// the chunks of two consecutive k-steps of one row (two loads 32 bytes apart
// in flight); each wave's stores are two contiguous kilobytes and its loads
// touch 32 rows, every source line being used whole by neighbouring waves.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void frag_copy_kernel(const __bf16* __restrict__ X, const int* __restrict__ idx,
                                                        const int* __restrict__ count_dev, int64_t rows_host, int H,
                                                        int64_t tiles, __bf16* __restrict__ Xf) {
  const int64_t rows = count_dev ? (int64_t)(*count_dev) : rows_host;
  const int cpr = H / 8;
  // with a device row count, tiles past the last gathered row are never read
  const int64_t used = count_dev ? min(tiles, (rows + BK - 1) / BK) : tiles;
  const int ks_per_wave = H / 64;
  const int groups = ks_per_wave / 2;  // each thread copies the chunks of two consecutive k-steps
  const int64_t total = used * 4 * groups * 64;  // (tile, wave slice, k-step pair, lane)
  for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < total; o += (int64_t)gridDim.x * 256) {
    const int lane = (int)(o & 63);
    const int64_t rest = o >> 6;
    const int gq = (int)(rest % (4 * groups));
    const int64_t t = rest / (4 * groups);
    const int w = gq / groups, ks0 = 2 * (gq - w * groups);
    const int64_t r = t * BK + (lane & 31);
    uint4 v0 = make_uint4(0u, 0u, 0u, 0u), v1 = v0;
    if (r < rows) {
      const int64_t src = idx ? (int64_t)idx[r] : r;
      const __bf16* base = X + src * H + (w * (H / 32) + 2 * ks0 + (lane >> 5)) * 8;
      v0 = *reinterpret_cast<const uint4*>(base);
      v1 = *reinterpret_cast<const uint4*>(base + 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(Xf) + ((t * 4 + w) * ks_per_wave + ks0) * 64 + lane;
    dst[0] = v0;
    dst[64] = v1;
  }
}

// ---------------------------------------------------------------------------
// Weight-gradient sweep: per vocabulary row v, over compacted tokens t,
//   dz[t,v] = gs_t ([v = y_t] - exp(z[t,v] - lse_t)),  gs_t = g_t / tau
//   grad_W[v] += sum_t dz[t,v] h_t,   grad_b[v] += sum_t dz[t,v]
// acc_mode: 0 write the output dtype; 1 store fp32 accumulator; 2 add into it;
// 3 add the fp32 accumulator and write the output dtype.
// ---------------------------------------------------------------------------
// Weight-gradient sweep as two roles per SIMD (eight waves, two per SIMD,
// 256 registers each), like the forward sweep's accumulator passes: waves
// 0-3 (S role) keep the resident W rows of their H quarter, compute the
// logits of token tile t+1 with its stage writes and loads, reduce the
// partials and run the epilogue (dz, grad_b); waves 4-7 (PV role) keep the
// grad_W accumulator of the same quarter and compute dZ^T h of tile t, its
// two contraction steps split over the two phases between the barriers.
// P (dz) is double buffered; every sum runs in the same order as in a single
// role, so results are bit-identical.
template <int KB, bool HAS_BIAS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_pp_kernel(const __bf16* __restrict__ Wf, const __bf16* __restrict__ bias,
                   const __bf16* __restrict__ hcf, const TokData* __restrict__ tok,
                   const int* __restrict__ count_dev, int V, float inv_tau, int acc_mode,
                   float* __restrict__ gW_acc, float* __restrict__ gb_acc, __bf16* __restrict__ gW_out,
                   __bf16* __restrict__ gb_out, int whole, int parts, float* __restrict__ part_w,
                   float* __restrict__ part_b, int tok_begin, int tok_len) {
  constexpr int H = 128 * KB;
  constexpr int DS = Stage<KB>::DS;
  constexpr int TS = Stage<KB>::TS;
  constexpr int KS = DS / 16;
  constexpr int DB = DS / 32;
  __shared__ f32x4 s_part[NW][2][4][64];
  __shared__ bf16x8 s_p[2][4][64];
  __shared__ TokData s_tok[2][BK];
  __shared__ unsigned short s_t[NW][2][BK * TS];
  double* s_xd = reinterpret_cast<double*>(&s_part[0][0][0][0]);  // [NW][64], after the sweep

  const int lane = threadIdx.x & 63;
  const int wall = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool srole = wall < 4;
  const int w = wall & 3;  // H quarter
  const int hh = lane >> 5, c = lane & 31;
  const int nbq = w & 1, kh = w >> 1;
  // this launch's share of the compacted tokens: [tok_begin, tok_begin + tok_len)
  // of the *count_dev (tok and hcf already point at tok_begin)
  const int n_tok = max(0, min(*count_dev - tok_begin, tok_len));
  const int n_tiles = (n_tok + BK - 1) / BK;
  // Workgroups below `whole` take a vocabulary block and all token tiles.
  // The blocks of the last, partial round are shared by `parts` workgroups
  // each, which take contiguous thirds (or halves...) of the token tiles and
  // write fp32 partial sums for tail_reduce_kernel.
  int blk = blockIdx.x, t_lo = 0, t_hi = n_tiles, slot = -1;
  if ((int)blockIdx.x >= whole) {
    slot = (int)blockIdx.x - whole;
    blk = whole + slot / parts;
    const int part = slot - (slot / parts) * parts;
    t_lo = (int)((int64_t)n_tiles * part / parts);
    t_hi = (int)((int64_t)n_tiles * (part + 1) / parts);
  }
  const int q0 = blk * BQ;
  const int d0 = w * DS;
  const bool any = t_hi > t_lo;

  if (srole) {
    // ======================= S role =======================
    // Stage write offsets (element) of lane (hh, c) for even / odd k-step:
    // row c, chunk 2ks + hh at position (2ks + hh) ^ s(c), s(c) = (c >> 1) & 3.
    int sw_base[2];
    {
      const int x = hh ^ ((c >> 1) & 3);
      sw_base[0] = c * TS + 8 * x;
      sw_base[1] = c * TS + 8 * (x ^ 2) - 16;
    }
    // Per-token data of tile t, loaded into registers one phase before it
    // is written to LDS (wave 0, lanes < 32). Held as a plain vector: a
    // TokData variable was placed in LDS by the compiler, whose store right
    // after the load then waited for every outstanding load of the wave.
    static_assert(sizeof(TokData) == 16, "one 16-byte record per token");
    const auto tok_r = __builtin_amdgcn_make_buffer_rsrc(const_cast<TokData*>(tok), 0, 0x7ffffff0, 0x00020000);
    u32x4 tk = {0u, 0u, 0u, 0u};
    auto load_tok = [&](int t) {
      if (w == 0 && lane < BK) tk = __builtin_amdgcn_raw_buffer_load_b128(tok_r, (t * BK + lane) * 16, 0, 0);
    };
    // Tokens past the count get a neutral record (lse = +inf, gs = 0, y = -1)
    // whose dz is exactly +0 with no per-element test in the epilogue.
    auto stage_tok = [&](int t) {
      if (w == 0 && lane < BK) {
        const u32x4 pad = {0x7f800000u, 0u, 0xffffffffu, 0u};
        u32x4 rec = t * BK + lane < n_tok ? tk : pad;
        rec[0] = __float_as_uint(__uint_as_float(rec[0]) * kLog2e);  // lse in base 2 (+inf stays +inf)
        *reinterpret_cast<u32x4*>(&s_tok[t & 1][lane]) = rec;
      }
    };
    if (any) load_tok(t_lo);
    // Resident W fragments (B operand of S^T), rows q0 + 32nb + c, cols
    // d0 + 16ks + 8hh, from the fragment-major copy (rows past V are zero),
    // and the first token tile, in k-step order so that the first MFMAs
    // wait only for their own operands.
    bf16x8 q[2][KS];
    bf16x8 a[KS];
    {
      const auto rq0 = frag_rsrc(frag_ptr<KB>(Wf, q0 / BK, w, 0, 0), KS * 1024);
      const auto rq1 = frag_rsrc(frag_ptr<KB>(Wf, q0 / BK + 1, w, 0, 0), KS * 1024);
      // an empty token range loads nothing (zero range)
      const auto ra = frag_rsrc(frag_ptr<KB>(hcf, any ? t_lo : 0, w, 0, 0), any ? KS * 1024 : 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        q[0][ks] = ld_buf_nt(rq0, lane * 16, ks * 1024);
        q[1][ks] = ld_buf_nt(rq1, lane * 16, ks * 1024);
        a[ks] = ld_buf(ra, lane * 16, ks * 1024);
      }
    }
    const int my_v = q0 + 32 * nbq + c;
    const float bvl = HAS_BIAS ? (float)bias[min(my_v, V - 1)] : 0.f;
    const float c2 = inv_tau * kLog2e;
    double gb_run = 0.0;

    auto s_step = [&](f32x16 (&acc)[2], int buf, int t_next) {
      const auto r = frag_rsrc(frag_ptr<KB>(hcf, t_next, w, 0, 0), KS * 1024);
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
    // Epilogue of tile t: dz = g / tau ([v = y] - p) as bf16 P of this
    // wave's quarter, and this lane's share of grad_b; p = 2^(z2 - lse2) in
    // base 2 (the records' lse is scaled by log2 e once, when staged), and
    // dz = [v = y] gs - gs p as one fma. Every token record is
    // read (padding included), so the reads are not guarded by branches;
    // rows past V give values that only reach their own grad_W / grad_b
    // rows, which are never stored.
    // The eight records (lse, gs, y, pad) of the lane's tokens are read as
    // plain vectors before the partial-logit reduce, so that all sixteen LDS
    // reads of the phase are in flight together.
    auto load_recs = [&](int t, f32x4 (&rec)[8]) {
#pragma unroll
      for (int j = 0; j < 8; ++j) rec[j] = *reinterpret_cast<const f32x4*>(&s_tok[t & 1][kvq(kh, hh, j)]);
    };
    auto epilogue = [&](int t, const f32x4 (&sf)[2], const f32x4 (&rec)[8]) {
      bf16x8 pa;
      float gsum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float lse2 = rec[j][0], gs = rec[j][1];
        const int y = __float_as_int(rec[j][2]);
        const float pr = __builtin_amdgcn_exp2f((sf[j >> 2][j & 3] + bvl) * c2 - lse2);
        const float dz = __builtin_fmaf(-gs, pr, y == my_v ? gs : 0.f);
        gsum += dz;
        pa[j] = (__bf16)dz;
      }
      gb_run += (double)gsum;
      s_p[t & 1][w][lane] = pa;
    };

    f32x16 acc[2];
    f32x4 sf[2];
    if (any) {
      stage_tok(t_lo);
      load_tok(min(t_lo + 1, t_hi - 1));
      s_step(acc, t_lo & 1, min(t_lo + 1, t_hi - 1));
      write_part(acc);
    }
    __syncthreads();  // P0
    if (any) {
      f32x4 rec[8];
      load_recs(t_lo, rec);
      reduce_part(sf);
      epilogue(t_lo, sf, rec);
    }
    for (int t = t_lo; t < t_hi; ++t) {
      __syncthreads();  // A
      const bool more = t + 1 < t_hi;
      if (more) {
        stage_tok(t + 1);
        load_tok(min(t + 2, t_hi - 1));
        s_step(acc, (t + 1) & 1, min(t + 2, t_hi - 1));
        write_part(acc);
      }
      __syncthreads();  // B
      if (more) {
        f32x4 rec[8];
        load_recs(t + 1, rec);
        reduce_part(sf);
        epilogue(t + 1, sf, rec);
      }
    }

    // grad_b: the four holders of a vocabulary row (two lane halves of two
    // waves) hold disjoint token subsets
    const double gbv = gb_run + __shfl_xor(gb_run, 32, 64);
    __syncthreads();  // R0
    if (hh == 0) s_xd[w * 64 + c] = gbv;
    __syncthreads();  // R1
    if (slot >= 0) {  // a share of a tail block: fp32 partial sum, combined by tail_reduce_kernel
      if (kh == 0 && hh == 0) part_b[slot * BQ + 32 * nbq + c] = (float)(gbv + s_xd[(w ^ 2) * 64 + c]);
      return;
    }
    const bool from_acc = acc_mode == 2 || acc_mode == 3;
    const bool to_acc = acc_mode == 1 || acc_mode == 2;
    if (kh == 0 && hh == 0 && my_v < V && (to_acc ? gb_acc != nullptr : gb_out != nullptr)) {
      double val = gbv + s_xd[(w ^ 2) * 64 + c];
      if (from_acc) val += (double)gb_acc[my_v];
      if (to_acc) gb_acc[my_v] = (float)val;
      else gb_out[my_v] = (__bf16)(float)val;
    }
  } else {
    // ======================= PV role =======================
    // Transposing-load offsets: provider lane p of 16-lane group G reads row
    // 4(G/2) + p/4 (and 8 further down) of contraction step ks, chunk
    // 4db + 2(G%2) + (p%4)/2 of column block db, half p%2.
    int tr_base[2];
    {
      const int p = lane & 15, G = lane >> 4;
      const int r = 4 * (G >> 1) + (p >> 2);
      const int b = 2 * (G & 1) + ((p >> 1) & 1);
      const int s = (r >> 1) & 3;  // the same for rows r + 8 and r + 16
      tr_base[0] = r * TS + 8 * (b ^ s) + 4 * (p & 1);
      tr_base[1] = (r + 8) * TS + 8 * (b ^ s) + 4 * (p & 1);
    }
    f32x16 o[2][DB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int db = 0; db < DB; ++db) o[qb][db] = zero16();
    // dZ^T h of tile t, contraction step ks (16 token rows)
    auto pv = [&](int t, int ks) {
      const int buf = t & 1;
      const unsigned short* tb = &s_t[w][buf][0];
      const bf16x8 p0 = s_p[buf][0 + 2 * ks][lane], p1 = s_p[buf][1 + 2 * ks][lane];
      auto frag = [&](int db) {
        return ld_tr(tb + tr_base[0] + 16 * ks * TS + 32 * db, tb + tr_base[1] + 16 * ks * TS + 32 * db);
      };
      // B fragments two column blocks ahead (one ahead in the forward
      // sweep, where two cost 6 %: here they gain 2-3 %)
      bf16x8 b0 = frag(0), b1 = frag(1 < DB ? 1 : DB - 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 b2 = frag(db + 2 < DB ? db + 2 : DB - 1);
        o[0][db] = mfma32(p0, b0, o[0][db]);
        o[1][db] = mfma32(p1, b0, o[1][db]);
        b0 = b1;
        b1 = b2;
      }
    };
    __syncthreads();  // P0
    for (int t = t_lo; t < t_hi; ++t) {
      __syncthreads();  // A
      pv(t, 0);
      __syncthreads();  // B
      pv(t, 1);
    }
    __syncthreads();  // R0
    __syncthreads();  // R1
    // The accumulator leaves through this quarter's stage buffer (the S-role
    // wave of the quarter no longer uses it).
    float* sbuf = reinterpret_cast<float*>(&s_t[w][0][0]);
    if (slot >= 0) {
      float* pw = part_w + (int64_t)slot * BQ * H;
      store_acc<4, DS, DB>(o, sbuf, hh, c, lane, [&](int qb, int r, int col, const f32x4 (&v)[1]) {
        *reinterpret_cast<f32x4*>(pw + (int64_t)(32 * qb + r) * H + d0 + col) = v[0];
      });
      return;
    }
    const bool from_acc = acc_mode == 2 || acc_mode == 3;
    const bool to_acc = acc_mode == 1 || acc_mode == 2;
    if (to_acc ? gW_acc == nullptr : gW_out == nullptr) return;  // uniform
    if (to_acc) {  // fp32 accumulator rows, one f32x4 per lane
      store_acc<4, DS, DB>(o, sbuf, hh, c, lane, [&](int qb, int r, int col, const f32x4 (&v)[1]) {
        const int vr = q0 + 32 * qb + r;
        if (vr >= V) return;
        f32x4* dst = reinterpret_cast<f32x4*>(gW_acc + (int64_t)vr * H + d0 + col);
        *dst = from_acc ? *dst + v[0] : v[0];
      });
    } else {  // output dtype, eight bf16 (16 bytes) per lane
      store_acc<8, DS, DB>(o, sbuf, hh, c, lane, [&](int qb, int r, int col, const f32x4 (&v)[2]) {
        const int vr = q0 + 32 * qb + r;
        if (vr >= V) return;
        const int64_t k = (int64_t)vr * H + d0 + col;
        f32x4 lo = v[0], hi = v[1];
        if (from_acc) {
          lo += *reinterpret_cast<const f32x4*>(gW_acc + k);
          hi += *reinterpret_cast<const f32x4*>(gW_acc + k + 4);
        }
        bf16x8 u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u[j] = (__bf16)lo[j];
          u[4 + j] = (__bf16)hi[j];
        }
        // written once and read by nobody in this call: non-temporal, so
        // that the token tiles stay in L2
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, u), reinterpret_cast<u32x4*>(gW_out + k));
      });
    }
  }
}

constexpr int kTailParts = 4;     // workgroups sharing one tail block of the weight-gradient sweep
constexpr int kMaxTailWGs = 256;  // bound of the partial-sum scratch (workgroups)

// Workgroups of `threads` threads of `Kernel` the device holds at once
// (compute units x workgroups per unit), computed once per device and
// kernel: the cache is a static of this instantiation, one per kernel
// (callers on several threads may compute it concurrently; they store the
// same value).
template <auto Kernel>
hipError_t resident_workgroups(int threads, int* out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) {
      *out = v;
      return hipSuccess;
    }
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, Kernel, threads, 0);
  if (e != hipSuccess) return e;
  const int n = cus * (per_cu > 0 ? per_cu : 1);
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return hipSuccess;
}

// Sum of the partial results of the tail blocks (fixed order over the parts)
// and the same output step as the sweep's own: accumulate into / store the
// fp32 accumulators or store bf16 grad_W and grad_b. One workgroup per row.
__global__ __launch_bounds__(256) void tail_reduce_kernel(const float* __restrict__ part_w,
                                                          const float* __restrict__ part_b, int whole, int parts,
                                                          int H, int V, int acc_mode, float* __restrict__ gW_acc,
                                                          float* __restrict__ gb_acc, __bf16* __restrict__ gW_out,
                                                          __bf16* __restrict__ gb_out) {
  const int tb = blockIdx.x / BQ, r = blockIdx.x - tb * BQ;
  const int vr = (whole + tb) * BQ + r;
  if (vr >= V) return;  // uniform
  const bool from_acc = acc_mode == 2 || acc_mode == 3;
  const bool to_acc = acc_mode == 1 || acc_mode == 2;
  const int64_t stride = (int64_t)BQ * H;
  const float* src = part_w + ((int64_t)tb * parts * BQ + r) * H;
  for (int c4 = threadIdx.x; c4 < H / 4; c4 += 256) {
    f32x4 v = *reinterpret_cast<const f32x4*>(src + 4 * c4);
    for (int p = 1; p < parts; ++p) v += *reinterpret_cast<const f32x4*>(src + p * stride + 4 * c4);
    const int64_t k = (int64_t)vr * H + 4 * c4;
    if (to_acc ? gW_acc != nullptr : gW_out != nullptr) {
      if (from_acc) v += *reinterpret_cast<const f32x4*>(gW_acc + k);
      if (to_acc) {
        *reinterpret_cast<f32x4*>(gW_acc + k) = v;
      } else {
        bf16x4 u;
        u[0] = (__bf16)v[0];
        u[1] = (__bf16)v[1];
        u[2] = (__bf16)v[2];
        u[3] = (__bf16)v[3];
        *reinterpret_cast<bf16x4*>(gW_out + k) = u;
      }
    }
  }
  if (threadIdx.x == 0 && (to_acc ? gb_acc != nullptr : gb_out != nullptr)) {
    double val = 0.0;
    for (int p = 0; p < parts; ++p) val += (double)part_b[((int64_t)tb * parts + p) * BQ + r];
    if (from_acc) val += (double)gb_acc[vr];
    if (to_acc) gb_acc[vr] = (float)val;
    else gb_out[vr] = (__bf16)(float)val;
  }
}

template <int KB>
hipError_t bwd_dispatch(const __bf16* Wf, const __bf16* b, const __bf16* hcf, const TokData* tok, const int* count_dev,
                        int tok_begin, int tok_len, int V, float inv_tau, int acc_mode, float* gW_acc, float* gb_acc,
                        __bf16* gW_out, __bf16* gb_out, float* tail_scratch, hipStream_t st) {
  hcf += (size_t)tok_begin * (128 * KB);
  tok += tok_begin;
  // Blocks of the last, partial round of workgroups are split over the token
  // tiles so that round ends sooner: `parts` workgroups per block, as many as
  // fit the free slots (at most kTailParts, and kMaxTailWGs in all).
  const int nblk = (V + BQ - 1) / BQ;
  int resident = 0;
  hipError_t e = b ? resident_workgroups<bwd_pp_kernel<KB, true>>(512, &resident)
                   : resident_workgroups<bwd_pp_kernel<KB, false>>(512, &resident);
  if (e != hipSuccess) return e;
  const int rem = resident > 0 ? nblk % resident : 0;
  int parts = rem > 0 ? min(kTailParts, min(resident, kMaxTailWGs) / rem) : 1;
  if (tail_scratch == nullptr || parts < 2) parts = 1;
  const int whole = parts > 1 ? nblk - rem : nblk;
  const int tail_wgs = parts > 1 ? rem * parts : 0;
  float* part_w = tail_scratch;
  float* part_b = tail_scratch ? tail_scratch + (size_t)kMaxTailWGs * BQ * (128 * KB) : nullptr;
  dim3 grid((unsigned)(whole + tail_wgs)), block(512);
  if (b)
    hipLaunchKernelGGL((bwd_pp_kernel<KB, true>), grid, block, 0, st, Wf, b, hcf, tok, count_dev, V, inv_tau,
                       acc_mode, gW_acc, gb_acc, gW_out, gb_out, whole, parts, part_w, part_b, tok_begin, tok_len);
  else
    hipLaunchKernelGGL((bwd_pp_kernel<KB, false>), grid, block, 0, st, Wf, b, hcf, tok, count_dev, V, inv_tau,
                       acc_mode, gW_acc, gb_acc, gW_out, gb_out, whole, parts, part_w, part_b, tok_begin, tok_len);
  e = hipGetLastError();
  if (e != hipSuccess || tail_wgs == 0) return e;
  hipLaunchKernelGGL(tail_reduce_kernel, dim3((unsigned)(rem * BQ)), dim3(256), 0, st, part_w, part_b, whole, parts,
                     128 * KB, V, acc_mode, gW_acc, gb_acc, gW_out, gb_out);
  return hipGetLastError();
}

}  // namespace

namespace {
__global__ __launch_bounds__(256) void bias_f32_kernel(const __bf16* __restrict__ b, int V, int len,
                                                       float* __restrict__ out) {
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v < len) out[v] = v < V ? (float)b[v] : 0.f;
}
}  // namespace

hipError_t launch_bias_f32(const __bf16* b, int V, float* out, hipStream_t st) {
  const int len = (int)bias_f32_len(V);
  hipLaunchKernelGGL(bias_f32_kernel, dim3((unsigned)((len + 255) / 256)), dim3(256), 0, st, b, V, len, out);
  return hipGetLastError();
}

hipError_t launch_frag_copy(const __bf16* X, const int* idx, const int* count_dev, int64_t rows, int64_t tiles, int H,
                            __bf16* Xf, hipStream_t st) {
  if (tiles <= 0) return hipSuccess;
  const int64_t total = tiles * BK * (H / 8) / 2;
  const int64_t blocks = (total + 255) / 256;
  // one thread per pair of chunks (no grid-stride repeats at the sizes
  // here: more loads in flight, about 4 % faster for W at V=151936)
  hipLaunchKernelGGL(frag_copy_kernel, dim3((unsigned)(blocks < (1 << 20) ? blocks : (1 << 20))), dim3(256), 0, st,
                     X, idx, count_dev, rows, H, tiles, Xf);
  return hipGetLastError();
}

hipError_t launch_bwd_mfma(const __bf16* Wf, const __bf16* b, const __bf16* hcf, const TokData* tok,
                           const int* count_dev, int tok_begin, int tok_len, int H, int V, float inv_tau, int acc_mode,
                           float* gW_acc, float* gb_acc, __bf16* gW_out, __bf16* gb_out, float* tail_scratch,
                           hipStream_t st) {
  switch (H / 128) {
    case 1: return bwd_dispatch<1>(Wf, b, hcf, tok, count_dev, tok_begin, tok_len, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    case 2: return bwd_dispatch<2>(Wf, b, hcf, tok, count_dev, tok_begin, tok_len, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    case 3: return bwd_dispatch<3>(Wf, b, hcf, tok, count_dev, tok_begin, tok_len, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    case 4: return bwd_dispatch<4>(Wf, b, hcf, tok, count_dev, tok_begin, tok_len, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    case 5: return bwd_dispatch<5>(Wf, b, hcf, tok, count_dev, tok_begin, tok_len, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    case 6: return bwd_dispatch<6>(Wf, b, hcf, tok, count_dev, tok_begin, tok_len, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    case 7: return bwd_dispatch<7>(Wf, b, hcf, tok, count_dev, tok_begin, tok_len, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    default: return hipErrorInvalidValue;
  }
}

size_t bwd_tail_scratch_floats(int H) { return (size_t)kMaxTailWGs * BQ * H + (size_t)kMaxTailWGs * BQ; }

}  // namespace plp
