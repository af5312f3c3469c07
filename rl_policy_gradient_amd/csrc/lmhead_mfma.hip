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
// MFMA: v_mfma_f32_32x32x16_bf16, the bf16 shape that runs at the full dense
// rate on gfx950 (the 16x16x32 shape issues at half of it). Lane l, with
// h = l/32 and c = l%32, holds A[c][8h+j], B[8h+j][c] (j = 0..7) and
// D[8(i/4)+4h+i%4][c] (i = 0..15).
//
// H is split across the 4 waves of a workgroup: wave w owns columns
// [w*H/4, (w+1)*H/4) of Q, of every KV tile and of Acc. Its slice of Q stays
// in registers for the whole sweep and Acc in accumulation registers. The
// partial S^T of each wave (its slice of the contraction) is reduce-scattered
// through LDS: wave w = nb + 2kh ends up with the complete logits of one
// quarter of the tile, resident-row block nb (32 rows) and tile-row half kh
// (16 rows); lane (h, c) holds resident row 32nb + c and the eight tile rows
// kvq(kh, h, e) = 16kh + 8(e/4) + 4h + e%4. Those eight values are exactly
// lane (h, c)'s A operand of the P KV product for row block nb and
// contraction step kh, so the bf16 P fragments are all-gathered through LDS
// unchanged, and the same tile-row order is the contraction index of the KV
// operand. A resident row's values are spread over four lanes (two lane
// halves of two waves); its running sums are kept per lane against a
// reference fixed before the sweep and combined once at the end.
//
// Each KV tile is read from global memory once. The P KV product contracts
// over tile rows, so its KV operand needs tile rows of one column in a lane:
// after a wave has used its slice of the tile for S^T, it stores that slice
// row-major into a wave-private LDS buffer and reads it back with the gfx950
// transposing load ds_read_b64_tr_b16, which, within each 16-lane group,
// hands lane l element l%4 of the 64-bit chunk that lane 4j + l/4 addressed,
// for j = 0..3. Pointing lane p at row r0 + p/4, columns c0 + 4(p%4) .. +3
// gives lane l the column c0 + l of rows r0 .. r0 + 3, the B-operand layout.
#include "common.h"

#include <math.h>

namespace plp {

namespace {

constexpr int BQ = 64;   // resident rows per workgroup (two 32-row blocks)
constexpr int BK = 32;   // streamed rows per tile
constexpr int NW = 4;    // waves per workgroup
// The forward sweep fixes each row's exponent reference m at the max of the
// row's first tile and never rescales the accumulator (a rescale of the
// register-resident accumulator does not fit the register file). A later
// logit above m + kRefSlack would make e^{z-m} exceed e^64; the row is then
// flagged and the merge kernel recomputes it exactly. e^64 ~ 6e27 keeps every
// running sum far inside fp32 and bf16 range.
constexpr float kRefSlack = 64.0f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr double kLn2 = 0.693147180559945309417;
constexpr float kRefSlack2 = kRefSlack * kLog2e;  // the slack in base-2 units

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Workgroup execution barrier without a memory fence. It orders the
// exchange writes after the previous tile's exchange reads: every wave has
// already consumed the values it read (they fed its MFMAs and epilogue), so
// no LDS access of another wave is outstanding on those buffers, and the
// wave's own stage writes, which only it reads back, need not drain first.
__device__ __forceinline__ void exec_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Tile row held in element e (0..7) by lane half h of the wave that owns
// tile-row half kh after the reduce (see the header comment).
__device__ __forceinline__ int kvq(int kh, int h, int e) { return 16 * kh + 8 * (e >> 2) + 4 * h + (e & 3); }

__device__ __forceinline__ bf16x8 ld16(const __bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// Two transposing LDS loads (rows r0..r0+3 and r0+8..r0+11 of a row-major
// bf16 tile, see the header) form one B-operand fragment.
__device__ __forceinline__ bf16x8 ld_tr(const unsigned short* p0, const unsigned short* p1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Values of the other lane half (l ^ 32) with the gfx950 lane swap:
// permlane32_swap(x, x) returns (low-half value, high-half value) in every lane.
__device__ __forceinline__ float other_half(float x, int h) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(h ? r[0] : r[1]);
}

// Layout of a wave's staged tile slice: 32 rows of TS elements; the 16-byte
// chunk k of row r sits at chunk position k ^ s(r), s(r) = (r >> 1) & 3. The
// LDS serves 128 bytes (32 banks of 4 bytes) per pass, and a 16-byte store or
// an 8-byte transposing load is served eight lanes at a time: the eight stage
// writes of a pass (rows 8m .. 8m+7, one chunk each) and the eight loads of a
// pass (two rows, two chunks, two halves) then touch 32 distinct banks. A row
// spans 4 (mod 8) chunks, so rows of opposite parity start 64 bytes apart;
// rows are padded by 32 elements for even KB to keep that.
template <int KB>
struct Stage {
  static constexpr int DS = 32 * KB;
  static constexpr int TS = DS + ((KB & 1) ? 0 : 32);
};

// Fragment-major copies: the operand a wave loads for one 16-wide contraction
// step of a 32-row tile is one contiguous kilobyte, lane-ordered:
//   Xf[((tile * 4 + w) * KS + ks) * 64 + lane][0..7]
//     = X[32 tile + lane % 32][w * DS + 16 ks + 8 (lane / 32) + 0..7].
template <int KB>
__device__ __forceinline__ const __bf16* frag_ptr(const __bf16* Xf, int64_t tile, int w, int ks, int lane) {
  constexpr int KS = 2 * KB;
  return Xf + ((((tile * 4 + w) * KS) + ks) * 64 + lane) * 8;
}

// Loads of fragment-major data through a buffer resource: the workgroup-
// uniform base (and a byte range that bounds the access) in scalar registers,
// the lane's byte offset in one vector register, a constant byte offset in a
// scalar register, so no 64-bit vector address per load is kept live.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t frag_rsrc(const __bf16* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ bf16x8 ld_buf(__amdgpu_buffer_rsrc_t r, int lane_bytes, int const_bytes) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, lane_bytes, const_bytes, 0));
}
// The same with the non-temporal hint: for data read once (the resident
// rows of the weight-gradient sweep), so that it does not push the token
// tiles every workgroup re-reads out of L2.
__device__ __forceinline__ bf16x8 ld_buf_nt(__amdgpu_buffer_rsrc_t r, int lane_bytes, int const_bytes) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, lane_bytes, const_bytes, 2));
}

// Ordering of one wave's own LDS accesses across its lanes. A wave's LDS
// instructions execute in issue order, so a read that follows a write of
// another lane of the same wave sees it; the fences keep the compiler from
// moving the accesses across this point. No workgroup barrier: it would also
// wait for the wave's outstanding global stores.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Store of a wave's accumulator (rows 32qb + 8(i/4) + 4h + i%4 of the
// resident block, columns 32db + c of the wave's slice) through a wave-private
// LDS buffer of 32 x DS floats, one 32-row half at a time, so that the global
// accesses run along rows: emit(qb, row, col, v) is called once per CH
// consecutive columns (CH = 4: v is one f32x4; CH = 8: v[0], v[1] hold
// columns col .. col+3, col+4 .. col+7). The buffer must be one no other wave
// touches from here on; the first half's global stores are still in flight
// while the second half goes through the buffer.
template <int CH, int DS, int DB, typename Emit>
__device__ __forceinline__ void store_acc(const f32x16 (&o)[2][DB], float* buf, int hh, int c, int lane, Emit&& emit) {
  static_assert(CH == 4 || CH == 8, "four or eight columns per call");
  static_assert(DS % CH == 0 && (DS & 1) == 0, "rows split into whole chunks");
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float* row = buf + (8 * (i >> 2) + 4 * hh + (i & 3)) * DS + c;
#pragma unroll
      for (int db = 0; db < DB; ++db) row[32 * db] = o[qb][db][i];
    }
    wave_lds_sync();
    const f32x4* b4 = reinterpret_cast<const f32x4*>(buf);
    for (int q = lane; q < 32 * DS / CH; q += 64) {
      const int r = q / (DS / CH), cc = q - r * (DS / CH);
      const f32x4* src = b4 + r * (DS / 4) + cc * (CH / 4);
      f32x4 v[CH / 4];
#pragma unroll
      for (int k = 0; k < CH / 4; ++k) v[k] = src[k];
      emit(qb, r, CH * cc, v);
    }
  }
}

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
// Schedule shared by both sweeps (per workgroup, per tile t of the sweep):
//
//   prologue: S^T(t0) -> LDS partials, barrier, reduce -> sf
//   loop t:   epilogue of tile t (vector ALU)   | interleaved with
//             S^T(t+1) MFMAs, staging of tile t+1 for the transposing load
//             and the loads of tile t+2
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

// Forward sweep: per token row, running (sum 2^{z2-m2}, sum 2^{z2-m2} z2)
// against the reference m2 (z2 = z log2 e), and (WITH_O) the accumulator
// O = sum_v e^{z-m} W_v. Grid: (row blocks) x Sv vocabulary splits, block
// id = rb * Sv + split.
template <int KB, bool WITH_O, bool HAS_BIAS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_mfma_kernel(const __bf16* __restrict__ h, const __bf16* __restrict__ Wf,
                     const __bf16* __restrict__ bias, int64_t N, int V, float inv_tau, int Sv,
                     int tiles_per_split, RowStats* __restrict__ stats, float* __restrict__ O) {
  constexpr int H = 128 * KB;
  constexpr int DS = Stage<KB>::DS;  // columns per wave
  constexpr int TS = Stage<KB>::TS;
  constexpr int KS = DS / 16;        // 16-wide contraction steps per wave
  constexpr int DB = DS / 32;        // 32-wide column blocks per wave
  __shared__ f32x4 s_part[NW][2][4][64];
  __shared__ bf16x8 s_p[4][64];
  __shared__ unsigned short s_t[WITH_O ? NW : 1][2][WITH_O ? BK * TS : 8];
  // cross-wave exchanges of per-row values reuse the P buffer (before the
  // sweep) and the partials buffer (after it)
  float* s_x = reinterpret_cast<float*>(&s_p[0][0]);              // [NW][64]
  double* s_xd = reinterpret_cast<double*>(&s_part[0][0][0][0]);   // [NW][2][64]

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, c = lane & 31;
  const int nbq = w & 1, kh = w >> 1;  // quarter this wave reduces: row block nbq, tile-row half kh
  const int rb = blockIdx.x / Sv, sv = blockIdx.x - rb * Sv;
  const int64_t q0 = (int64_t)rb * BQ;
  const int d0 = w * DS;
  // Stage write offsets (element) of lane (hh, c) for even / odd k-step:
  // row c, chunk 2ks + hh at position (2ks + hh) ^ s(c), s(c) = (c >> 1) & 3.
  int sw_base[2];
  {
    const int x = hh ^ ((c >> 1) & 3);
    sw_base[0] = c * TS + 8 * x;
    sw_base[1] = c * TS + 8 * (x ^ 2) - 16;
  }
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

  f32x16 o[2][WITH_O ? DB : 1];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < (WITH_O ? DB : 1); ++db) o[qb][db] = zero16();

  const int64_t my_row = q0 + 32 * nbq + c;  // row whose epilogue this lane runs (with 3 other lanes)
  // The epilogue works in base 2: z2 = z log2(e), p = 2^(z2 - m2).
  const float c2 = inv_tau * kLog2e;
  float m2 = -INFINITY;
  double s_acc = 0.0, sz_acc = 0.0;  // this lane's share of sum p, sum p z2
  bool flag = false;

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
  // fragment-major copy and masked in the epilogue); each k-slice of `a`, once its MFMAs are
  // issued, is staged for the transposing load (WITH_O) and reloaded with
  // the same slice of tile `t_next`.
  auto s_step = [&](bf16x8 (&a)[KS], f32x16 (&acc)[2], int buf, int t_next) {
    const auto r = frag_rsrc(frag_ptr<KB>(Wf, t_next, w, 0, 0), KS * 1024);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[nb] = mfma32(a[ks], q[nb][ks], ks == 0 ? zero16() : acc[nb]);
      if constexpr (WITH_O)
        *reinterpret_cast<bf16x8*>(&s_t[w][buf][sw_base[ks & 1] + 16 * ks]) = a[ks];
      a[ks] = ld_buf(r, lane * 16, ks * 1024);
      // keep the matrix, LDS and memory instructions of each k-step in this
      // order (vector ALU work may move across): left to itself the compiler
      // bunches the stage writes, and the waves then stall on the LDS queue
      // (2 % faster here; the same fence slows the weight-gradient sweep)
      __builtin_amdgcn_sched_barrier(0x002);
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
  // P KV of the staged tile in `buf` (A = P of row block qb, k-step ks from
  // the wave that reduced quarter (qb, ks); B = staged rows kvq(ks, hh, *),
  // columns 32db + c), with the reduce of the next tile's partials issued
  // near the end.
  auto pv_reduce = [&](int buf, f32x4 (&sf)[2]) {
    f32x4 r[NW];
    if constexpr (WITH_O) {
      bf16x8 pf[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) pf[qb][ks] = s_p[qb + 2 * ks][lane];
      const unsigned short* tb = &s_t[w][buf][0];
      constexpr int NF = 2 * DB;  // fragments (db, ks) in order
      auto frag = [&](int f) {
        const int db = f >> 1, ks = f & 1;
        return ld_tr(tb + tr_base[0] + 16 * ks * TS + 32 * db, tb + tr_base[1] + 16 * ks * TS + 32 * db);
      };
      bf16x8 b0 = frag(0), b1 = frag(1);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const bf16x8 b2 = frag(f + 2 < NF ? f + 2 : NF - 1);
        if (f == (NF > 6 ? NF - 6 : 0)) {
#pragma unroll
          for (int src = 0; src < NW; ++src) r[src] = s_part[src][nbq][2 * kh][lane];
        }
        if (f == (NF > 3 ? NF - 3 : 0)) {
          sf[0] = (r[0] + r[1]) + (r[2] + r[3]);
#pragma unroll
          for (int src = 0; src < NW; ++src) r[src] = s_part[src][nbq][2 * kh + 1][lane];
        }
        const int db = f >> 1, ks = f & 1;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) o[qb][db] = mfma32(pf[qb][ks], b0, o[qb][db]);
        b0 = b1;
        b1 = b2;
      }
    } else {
#pragma unroll
      for (int src = 0; src < NW; ++src) r[src] = s_part[src][nbq][2 * kh][lane];
      sf[0] = (r[0] + r[1]) + (r[2] + r[3]);
#pragma unroll
      for (int src = 0; src < NW; ++src) r[src] = s_part[src][nbq][2 * kh + 1][lane];
    }
    sf[1] = (r[0] + r[1]) + (r[2] + r[3]);
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
    s_step(a, acc, t_begin & 1, min(t_begin + 1, t_end - 1));
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
    bf16x8 pa;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      flag |= z[j] > m2 + kRefSlack2;
      const float pj = __builtin_amdgcn_exp2f(fminf(z[j] - m2, kRefSlack2));
      sp += pj;
      szp = fmaf(pj, z[j], szp);
      pa[j] = (__bf16)pj;
    }
    s_acc += (double)sp;
    sz_acc += (double)szp;
    // ---- logits of tile t+1 on the matrix cores, stage t+1, load t+2 -------
    s_step(a, acc, (t + 1) & 1, tnn);
    __builtin_amdgcn_sched_barrier(0);
    exec_barrier();
    if constexpr (WITH_O) s_p[w][lane] = pa;
    write_part(acc);
    __syncthreads();
    // ---- accumulator product of tile t, reduce of tile t+1 -----------------
    pv_reduce(t & 1, sf);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) bv[hf] = bvn[hf];
  }

  // ---- results: combine the four holders of each row ----------------------
  double sx = s_acc + (double)__shfl_xor(s_acc, 32, 64);
  double szx = sz_acc + (double)__shfl_xor(sz_acc, 32, 64);
  int fl = flag ? 1 : 0;
  fl |= __shfl_xor(fl, 32, 64);
  __syncthreads();
  if (hh == 0) {
    s_xd[(2 * w) * 64 + c] = sx;
    s_xd[(2 * w + 1) * 64 + c] = szx;
    s_x[w * 64 + c] = __int_as_float(fl);
  }
  __syncthreads();
  if (kh == 0 && hh == 0 && my_row < N) {
    RowStats rs;
    rs.m = (float)((double)m2 * kLn2);
    rs.zy = 0.f;
    rs.s = sx + s_xd[(2 * (w ^ 2)) * 64 + c];
    rs.sz = (szx + s_xd[(2 * (w ^ 2) + 1) * 64 + c]) * kLn2;
    rs.flag = (fl | __float_as_int(s_x[(w ^ 2) * 64 + c])) ? 1 : 0;
    rs.pad = 0;
    stats[(int64_t)sv * N + my_row] = rs;
  }
  if constexpr (WITH_O) {
    float* Ob = O + (int64_t)sv * N * H;
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

// ---------------------------------------------------------------------------
// Weight-gradient sweep: per vocabulary row v, over compacted tokens t,
//   dz[t,v] = gs_t ([v = y_t] - exp(z[t,v] - lse_t)),  gs_t = g_t / tau
//   grad_W[v] += sum_t dz[t,v] h_t,   grad_b[v] += sum_t dz[t,v]
// acc_mode: 0 write the output dtype; 1 store fp32 accumulator; 2 add into it;
// 3 add the fp32 accumulator and write the output dtype.
// ---------------------------------------------------------------------------
template <int KB, bool HAS_BIAS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_mfma_kernel(const __bf16* __restrict__ Wf, const __bf16* __restrict__ bias,
                     const __bf16* __restrict__ hcf, const TokData* __restrict__ tok,
                     const int* __restrict__ count_dev, int V, float inv_tau, int acc_mode,
                     float* __restrict__ gW_acc, float* __restrict__ gb_acc, __bf16* __restrict__ gW_out,
                     __bf16* __restrict__ gb_out, int whole, int parts, float* __restrict__ part_w,
                     float* __restrict__ part_b) {
  constexpr int H = 128 * KB;
  constexpr int DS = Stage<KB>::DS;
  constexpr int TS = Stage<KB>::TS;
  constexpr int KS = DS / 16;
  constexpr int DB = DS / 32;
  __shared__ f32x4 s_part[NW][2][4][64];
  __shared__ bf16x8 s_p[4][64];
  __shared__ TokData s_tok[2][BK];
  __shared__ unsigned short s_t[NW][2][BK * TS];
  double* s_xd = reinterpret_cast<double*>(&s_part[0][0][0][0]);  // [NW][64], after the sweep

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, c = lane & 31;
  const int nbq = w & 1, kh = w >> 1;
  const int n_tok = *count_dev;
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
  // Stage write offsets (element) of lane (hh, c) for even / odd k-step:
  // row c, chunk 2ks + hh at position (2ks + hh) ^ s(c), s(c) = (c >> 1) & 3.
  int sw_base[2];
  {
    const int x = hh ^ ((c >> 1) & 3);
    sw_base[0] = c * TS + 8 * x;
    sw_base[1] = c * TS + 8 * (x ^ 2) - 16;
  }
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

  // Per-token data of tile t, loaded into registers one phase before it is
  // written to LDS (wave 0, lanes < 32), so the load latency stays hidden.
  // Held as a plain vector: a TokData variable was placed in LDS by the
  // compiler, whose store right after the load then waited for every
  // outstanding load of the wave, the token tiles included.
  const bool any = t_hi > t_lo;
  static_assert(sizeof(TokData) == 16, "one 16-byte record per token");
  const auto tok_r = __builtin_amdgcn_make_buffer_rsrc(const_cast<TokData*>(tok), 0, 0x7ffffff0, 0x00020000);
  u32x4 tk = {0u, 0u, 0u, 0u};
  auto load_tok = [&](int t) {
    if (w == 0 && lane < BK) tk = __builtin_amdgcn_raw_buffer_load_b128(tok_r, (t * BK + lane) * 16, 0, 0);
  };
  auto stage_tok = [&](int t) {
    if (w == 0 && lane < BK) *reinterpret_cast<u32x4*>(&s_tok[t & 1][lane]) = tk;
  };
  if (any) load_tok(t_lo);
  // Resident W fragments (B operand of S^T), rows q0 + 32nb + c, cols
  // d0 + 16ks + 8hh, from the fragment-major copy (rows past V are zero),
  // and the first token tile, in k-step order so that the first MFMAs wait
  // only for their own operands.
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
  f32x16 o[2][DB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = zero16();

  const int my_v = q0 + 32 * nbq + c;
  const float bvl = HAS_BIAS ? (float)bias[min(my_v, V - 1)] : 0.f;
  double gb_run = 0.0;

  auto s_step = [&](bf16x8 (&a)[KS], f32x16 (&acc)[2], int buf, int t_next) {
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
  auto pv_reduce = [&](int buf, f32x4 (&sf)[2]) {
    f32x4 r[NW];
    bf16x8 pf[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) pf[qb][ks] = s_p[qb + 2 * ks][lane];
    const unsigned short* tb = &s_t[w][buf][0];
    constexpr int NF = 2 * DB;
    auto frag = [&](int f) {
      const int db = f >> 1, ks = f & 1;
      return ld_tr(tb + tr_base[0] + 16 * ks * TS + 32 * db, tb + tr_base[1] + 16 * ks * TS + 32 * db);
    };
    bf16x8 b0 = frag(0), b1 = frag(1);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const bf16x8 b2 = frag(f + 2 < NF ? f + 2 : NF - 1);
      if (f == (NF > 6 ? NF - 6 : 0)) {
#pragma unroll
        for (int src = 0; src < NW; ++src) r[src] = s_part[src][nbq][2 * kh][lane];
      }
      if (f == (NF > 3 ? NF - 3 : 0)) {
        sf[0] = (r[0] + r[1]) + (r[2] + r[3]);
#pragma unroll
        for (int src = 0; src < NW; ++src) r[src] = s_part[src][nbq][2 * kh + 1][lane];
      }
      const int db = f >> 1, ks = f & 1;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) o[qb][db] = mfma32(pf[qb][ks], b0, o[qb][db]);
      b0 = b1;
      b1 = b2;
    }
    sf[1] = (r[0] + r[1]) + (r[2] + r[3]);
  };

  f32x16 acc[2];
  f32x4 sf[2];
  if (any) {
    stage_tok(t_lo);
    load_tok(min(t_lo + 1, t_hi - 1));
    s_step(a, acc, t_lo & 1, min(t_lo + 1, t_hi - 1));
    write_part(acc);
  }
  __syncthreads();
  if (t_hi > t_lo) reduce_part(sf);

  for (int t = t_lo; t < t_hi; ++t) {
    const int t0 = t * BK;
    const int tn = min(t + 1, t_hi - 1);
    const int tnn = min(t + 2, t_hi - 1);
    // ---- epilogue of tile t (vector ALU; the scheduler interleaves it with
    //      the logit MFMAs of tile t+1 below) -------------------------------
    bf16x8 pa;
    float gsum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kv = kvq(kh, hh, j);
      const TokData td = s_tok[t & 1][kv];
      const float sv_ = sf[j >> 2][j & 3];
      const float z = (sv_ + bvl) * inv_tau;
      const float pr = __expf(z - td.lse);
      float dz = td.gs * ((td.y == my_v ? 1.f : 0.f) - pr);
      dz = (t0 + kv < n_tok && my_v < V) ? dz : 0.f;
      gsum += dz;
      pa[j] = (__bf16)dz;
    }
    gb_run += (double)gsum;
    // ---- logits of tile t+1, stage t+1, load t+2 ---------------------------
    s_step(a, acc, (t + 1) & 1, tnn);
    __builtin_amdgcn_sched_barrier(0);
    exec_barrier();
    s_p[w][lane] = pa;
    write_part(acc);
    stage_tok(tn);
    __syncthreads();
    load_tok(tnn);
    pv_reduce(t & 1, sf);
  }

  // grad_b: the four holders of a vocabulary row (two lane halves of two
  // waves) hold disjoint token subsets
  double gbv = gb_run + __shfl_xor(gb_run, 32, 64);
  __syncthreads();
  if (hh == 0) s_xd[w * 64 + c] = gbv;
  __syncthreads();
  if (slot >= 0) {  // a share of a tail block: fp32 partial sums, combined by tail_reduce_kernel
    if (kh == 0 && hh == 0) part_b[slot * BQ + 32 * nbq + c] = (float)(gbv + s_xd[(w ^ 2) * 64 + c]);
    float* pw = part_w + (int64_t)slot * BQ * H;
    store_acc<4, DS, DB>(o, reinterpret_cast<float*>(&s_t[w][0][0]), hh, c, lane,
                         [&](int qb, int r, int col, const f32x4 (&v)[1]) {
                           *reinterpret_cast<f32x4*>(pw + (int64_t)(32 * qb + r) * H + d0 + col) = v[0];
                         });
    return;  // uniform
  }
  const bool from_acc = acc_mode == 2 || acc_mode == 3;
  const bool to_acc = acc_mode == 1 || acc_mode == 2;
  if (kh == 0 && hh == 0 && my_v < V && (to_acc ? gb_acc != nullptr : gb_out != nullptr)) {
    double val = gbv + s_xd[(w ^ 2) * 64 + c];
    if (from_acc) val += (double)gb_acc[my_v];
    if (to_acc) gb_acc[my_v] = (float)val;
    else gb_out[my_v] = (__bf16)(float)val;
  }
  if (to_acc ? gW_acc == nullptr : gW_out == nullptr) return;  // uniform: every wave returns
  float* sbuf = reinterpret_cast<float*>(&s_t[w][0][0]);
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
      // written once and read by nobody in this call: non-temporal, so that
      // the token tiles stay in L2
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, u), reinterpret_cast<u32x4*>(gW_out + k));
    });
  }
}

template <int KB>
hipError_t fwd_dispatch(const __bf16* h, const __bf16* Wf, const __bf16* b, int64_t N, int V, float inv_tau, int Sv,
                        int tps, bool with_o, RowStats* stats, float* O, hipStream_t st) {
  const int64_t nrb = (N + BQ - 1) / BQ;
  dim3 grid((unsigned)(nrb * Sv)), block(256);
  if (with_o && b)
    hipLaunchKernelGGL((fwd_mfma_kernel<KB, true, true>), grid, block, 0, st, h, Wf, b, N, V, inv_tau, Sv, tps, stats,
                       O);
  else if (with_o)
    hipLaunchKernelGGL((fwd_mfma_kernel<KB, true, false>), grid, block, 0, st, h, Wf, b, N, V, inv_tau, Sv, tps, stats,
                       O);
  else if (b)
    hipLaunchKernelGGL((fwd_mfma_kernel<KB, false, true>), grid, block, 0, st, h, Wf, b, N, V, inv_tau, Sv, tps, stats,
                       O);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<KB, false, false>), grid, block, 0, st, h, Wf, b, N, V, inv_tau, Sv, tps,
                       stats, O);
  return hipGetLastError();
}

constexpr int kTailParts = 4;     // workgroups sharing one tail block of the weight-gradient sweep
constexpr int kMaxTailWGs = 256;  // bound of the partial-sum scratch (workgroups)

// Workgroups of 256 threads of `kernel` the device holds at once (compute
// units x workgroups per unit), computed once per device and kernel.
template <typename K>
hipError_t resident_workgroups(K kernel, int* out) {
  constexpr int kMaxDevices = 64;
  static int cache[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && cache[dev] > 0) {
    *out = cache[dev];
    return hipSuccess;
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0);
  if (e != hipSuccess) return e;
  const int n = cus * (per_cu > 0 ? per_cu : 1);
  if (dev >= 0 && dev < kMaxDevices) cache[dev] = n;
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
                        int V, float inv_tau, int acc_mode, float* gW_acc, float* gb_acc, __bf16* gW_out,
                        __bf16* gb_out, float* tail_scratch, hipStream_t st) {
  // Blocks of the last, partial round of workgroups are split over the token
  // tiles so that round ends sooner: `parts` workgroups per block, as many as
  // fit the free slots (at most kTailParts, and kMaxTailWGs in all).
  const int nblk = (V + BQ - 1) / BQ;
  int resident = 0;
  hipError_t e = b ? resident_workgroups(bwd_mfma_kernel<KB, true>, &resident)
                   : resident_workgroups(bwd_mfma_kernel<KB, false>, &resident);
  if (e != hipSuccess) return e;
  const int rem = resident > 0 ? nblk % resident : 0;
  int parts = rem > 0 ? min(kTailParts, min(resident, kMaxTailWGs) / rem) : 1;
  if (tail_scratch == nullptr || parts < 2) parts = 1;
  const int whole = parts > 1 ? nblk - rem : nblk;
  const int tail_wgs = parts > 1 ? rem * parts : 0;
  float* part_w = tail_scratch;
  float* part_b = tail_scratch ? tail_scratch + (size_t)kMaxTailWGs * BQ * (128 * KB) : nullptr;
  dim3 grid((unsigned)(whole + tail_wgs)), block(256);
  if (b)
    hipLaunchKernelGGL((bwd_mfma_kernel<KB, true>), grid, block, 0, st, Wf, b, hcf, tok, count_dev, V, inv_tau,
                       acc_mode, gW_acc, gb_acc, gW_out, gb_out, whole, parts, part_w, part_b);
  else
    hipLaunchKernelGGL((bwd_mfma_kernel<KB, false>), grid, block, 0, st, Wf, b, hcf, tok, count_dev, V, inv_tau,
                       acc_mode, gW_acc, gb_acc, gW_out, gb_out, whole, parts, part_w, part_b);
  e = hipGetLastError();
  if (e != hipSuccess || tail_wgs == 0) return e;
  hipLaunchKernelGGL(tail_reduce_kernel, dim3((unsigned)(rem * BQ)), dim3(256), 0, st, part_w, part_b, whole, parts,
                     128 * KB, V, acc_mode, gW_acc, gb_acc, gW_out, gb_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_frag_copy(const __bf16* X, const int* idx, const int* count_dev, int64_t rows, int64_t tiles, int H,
                            __bf16* Xf, hipStream_t st) {
  if (tiles <= 0) return hipSuccess;
  const int64_t total = tiles * BK * (H / 8) / 2;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(frag_copy_kernel, dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(256), 0, st, X, idx,
                     count_dev, rows, H, tiles, Xf);
  return hipGetLastError();
}

hipError_t launch_fwd_mfma(const __bf16* h, const __bf16* Wf, const __bf16* b, int64_t N, int H, int V, float inv_tau,
                           int Sv, bool with_o, RowStats* stats, float* O, hipStream_t st) {
  const int n_tiles = (V + BK - 1) / BK;
  const int tps = (n_tiles + Sv - 1) / Sv;
  switch (H / 128) {
    case 1: return fwd_dispatch<1>(h, Wf, b, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    case 2: return fwd_dispatch<2>(h, Wf, b, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    case 3: return fwd_dispatch<3>(h, Wf, b, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    case 4: return fwd_dispatch<4>(h, Wf, b, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    case 5: return fwd_dispatch<5>(h, Wf, b, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    case 6: return fwd_dispatch<6>(h, Wf, b, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    case 7: return fwd_dispatch<7>(h, Wf, b, N, V, inv_tau, Sv, tps, with_o, stats, O, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_mfma(const __bf16* Wf, const __bf16* b, const __bf16* hcf, const TokData* tok,
                           const int* count_dev, int H, int V, float inv_tau, int acc_mode, float* gW_acc,
                           float* gb_acc, __bf16* gW_out, __bf16* gb_out, float* tail_scratch, hipStream_t st) {
  switch (H / 128) {
    case 1: return bwd_dispatch<1>(Wf, b, hcf, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    case 2: return bwd_dispatch<2>(Wf, b, hcf, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    case 3: return bwd_dispatch<3>(Wf, b, hcf, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    case 4: return bwd_dispatch<4>(Wf, b, hcf, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    case 5: return bwd_dispatch<5>(Wf, b, hcf, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    case 6: return bwd_dispatch<6>(Wf, b, hcf, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    case 7: return bwd_dispatch<7>(Wf, b, hcf, tok, count_dev, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out, gb_out,
                                   tail_scratch, st);
    default: return hipErrorInvalidValue;
  }
}

size_t bwd_tail_scratch_floats(int H) { return (size_t)kMaxTailWGs * BQ * H + (size_t)kMaxTailWGs * BQ; }

}  // namespace plp
