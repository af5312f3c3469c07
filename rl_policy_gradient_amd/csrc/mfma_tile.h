// Tile machinery shared by the MFMA sweeps of the LM head (gfx950).
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
#pragma once

#include "common.h"

#include <math.h>

namespace plp {

// Internal to the sweeps' translation units.
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
// fp32 data through a buffer resource (byte range `bytes`), 16 bytes per lane.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t f32_rsrc(const float* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 ld_f4(__amdgpu_buffer_rsrc_t r, int lane_bytes) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, lane_bytes, 0, 0));
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

}  // namespace
}  // namespace plp
