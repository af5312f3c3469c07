// One token row over the whole vocabulary with an exact online max, on the
// vector ALU (one 256-thread block per row). Used by the generic forward
// sweep and by the merge kernel's recompute of flagged rows.
//
// Recurrence (Liger PR #1558, _selective_entropy_forward): running
// (m, s = sum e^{z-m}, sz = sum e^{z-m} z), both sums rescaled by e^{m_old-m}
// whenever the max moves; optionally O = sum_v e^{z-m} W_v rescaled alike.
#pragma once

#include "common.h"

#include <math.h>

namespace plp {

constexpr int kRowNT = 256;

template <typename T>
__device__ __forceinline__ float ld_as_f(const T* p, int64_t i) {
  return (float)p[i];
}

__device__ inline float row_block_max(float v, float* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int s = kRowNT / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__device__ inline double row_block_sum(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int s = kRowNT / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

struct RowResult {
  float m;
  float zy;
  double s;
  double sz;
};

// Shared-memory floats needed by row_exact (doubles counted as two floats).
__host__ __device__ inline size_t row_exact_smem_bytes(int H) {
  return (size_t)(2 * H + 2 * kRowNT) * sizeof(float) + kRowNT * sizeof(double) + 16;
}

// All kRowNT threads call it; every thread gets the same result. With with_o,
// os[0..H) holds O relative to the returned m on exit.
template <typename T>
__device__ RowResult row_exact(const T* __restrict__ hrow, const T* __restrict__ W, const T* __restrict__ bias,
                               int64_t yv, int H, int V, float inv_tau, bool with_o, float* smem) {
  float* hs = smem;            // [H]
  float* os = hs + H;          // [H]
  float* pc = os + H;          // [kRowNT]
  float* redf = pc + kRowNT;   // [kRowNT]
  double* redd = reinterpret_cast<double*>(redf + kRowNT);
  __shared__ float zy_sh;
  const int tid = threadIdx.x;
  for (int d = tid; d < H; d += kRowNT) {
    hs[d] = ld_as_f<T>(hrow, d);
    os[d] = 0.f;
  }
  if (tid == 0) zy_sh = 0.f;
  __syncthreads();
  float m_run = -INFINITY;
  double s_run = 0.0, sz_run = 0.0;
  for (int v0 = 0; v0 < V; v0 += kRowNT) {
    const int v = v0 + tid;
    float z = -INFINITY;
    if (v < V) {
      float acc = 0.f;
      const T* wr = W + (int64_t)v * H;
      for (int d = 0; d < H; ++d) acc = fmaf(hs[d], ld_as_f<T>(wr, d), acc);
      z = (acc + (bias ? ld_as_f<T>(bias, v) : 0.f)) * inv_tau;
      if ((int64_t)v == yv) zy_sh = z;
    }
    const float mx = row_block_max(z, redf);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = expf(m_run - m_new);
    const float p = v < V ? expf(z - m_new) : 0.f;
    const double sp = row_block_sum((double)p, redd);
    const double szp = row_block_sum(v < V ? (double)p * (double)z : 0.0, redd);
    s_run = s_run * (double)alpha + sp;
    sz_run = sz_run * (double)alpha + szp;
    m_run = m_new;
    if (with_o) {
      pc[tid] = p;
      __syncthreads();
      const int nv = min(kRowNT, V - v0);
      for (int d = tid; d < H; d += kRowNT) {
        float a = os[d] * alpha;
        for (int k = 0; k < nv; ++k) a = fmaf(pc[k], ld_as_f<T>(W, (int64_t)(v0 + k) * H + d), a);
        os[d] = a;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  RowResult r;
  r.m = m_run;
  r.zy = zy_sh;
  r.s = s_run;
  r.sz = sz_run;
  __syncthreads();
  return r;
}

}  // namespace plp
