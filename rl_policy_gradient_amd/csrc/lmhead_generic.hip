// Generic (vector ALU) sweeps of the LM head for fp32 inputs and for hidden
// sizes the MFMA sweeps do not cover (H not a multiple of 128, or above 896).
// One workgroup per token row (forward) or per vocabulary row (weight
// gradient); fp32 arithmetic, fp64 running sums. Slow, exact in structure,
// used for small shapes.
#include "common.h"
#include "generic_row.h"

#include <math.h>

namespace plp {

namespace {

constexpr int NT = 256;
constexpr int kMaxGenericH = 4096;

template <typename T>
__device__ __forceinline__ float ldf(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ldf<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ldf<__bf16>(const __bf16* p, int64_t i) { return (float)p[i]; }

template <typename T>
__device__ __forceinline__ void stf(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void stf<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void stf<__bf16>(__bf16* p, int64_t i, float v) { p[i] = (__bf16)v; }

__device__ double block_sum_d(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// Forward: one block per row, exact online max (row_exact).
template <typename T, bool WITH_O>
__global__ __launch_bounds__(NT) void fwd_generic_kernel(const T* __restrict__ h, const T* __restrict__ W,
                                                         const T* __restrict__ bias,
                                                         const int64_t* __restrict__ y, int64_t N, int H,
                                                         int V, float inv_tau, RowStats* __restrict__ stats,
                                                         float* __restrict__ O) {
  extern __shared__ float sm[];
  const int64_t row = blockIdx.x;
  const int64_t yv = y ? y[row] : -1;
  const RowResult r = row_exact<T>(h + row * H, W, bias, yv, H, V, inv_tau, WITH_O, sm);
  if (threadIdx.x == 0) {
    RowStats rs;
    rs.m = r.m;
    rs.zmax = r.m;  // the exact online maximum
    rs.s = r.s;
    rs.sz = r.sz;
    rs.flag = 0;
    stats[row] = rs;
  }
  if constexpr (WITH_O) {
    const float* os = sm + H;
    for (int d = threadIdx.x; d < H; d += NT) O[row * H + d] = os[d];
  }
}

// Weight gradient: one block per vocabulary row over the compacted tokens.
template <typename T>
__global__ __launch_bounds__(NT) void bwd_generic_kernel(const T* __restrict__ W, const T* __restrict__ bias,
                                                         const T* __restrict__ hc,
                                                         const TokData* __restrict__ tok,
                                                         const int* __restrict__ count_dev, int H, int V,
                                                         float inv_tau, int acc_mode, float* __restrict__ gW_acc,
                                                         float* __restrict__ gb_acc, T* __restrict__ gW_out,
                                                         T* __restrict__ gb_out) {
  extern __shared__ float sm[];
  float* ws = sm;            // [H]
  float* gs = ws + H;        // [H]
  float* dzc = gs + H;       // [NT]
  double* redd = reinterpret_cast<double*>(dzc + NT);
  const int v = blockIdx.x;
  const int tid = threadIdx.x;
  for (int d = tid; d < H; d += NT) {
    ws[d] = ldf<T>(W, (int64_t)v * H + d);
    gs[d] = 0.f;
  }
  __syncthreads();
  const float bv = bias ? ldf<T>(bias, v) : 0.f;
  const int n_tok = *count_dev;
  double gb = 0.0;
  for (int t0 = 0; t0 < n_tok; t0 += NT) {
    const int t = t0 + tid;
    float dz = 0.f;
    if (t < n_tok) {
      float acc = 0.f;
      const T* hr = hc + (int64_t)t * H;
      for (int d = 0; d < H; ++d) acc = fmaf(ws[d], ldf<T>(hr, d), acc);
      const float z = (acc + bv) * inv_tau;
      const TokData td = tok[t];
      dz = td.gs * ((td.y == v ? 1.f : 0.f) - expf(z - td.lse));
    }
    dzc[tid] = dz;
    gb += block_sum_d((double)dz, redd);
    const int nt = min(NT, n_tok - t0);
    for (int d = tid; d < H; d += NT) {
      float a = gs[d];
      for (int k = 0; k < nt; ++k) a = fmaf(dzc[k], ldf<T>(hc, (int64_t)(t0 + k) * H + d), a);
      gs[d] = a;
    }
    __syncthreads();
  }
  const bool from_acc = acc_mode == 2 || acc_mode == 3;
  const bool to_acc = acc_mode == 1 || acc_mode == 2;
  if (to_acc ? gW_acc != nullptr : gW_out != nullptr) {
    for (int d = tid; d < H; d += NT) {
      float val = gs[d];
      const int64_t k = (int64_t)v * H + d;
      if (from_acc) val += gW_acc[k];
      if (to_acc) gW_acc[k] = val;
      else stf<T>(gW_out, k, val);
    }
  }
  if (tid == 0 && (to_acc ? gb_acc != nullptr : gb_out != nullptr)) {
    double val = gb;
    if (from_acc) val += (double)gb_acc[v];
    if (to_acc) gb_acc[v] = (float)val;
    else stf<T>(gb_out, v, (float)val);
  }
}

template <typename T>
hipError_t fwd_t(const void* h, const void* W, const void* b, const int64_t* y, int64_t N, int H, int V,
                 float inv_tau, bool with_o, RowStats* stats, float* O, hipStream_t st) {
  const size_t lds = row_exact_smem_bytes(H);
  if (with_o)
    hipLaunchKernelGGL((fwd_generic_kernel<T, true>), dim3((unsigned)N), dim3(NT), lds, st, (const T*)h,
                       (const T*)W, (const T*)b, y, N, H, V, inv_tau, stats, O);
  else
    hipLaunchKernelGGL((fwd_generic_kernel<T, false>), dim3((unsigned)N), dim3(NT), lds, st, (const T*)h,
                       (const T*)W, (const T*)b, y, N, H, V, inv_tau, stats, O);
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_t(const void* W, const void* b, const void* hc, const TokData* tok, const int* count_dev, int H,
                 int V, float inv_tau, int acc_mode, float* gW_acc, float* gb_acc, void* gW_out, void* gb_out,
                 hipStream_t st) {
  const size_t lds = (size_t)(2 * H + NT) * sizeof(float) + NT * sizeof(double) + 16;
  hipLaunchKernelGGL((bwd_generic_kernel<T>), dim3((unsigned)V), dim3(NT), lds, st, (const T*)W, (const T*)b,
                     (const T*)hc, tok, count_dev, H, V, inv_tau, acc_mode, gW_acc, gb_acc, (T*)gW_out,
                     (T*)gb_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_generic(int dtype, const void* h, const void* W, const void* b, const int64_t* y, int64_t N,
                              int H, int V, float inv_tau, bool with_o, RowStats* stats, float* O, hipStream_t st) {
  if (H > kMaxGenericH || N <= 0) return N <= 0 ? hipSuccess : hipErrorInvalidValue;
  return dtype == 0 ? fwd_t<float>(h, W, b, y, N, H, V, inv_tau, with_o, stats, O, st)
                    : fwd_t<__bf16>(h, W, b, y, N, H, V, inv_tau, with_o, stats, O, st);
}

hipError_t launch_bwd_generic(int dtype, const void* W, const void* b, const void* hc, const TokData* tok,
                              const int* count_dev, int H, int V, float inv_tau, int acc_mode, float* gW_acc,
                              float* gb_acc, void* gW_out, void* gb_out, hipStream_t st) {
  if (H > kMaxGenericH) return hipErrorInvalidValue;
  return dtype == 0 ? bwd_t<float>(W, b, hc, tok, count_dev, H, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out,
                                   gb_out, st)
                    : bwd_t<__bf16>(W, b, hc, tok, count_dev, H, V, inv_tau, acc_mode, gW_acc, gb_acc, gW_out,
                                    gb_out, st);
}

}  // namespace plp
