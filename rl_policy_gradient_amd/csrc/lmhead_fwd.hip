// Forward sweep: the launcher; the statistics-only passes (no grad_h
// accumulator) use the single-role kernel, compiled here.
#include "fwd_sweep.h"

namespace plp {

hipError_t launch_fwd_mfma(const __bf16* h, const __bf16* Wf, const float* b32, const __bf16* b16, int64_t N, int H,
                           int V, float inv_tau, int Sv, bool with_o, RowStats* stats, float* O, hipStream_t st,
                           const int* count_dev, const float* mref, int mref_stride, const int* row_idx,
                           int* clear_count) {
  if ((b32 == nullptr) != (b16 == nullptr)) return hipErrorInvalidValue;  // both copies of the bias, or neither
  if (with_o)
    return launch_fwd_mfma_o(h, Wf, b32, N, H, V, inv_tau, Sv, stats, O, count_dev, mref, mref_stride, row_idx,
                             clear_count, st);
  if (count_dev || mref || row_idx) return hipErrorInvalidValue;  // the compacted passes are accumulator passes
  if (b16) return fwd_stats_launch<true>(h, Wf, b16, N, H, V, inv_tau, Sv, stats, clear_count, st);
  return fwd_stats_launch<false>(h, Wf, b16, N, H, V, inv_tau, Sv, stats, clear_count, st);
}

}  // namespace plp
