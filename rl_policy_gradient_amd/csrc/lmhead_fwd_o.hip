// Forward sweep with the grad_h accumulator: the two-role kernel, with and
// without a bias.
#include "fwd_sweep.h"

namespace plp {

hipError_t launch_fwd_mfma_o(const __bf16* h, const __bf16* Wf, const float* b, int64_t N, int H, int V, float inv_tau,
                             int Sv, RowStats* stats, float* O, const int* count_dev, const float* mref,
                             int mref_stride, const int* row_idx, int* clear_count, hipStream_t st) {
  if (b)
    return fwd_pp_launch<true>(h, Wf, b, N, H, V, inv_tau, Sv, stats, O, count_dev, mref, mref_stride, row_idx,
                               clear_count, st);
  return fwd_pp_launch<false>(h, Wf, b, N, H, V, inv_tau, Sv, stats, O, count_dev, mref, mref_stride, row_idx,
                              clear_count, st);
}

}  // namespace plp
